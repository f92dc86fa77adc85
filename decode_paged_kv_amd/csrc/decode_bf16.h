// bf16 paged GQA decode attention for one workgroup, shared by the decode
// kernel and the mixed-batch kernel.  The split plans are described at the
// top of attn_decode.hip.
#pragma once

#include "pkv_internal.h"

namespace pkv {
namespace decode_impl {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

// ------------------------------------------------------------------------
// bf16 kernel.  Same work decomposition (one workgroup of 4 waves per
// (split, KV head, request)); each wave walks 32-key tiles (tile i of the
// split to wave i % 4).  A tile is two 16-key halves, each inside one block,
// so a half's block id is wave-uniform: it is read with a scalar load and
// the half's (block, head) K and V tiles are addressed through buffer
// descriptors in scalar registers; a lane adds only a fixed offset.  Every
// K/V byte is read once.  The V loads carry the non-temporal hint (each
// instruction reads whole lines).  The K loads do not: one instruction
// reads 64 bytes of each of 16 rows, the other half of every 128-byte line
// comes with the next instruction, and without the hint the two halves meet
// in the L1 (on a CU-masked half of the device this is worth about a fifth
// of the decode bandwidth).
//
// The GQA group's contraction runs on the matrix cores, in transposed form
// so the G <= 16 q-heads are the 16 columns of 16x16 MFMA tiles:
//   S^T = K Q^T    v_mfma_f32_16x16x32_bf16 per (half, 32 head dims):
//                  A = 16 K rows (lane l: key l%16, dims 8(l/16)..+7 of the
//                  chunk, one 16-byte load), B = q (lane l: head l%16).
//   softmax        lane l holds keys 4(l/16)..+3 of each half for head
//                  l%16; the per-head max over the tile needs two lane swaps
//                  (v_permlane16_swap, v_permlane32_swap); exp2 domain; the
//                  running max moves only by more than a slack, so the
//                  accumulators are rescaled rarely.
//   O^T += V^T P^T v_mfma_f32_16x16x16_bf16 per (half, 16 head dims): the
//                  S^T accumulator layout is already P's operand layout (4
//                  keys per lane), and A = the dim-major V tile (lane l: dim
//                  l%16, keys 4(l/16)..+3: 8 bytes; one instruction reads 16
//                  whole 32-byte dim rows, 512 contiguous bytes).
// Nothing goes through LDS until the final 4-wave merge.  The operand
// registers of a wave's tile are refilled with its next tile as soon as
// they are consumed: K right after S^T, V right after P V.  At head dim
// 128 the kernel holds about 250 registers per lane, two waves per SIMD,
// each with two 16 KB tiles in flight.
// In the stream split a workgroup's range can span several (request, KV
// head) segments; each wave issues the next segment's q, block ids and first
// tile loads as soon as it is done with the current segment's tiles, before
// the 4-wave merge of the current segment, so the merge and the next
// segment's first load latency overlap (about 1% on uneven contexts).
// A request whose context fits one split writes its output directly;
// otherwise each split writes its partial (m, l, acc) and the merge kernel
// combines them (a device-wide handoff inside the kernel would need L2
// write-back and invalidation on this multi-XCD part, costlier than a
// second launch).
// ------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_qk(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_pv(const uint2& a, const uint2& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b), c,
                                                   0, 0, 0);
}
// reduce over the four lanes l, l^16, l^32, l^48 (one MFMA column)
__device__ __forceinline__ float col_max(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float col_sum(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// One 32-key tile's MFMA operands and its two block ids (-1: absent).
template <int D>
struct DecodeTile {
  uint4 k[2][D / 32];       // A of S^T: key 16h + l%16, dims 32c + 8(l/16) .. +7
  uint2 v[2][D / 16];       // A of O^T: dim 16m + l%16, keys 16h + 4(l/16) .. +3
  int blk[2];
};

template <int D, int G>
struct DecodeBf16Smem {
  float acc[kWaves][G][D];
  float m[kWaves][G];
  float l[kWaves][G];
  float snew[G];            // score of the appended key, per q-head (log2 units)
};

// Running max update rule (log2 units): the max used for exp2 moves only
// when a tile's max exceeds it by more than this, so p <= 2^8.
constexpr float kDecodeSlack = 8.0f;

// Stream split bookkeeping.  Request b holds Hkv * ceil(L_b / 32) pair-tiles
// (L_b clamped to max_context_len), laid out by request, then KV
// head, then key.  scan_tiles returns the total, the request holding pair-
// tile `target` (-1: none) with the index of its first pair-tile, and the
// index of request rb's first pair-tile; every lane of the wave gets the
// same values (a wave-wide prefix sum, 64 requests per pass).
struct TileScan {
  long long total;
  int b;
  long long base;
  long long base_rb;
  bool over;                                    // some context exceeds the cap
};
__device__ __forceinline__ long long uniform64(long long x) {
  const int lo = __builtin_amdgcn_readfirstlane((int)(unsigned)(unsigned long long)x);
  const int hi = __builtin_amdgcn_readfirstlane((int)(unsigned)((unsigned long long)x >> 32));
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ TileScan scan_tiles(const int32_t* __restrict__ ctx, int batch, int cap, int hkv, long long target, int rb) {
  const int lane = threadIdx.x & 63;
  long long run = 0, base = 0, base_rb = 0;
  int fb = -1;
  bool over = false;
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int bb = b0 + lane;
    const int L = bb < batch ? ctx[bb] : 0;
    over |= L > cap;
    const long long x = (long long)hkv * ((max(min(L, cap), 0) + 31) >> 5);
    long long inc = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const long long y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
    }
    const long long excl = run + inc - x;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(bb < batch && excl <= target && target < excl + x);
    if (fb < 0 && hit) {
      const int l = __builtin_ctzll(hit);
      fb = b0 + l;
      base = __shfl(excl, l);
    }
    if (rb >= b0 && rb < b0 + 64) base_rb = __shfl(excl, rb - b0);
    run += __shfl(inc, 63);
  }
  TileScan r;
  r.total = uniform64(run);
  r.b = __builtin_amdgcn_readfirstlane(fb);
  r.base = uniform64(base);
  r.base_rb = uniform64(base_rb);
  r.over = __builtin_amdgcn_ballot_w64(over) != 0;
  return r;
}
// the workgroup whose pair-tile range holds pair-tile x (NW workgroups, W tiles)
__device__ __forceinline__ long long stream_owner(long long x, long long NW, long long W) {
  return ((x + 1) * NW + W - 1) / W - 1;
}

// One workgroup's work.  Equal splits (STREAM false): block (bx, by, bz) =
// (split, KV head, request).  Stream split: block bx of nbx.
template <int D, int G, bool STREAM, bool APPEND = false>
__device__ __forceinline__ void decode_bf16_block(PoolDev pool, const bf16_t* __restrict__ q,
                                                  bf16_t* __restrict__ out, const int32_t* __restrict__ bt,
                                                  int bt_stride, const int32_t* __restrict__ ctx, int batch,
                                                  int num_q_heads, float scale_log2, int split_tokens,
                                                  int num_splits, int max_len, float* __restrict__ part_o,
                                                  float* __restrict__ part_ml, const bf16_t* __restrict__ k_new,
                                                  const bf16_t* __restrict__ v_new, int bx, int by, int bz,
                                                  int nbx, DecodeBf16Smem<D, G>& sm) {
  static_assert(G >= 1 && G <= 16, "the q-heads of a KV head are the 16 MFMA columns");
  constexpr int KC = D / 32, DT = D / 16, TK = 32;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, j4 = lane >> 4;
  // keys a request may have: max_context_len, which the host has checked
  // against the table's capacity; a longer context is cut to it and flagged
  const int cap = max_len;
  const int hl = pool.heads_per_shard;
  const int bs = pool.block_size;
  const size_t block_stride = (size_t)hl * bs * D;
  const int tile_bytes = bs * D * 2;

  // One segment: keys [start, end) of request b and KV head kvh; the result
  // goes to out when final_out, else to the partial rows prow + g * pstride.
  // With `last` (append mode) the request's new key L-1 follows the segment:
  // its K/V come from k_new / v_new, are added to the softmax in the merge,
  // and are written to the pool there; the tiles stop at L-1.
  struct Seg {
    int b, kvh, start, end;
    bool final_out;
    size_t prow;
    int pstride;
    bool last;
  };
  // the segment whose loads are being issued: its KV head's pools, its
  // table, its end (wave-uniform, in scalar registers)
  const bf16_t* kpool = nullptr;
  const bf16_t* vpool = nullptr;
  size_t head_off = 0;                                          // elements
  const int32_t* table = bt;
  int end = 0;
  // q as the B operand of S^T: head l16 (zero columns past G), dims 32c + 8 j4
  uint4 qf[KC];
  auto bind = [&](const Seg& sg) {
    const int sh = sg.kvh / hl, lh = sg.kvh - sh * hl;
    kpool = reinterpret_cast<const bf16_t*>(pool.k[sh]);
    vpool = reinterpret_cast<const bf16_t*>(pool.v[sh]);
    head_off = (size_t)lh * bs * D;
    table = bt + (size_t)sg.b * bt_stride;
    end = sg.end;
    const bool hv = l16 < G;
    const bf16_t* qrow = q + ((size_t)sg.b * num_q_heads + (size_t)sg.kvh * G + (hv ? l16 : 0)) * D + 8 * j4;
#pragma unroll
    for (int c = 0; c < KC; ++c) qf[c] = hv ? *reinterpret_cast<const uint4*>(qrow + 32 * c) : make_uint4(0, 0, 0, 0);
  };

  const int k_voff = (l16 * D + 8 * j4) * 2;                    // bytes within a half's 16 K rows
  const int v_voff = (l16 * bs + 4 * j4) * 2;                   // dim l16 of a 16-dim slab, 4 keys
  // block ids of the tile at k0 (-1: past the split or out of range) from
  // the table entries of its two halves (raw, read beforehand)
  auto ids_from = [&](int k0, const int (&raw)[2], int (&ids)[2]) {
    bool bad = false;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int key16 = k0 + 16 * h;
      const int blk = key16 < end ? raw[h] : -1;
      const bool ok = blk >= 0 && blk < pool.num_blocks;
      bad |= key16 < end && !ok;
      // the id is wave-uniform; saying so keeps the descriptors built from
      // it in scalar registers
      ids[h] = __builtin_amdgcn_readfirstlane(ok ? blk : -1);
    }
    if (bad && lane == 0) flag_error(pool.err, PKV_ERRBIT_BLOCK_ID);
  };
  // the same, reading the entries
  auto fetch_ids = [&](int k0, int (&ids)[2]) {
    int raw[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) raw[h] = k0 + 16 * h < end ? table[(k0 + 16 * h) >> pool.bs_shift] : -1;
    ids_from(k0, raw, ids);
  };
  auto issue_k = [&](int k0, DecodeTile<D>& r) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bool ok = r.blk[h] >= 0;
      const buffer_rsrc_t rs = buffer_rsrc(kpool + (ok ? (size_t)r.blk[h] * block_stride + head_off : 0),
                                           ok ? tile_bytes : 0);
      const int soff = ((k0 + 16 * h) & (bs - 1)) * D * 2;
#pragma unroll
      for (int c = 0; c < KC; ++c) r.k[h][c] = buffer_load16<kCached>(rs, k_voff + 64 * c, soff);
    }
  };
  auto issue_v = [&](int k0, DecodeTile<D>& r) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bool ok = r.blk[h] >= 0;
      const buffer_rsrc_t rs = buffer_rsrc(vpool + (ok ? (size_t)r.blk[h] * block_stride + head_off : 0),
                                           ok ? tile_bytes : 0);
      const int soff = ((k0 + 16 * h) & (bs - 1)) * 2;
#pragma unroll
      for (int mm = 0; mm < DT; ++mm) r.v[h][mm] = buffer_load8<kStream>(rs, v_voff, soff + mm * 32 * bs);
    }
  };

  f32x4_t o[DT];
  // running max of head l16 (log2 units; finite start, so a tile whose keys
  // are all absent gives p = exp2(-inf) = 0) and this lane's share of the sum
  float m = -1e30f, lsum = 0.f;
  constexpr uint32_t kOnes = 0x3F803F80u;       // bf16 (1, 1)

  // one tile: S^T, softmax, P V; the registers are refilled with the tile
  // at k0_next (< 0: none) as they are consumed, whose block ids were read
  // one tile earlier into ids_next; then the ids of the tile at k0_next2
  int ids_next[2] = {-1, -1};
  auto process = [&](int k0, DecodeTile<D>& r, int k0_next, int k0_next2) {
    f32x4_t st[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      st[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) st[h] = mfma_qk(r.k[h][c], qf[c], st[h]);
    }
    const bool ok0 = r.blk[0] >= 0, ok1 = r.blk[1] >= 0;
    if (k0_next >= 0) {
      r.blk[0] = ids_next[0];
      r.blk[1] = ids_next[1];
      issue_k(k0_next, r);
      if (k0_next2 >= 0) fetch_ids(k0_next2, ids_next);
    }
    float x[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = k0 + 16 * h + 4 * j4 + rr;
        const bool valid = key < end && (h ? ok1 : ok0);
        x[h][rr] = valid ? st[h][rr] : -INFINITY;
        mx = fmaxf(mx, x[h][rr]);
      }
    mx = col_max(mx) * scale_log2;
    const bool grow = mx > m + kDecodeSlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {          // wave-uniform branch
      const float mnew = grow ? mx : m;
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int mm = 0; mm < DT; ++mm) o[mm] *= alpha;
    }
    uint2 pb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float p[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) p[rr] = __builtin_amdgcn_exp2f(fmaf(x[h][rr], scale_log2, -m));
      pb[h] = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
      lsum = dot2_bf16(pb[h].x, kOnes, lsum);         // the sum of the same bf16 p the MFMA uses
      lsum = dot2_bf16(pb[h].y, kOnes, lsum);
    }
    // the request's last tile: V entries of keys past the context hold
    // arbitrary bits and must be zero (p = 0 times a NaN pattern is NaN)
    if (k0 + TK > end) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int nvalid = end - (k0 + 16 * h + 4 * j4);
#pragma unroll
        for (int mm = 0; mm < DT; ++mm) {
          if (nvalid <= 0) r.v[h][mm] = make_uint2(0, 0);
          else if (nvalid < 4) {
            uint32_t* w = reinterpret_cast<uint32_t*>(&r.v[h][mm]);
#pragma unroll
            for (int e = 1; e < 4; ++e)
              if (e >= nvalid) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
          }
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int mm = 0; mm < DT; ++mm) o[mm] = mfma_pv(r.v[h][mm], pb[h], o[mm]);
    if (k0_next >= 0) issue_v(k0_next, r);
  };

  // two tiles in flight per wave: ra holds tiles wave + 8i, rb tiles wave + 8i + 4
  DecodeTile<D> ra, rb;
  constexpr int W = kWaves;
  // q, the block ids and the loads of a segment's first tiles; issued for
  // the next segment as soon as this wave is done with the current one's
  // tiles, ahead of the current segment's merge
  auto prologue = [&](const Seg& sg) {
    bind(sg);
    const int ntiles = (sg.end - sg.start + TK - 1) / TK;
    if (wave < ntiles) {
      fetch_ids(sg.start + wave * TK, ra.blk);
      issue_k(sg.start + wave * TK, ra);
      issue_v(sg.start + wave * TK, ra);
    }
    if (wave + W < ntiles) {
      fetch_ids(sg.start + (wave + W) * TK, rb.blk);
      issue_k(sg.start + (wave + W) * TK, rb);
      issue_v(sg.start + (wave + W) * TK, rb);
    }
    if (wave + 2 * W < ntiles) fetch_ids(sg.start + (wave + 2 * W) * TK, ids_next);
  };
  // the same, with the block-table entries of the first three tiles read
  // ahead (before the context length was known)
  auto prologue_pre = [&](const Seg& sg, const int (&raw)[3][2]) {
    bind(sg);
    const int ntiles = (sg.end - sg.start + TK - 1) / TK;
    if (wave < ntiles) {
      ids_from(sg.start + wave * TK, raw[0], ra.blk);
      issue_k(sg.start + wave * TK, ra);
      issue_v(sg.start + wave * TK, ra);
    }
    if (wave + W < ntiles) {
      ids_from(sg.start + (wave + W) * TK, raw[1], rb.blk);
      issue_k(sg.start + (wave + W) * TK, rb);
      issue_v(sg.start + (wave + W) * TK, rb);
    }
    if (wave + 2 * W < ntiles) ids_from(sg.start + (wave + 2 * W) * TK, raw[2], ids_next);
  };
  // the tiles of the bound segment (its prologue has run)
  auto body = [&](const Seg& sg) {
#pragma unroll
    for (int mm = 0; mm < DT; ++mm) o[mm] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m = -1e30f;
    lsum = 0.f;
    const int start = sg.start;
    const int ntiles = (sg.end - start + TK - 1) / TK;
    auto at = [&](int t) { return t < ntiles ? start + t * TK : -1; };
    for (int t = wave; t < ntiles; t += 2 * W) {
      process(start + t * TK, ra, at(t + 2 * W), at(t + 3 * W));
      if (t + W < ntiles) process(start + (t + W) * TK, rb, at(t + 3 * W), at(t + 4 * W));
    }
  };
  // The appended key of a segment (append mode, last piece of the request):
  // its row is written to the pool at position L-1 (the tiles never read
  // that slot) and its score for each q-head computed into LDS (wave w takes
  // heads w, w+4, ...; a lane 1 or 2 dims); a block id outside the pool
  // makes it absent, as for any key.  Run by every wave right after its
  // tiles, before the next segment's loads are issued (fewer live
  // registers); the merge's first barrier publishes the scores.
  auto append_key = [&](const Seg& sg) -> bool {
    bool add_new = false;
    if (APPEND && sg.last) {
      const int L = sg.end + 1;
      const bf16_t* kn = k_new + ((size_t)sg.b * (num_q_heads / G) + sg.kvh) * D;
      const bf16_t* vn = v_new + ((size_t)sg.b * (num_q_heads / G) + sg.kvh) * D;
      const int32_t* tb = bt + (size_t)sg.b * bt_stride;
      const int blk = tb[(L - 1) >> pool.bs_shift];
      add_new = blk >= 0 && blk < pool.num_blocks;
      if (add_new) {
        for (int g = wave; g < G; g += kWaves) {
          const bf16_t* qr = q + ((size_t)sg.b * num_q_heads + (size_t)sg.kvh * G + g) * D;
          float part = 0.f;
          for (int d = lane; d < D; d += 64) part = fmaf(bf16_to_f32(qr[d]), bf16_to_f32(kn[d]), part);
#pragma unroll
          for (int o2 = 32; o2 >= 1; o2 >>= 1) part += __shfl_xor(part, o2);
          if (lane == 0) sm.snew[g] = part * scale_log2;
        }
        const int sh = sg.kvh / hl, lh = sg.kvh - sh * hl;
        const size_t tile = ((size_t)blk * hl + lh) * ((size_t)bs * D);
        const int off = (L - 1) & (bs - 1);
        bf16_t* kp = const_cast<bf16_t*>(reinterpret_cast<const bf16_t*>(pool.k[sh])) + tile + (size_t)off * D;
        bf16_t* vp = const_cast<bf16_t*>(reinterpret_cast<const bf16_t*>(pool.v[sh])) + tile + off;
        for (int d = threadIdx.x; d < D; d += kThreads) {
          kp[d] = kn[d];
          vp[(size_t)d * bs] = vn[d];
        }
      } else if (threadIdx.x == 0) {
        flag_error(pool.err, PKV_ERRBIT_BLOCK_ID);
      }
    }
    return add_new;
  };
  // the 4 waves' (m, l, acc) of a segment, combined and written
  auto merge = [&](const Seg& sg, bool add_new) {
    lsum = col_sum(lsum);
    if (l16 < G) {
      if (j4 == 0) {
        sm.m[wave][l16] = m;
        sm.l[wave][l16] = lsum;
      }
#pragma unroll
      for (int mm = 0; mm < DT; ++mm)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) sm.acc[wave][l16][16 * mm + 4 * j4 + rr] = o[mm][rr];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < G * D; i += kThreads) {
      const int g = i / D, d = i - g * D;
      float mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm.m[w][g]);
      float l = 0.f, acc = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(sm.m[w][g] - mx);
        l += sm.l[w][g] * f;
        acc += sm.acc[w][g][d] * f;
      }
      if (add_new) {
        const float sn = sm.snew[g];
        const float mf = fmaxf(mx, sn);
        const float fo = __builtin_amdgcn_exp2f(mx - mf), fn = __builtin_amdgcn_exp2f(sn - mf);
        const bf16_t* vn = v_new + ((size_t)sg.b * (num_q_heads / G) + sg.kvh) * D;
        l = l * fo + fn;
        acc = acc * fo + fn * bf16_to_f32(vn[d]);
        mx = mf;
      }
      const int h = sg.kvh * G + g;
      if (sg.final_out) {
        out[((size_t)sg.b * num_q_heads + h) * D + d] = f32_to_bf16(acc / l);
      } else {
        const size_t row = sg.prow + (size_t)g * sg.pstride;
        part_o[row * D + d] = acc;
        if (d == 0) {
          part_ml[row * 2 + 0] = mx;
          part_ml[row * 2 + 1] = l;
        }
      }
    }
    __syncthreads();                              // the merge buffers are free again
  };

  if constexpr (!STREAM) {
    // one segment: split bx of (request bz, KV head by)
    const int split = bx, kvh = by, b = bz;
    // the table entries of this wave's first three tiles do not depend on
    // the context length: read them together with it
    int raw[3][2];
    {
      const int32_t* tb = bt + (size_t)b * bt_stride;
#pragma unroll
      for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          raw[i][h] = tb[min((split * split_tokens + (wave + i * kWaves) * TK + 16 * h) >> pool.bs_shift, bt_stride - 1)];
    }
    int L = ctx[b];
    if (L > cap) {                              // past max_context_len: cut, flagged
      if (threadIdx.x == 0 && split == 0 && kvh == 0) flag_error(pool.err, PKV_ERRBIT_CONTEXT);
      L = cap;
    }
    const int start = split * split_tokens;
    if (start >= L) return;
    const int end = min(L, start + split_tokens);
    const bool last = APPEND && ctx[b] <= cap && end == L;
    const Seg sg{b, kvh, start, last ? end - 1 : end, L <= split_tokens,
                 ((size_t)b * num_q_heads + (size_t)kvh * G) * num_splits + split, num_splits, last};
    prologue_pre(sg, raw);
    body(sg);
    const bool add_new = append_key(sg);
    merge(sg, add_new);
  } else {
    // stream split: workgroup w takes the pair-tiles [w W / NW, (w+1) W / NW)
    // of the W = Hkv * sum_b ceil(L_b / 32) tiles of the batch, ordered by
    // request, KV head, key; a pair met by several workgroups leaves one
    // partial per workgroup, in row (w + pair index) * G + g.  NW is the grid
    // size or W if smaller (the grid is sized from max_context_len, an upper
    // bound): then every workgroup below NW has at least one tile and writes
    // every partial row the merge kernel will read, and the rest exit.
    const int hkv = num_q_heads / G;
    const TileScan tot = scan_tiles(ctx, batch, cap, hkv, -1, 0);
    if (tot.over && bx == 0 && threadIdx.x == 0) flag_error(pool.err, PKV_ERRBIT_CONTEXT);
    const long long Wt = tot.total;
    const long long NW = min((long long)nbx, Wt), w = bx;
    if (w >= NW) return;
    long long t = w * Wt / NW;
    const long long t1 = (w + 1) * Wt / NW;
    const TileScan at = scan_tiles(ctx, batch, cap, hkv, t, 0);
    int b = at.b;
    long long base = at.base;
    // the segments of this workgroup's range, in order
    auto next_seg = [&](Seg& sg) -> bool {
      while (t < t1) {
        const int raw = ctx[b];
        const int L = max(min(raw, cap), 0);
        const int ntb = (L + TK - 1) / TK;
        if (ntb == 0) {                         // an empty request holds no tiles
          ++b;
          continue;
        }
        const int kvh = (int)((t - base) / ntb);
        const long long pstart = base + (long long)kvh * ntb;
        const long long seg_end = min(t1, pstart + ntb);
        sg.b = b;
        sg.kvh = kvh;
        sg.start = (int)(t - pstart) * TK;
        sg.end = min(L, (int)(seg_end - pstart) * TK);
        sg.final_out = stream_owner(pstart, NW, Wt) == stream_owner(pstart + ntb - 1, NW, Wt);
        sg.prow = (size_t)(w + (long long)b * hkv + kvh) * G;
        sg.pstride = 1;
        sg.last = APPEND && raw <= cap && sg.end == L;
        if (sg.last) sg.end = L - 1;
        t = seg_end;
        if (t == base + (long long)hkv * ntb) {
          base = t;
          ++b;
        }
        return true;
      }
      return false;
    };
    Seg cur{}, nxt{};
    if (!next_seg(cur)) return;
    prologue(cur);
    while (true) {
      body(cur);
      const bool add_new = append_key(cur);
      const bool more = next_seg(nxt);
      if (more) prologue(nxt);
      merge(cur, add_new);
      if (!more) break;
      cur = nxt;
    }
  }
}

}  // namespace decode_impl
}  // namespace pkv
