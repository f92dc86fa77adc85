// bf16 paged causal prefill attention for one workgroup, shared by the
// prefill kernel and the mixed-batch kernel.  The design is described at the
// top of attn_prefill.hip.
#pragma once

#include <type_traits>

#include "pkv_internal.h"

namespace pkv {
namespace prefill_impl {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kXcds = 8;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
struct f32x16x2 {
  f32x16_t v[2];
};

__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4_t mfma16x32(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Q scaled by scale * log2(e) once, at load: bf16 products rounded to bf16.
__device__ __forceinline__ uint4 scale_bf16x8(uint4 v, float c) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(bf16_lo(w[i]) * c, bf16_hi(w[i]) * c);
  return make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ float round_bf16(float x) { return bf16_to_f32(f32_to_bf16(x)); }

// Row of the 32-key half tile that lane row m of the S^T MFMA's A operand
// holds: chosen so that accumulator registers 8s..8s+7 of a lane in half
// h = lane/32 are keys 16s + 8h + 0..7.
__device__ __forceinline__ int key_perm(int m) {
  return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

template <int D>
struct PrefillCfg {
  static constexpr int BM = 128, BN = 64, THREADS = 256;
  static constexpr int KS = D / 16;            // MFMA k-steps of q.k
  static constexpr int DT = D / 32;            // 32-dim output tiles
  static constexpr int KCH = D / 8;            // 16-byte chunks per K row
  static constexpr int TILE = BN * D * 2;      // bytes of one K (or V) tile in LDS
  static constexpr int KRPI = 1024 / (2 * D);  // K rows per 1 KB DMA instruction
  static constexpr int NDMA = D / 32;          // DMA instructions per wave for its group's K (and V)
  static constexpr int VGRP = D * 32;          // bytes of one 16-key group of the V tile
};

// Running max update rule: the max used for exp2 moves only when a tile's
// max exceeds it by more than this (log2 units), so p <= 2^8 and the O
// accumulators are rescaled rarely.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ void lds_dma16(buffer_rsrc_t r, char* lds, int voffset, int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voffset, soffset, 0,
                                           0);
}
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Order of the MFMAs of one step (block) for head dim D: eight groups,
// S0 S1 S2 PV0 S3 PV1 PV2 PV3, where Sq is quarter q of the S^T = K Q^T
// MFMAs (QPG each) and PVc the O^T += V^T P^T MFMAs of quarter c of P (DT
// each).  The 16 pairs of P values a lane forms are spread over the slots
// so that quarter c is complete before PVc, and the row max of each S half
// is taken a few slots after its last MFMA.
template <int D>
struct BlockPlan {
  static constexpr int KS = D / 16, DT = D / 32, QPG = KS / 2;
  static constexpr int NS = 4 * QPG + 4 * DT;                   // MFMA slots
  static constexpr int gtype(int g) { return (g == 3 || g >= 5) ? 1 : 0; }   // 0: S, 1: PV
  static constexpr int gq(int g) { return g == 3 ? 0 : g == 4 ? 3 : g == 5 ? 1 : g == 6 ? 2 : g == 7 ? 3 : g; }
  static constexpr int gstart(int g) {
    int s = 0;
    for (int i = 0; i < g; ++i) s += gtype(i) ? DT : QPG;
    return s;
  }
  static constexpr int group_of(int s) {
    int g = 0;
    while (g < 7 && gstart(g + 1) <= s) ++g;
    return g;
  }
  static constexpr int pair_slot(int j) { return j * (NS - NS / 8) / 16; }
  static constexpr int max_slot(int h, int k) {
    const int start = h ? gstart(5) + 2 : gstart(2) + 2 * (QPG / 2);
    const int end = h ? NS - 1 : gstart(5);
    return start + k * (end - start) / 8;
  }
  // every quarter of P is complete before its PV group; every half of S is
  // complete before its max is taken
  static constexpr bool valid() {
    for (int j = 0; j < 16; ++j) {
      const int c = j >> 2;
      int g = 0;
      while (!(gtype(g) == 1 && gq(g) == c)) ++g;
      if (pair_slot(j) >= gstart(g)) return false;
    }
    for (int k = 0; k < 8; ++k) {
      if (max_slot(0, k) < gstart(2) + 1 || max_slot(0, k) >= NS) return false;
      if (max_slot(1, k) < gstart(5) + 1 || max_slot(1, k) >= NS) return false;
    }
    return true;
  }
};
static_assert(BlockPlan<128>::valid() && BlockPlan<64>::valid(), "block schedule");

// The LDS of one workgroup: double-buffered K and V tiles per key-tile
// group, four separate arrays so the compiler sees that a DMA into one
// buffer never overlaps reads of another.  Declared by the kernel (the
// mixed-batch kernel overlays them with the decode workgroups' LDS).
template <int D, int NG>
using PrefillTiles = char[NG][PrefillCfg<D>::TILE];
template <int D, int NG>
struct PrefillSmem {
  __attribute__((aligned(1024))) PrefillTiles<D, NG> kb0, kb1, vb0, vb1;
};

// One workgroup's work: block `bid` of a grid of `nblocks` (a multiple of
// the XCD count) over `total_items` work items.  NG = key-tile groups per
// workgroup.  NG = 1: 4 waves, two workgroups per CU.  NG = 2 (small
// grids): 8 waves in two groups of 4 that share the queries and walk
// alternate key tiles with their own buffers, merging their (m, l, O)
// through LDS at the end; one workgroup per CU.
template <int D, int NG>
__device__ __forceinline__ void prefill_bf16_block(PoolDev pool, const bf16_t* __restrict__ q,
                                                   bf16_t* __restrict__ out, const int32_t* __restrict__ bt,
                                                   int bt_stride, const int32_t* __restrict__ start_loc,
                                                   const int32_t* __restrict__ chunk_start, int batch, int ntiles,
                                                   int num_q_heads, int group, float scale_log2, int total_items,
                                                   int max_total, int bid, int nblocks,
                                                   PrefillTiles<D, NG>& kb0, PrefillTiles<D, NG>& kb1,
                                                   PrefillTiles<D, NG>& vb0, PrefillTiles<D, NG>& vb1) {
  using C = PrefillCfg<D>;

  // ---- work item (XCD-contiguous runs) ----
  const int per_xcd = nblocks / kXcds;
  const int item = (bid % kXcds) * per_xcd + bid / kXcds;
  if (item >= total_items) return;
  const int per_kvh = ntiles * group * batch;
  const int kvh = item / per_kvh;
  int rem = item - kvh * per_kvh;
  const int qt = ntiles - 1 - rem / (group * batch);
  rem %= group * batch;
  const int g = rem / batch;
  const int b = rem - g * batch;
  const int h = kvh * group + g;

  const int q0 = start_loc[b];
  const int T = start_loc[b + 1] - q0;
  if (qt * C::BM >= T) return;
  const int S = chunk_start[b];
  // keys [0, S+T), cut to max_total_len (which the host has checked against
  // the table's capacity) and flagged if a chunk reaches past it
  const int kv_len = min(S + T, max_total);
  if (S + T > max_total && threadIdx.x == 0) flag_error(pool.err, PKV_ERRBIT_CONTEXT);
  const int kend = min(kv_len, S + min(T, (qt + 1) * C::BM));   // one past the last query's position

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave8 = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int grp = wave8 >> 2, wave = wave8 & 3;                 // key-tile group, wave within it
  const int half = lane >> 5, l32 = lane & 31;
  const int hl = pool.heads_per_shard;
  const int sh = kvh / hl, lh = kvh - sh * hl;
  const char* kpool = reinterpret_cast<const char*>(pool.k[sh]);
  const char* vpool = reinterpret_cast<const char*>(pool.v[sh]);
  const int bs = pool.block_size;
  const int tile_bytes = bs * D * 2;                            // one (block, head) tile
  const size_t head_off = (size_t)lh * tile_bytes;
  const size_t block_stride = (size_t)hl * tile_bytes;
  const int32_t* table = bt + (size_t)b * bt_stride;

  // ---- this lane's query row and its Q fragments (B operand of S^T) ----
  const int qrel = qt * C::BM + wave * 32 + l32;
  // the causal limit of this lane's query: its position, or the last key
  // when the chunk is cut at max_total_len (keys past it are never seen)
  const int qpos = min(S + qrel, kv_len - 1);
  uint4 qf[C::KS];
  {
    const bool ok = qrel < T;
    const bf16_t* qrow = q + ((size_t)(q0 + (ok ? qrel : 0)) * num_q_heads + h) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      qf[s] = ok ? *reinterpret_cast<const uint4*>(qrow + 16 * s) : make_uint4(0, 0, 0, 0);
      qf[s] = scale_bf16x8(qf[s], scale_log2);
    }
  }
  const int wave_first_q = min(S + qt * C::BM + wave * 32, kv_len - 1);

  // ---- tile loads: LDS DMA, wave w moves 16-key group w of K and of V ----
  // K tile in LDS: row r holds key 32(r/32) + key_perm(r%32) (so that the
  // accumulator registers a lane converts to bf16 are 8 consecutive keys);
  // its 16-byte chunk c sits at position c ^ (r % KCH), so the MFMA's
  // row-per-lane reads of one chunk hit distinct banks.  A DMA instruction
  // fills KRPI whole rows (1 KB); lane t fetches the chunk that belongs at
  // its slot.
  int k_voff[C::NDMA];
#pragma unroll
  for (int jj = 0; jj < C::NDMA; ++jj) {
    const int r = C::KRPI * jj + lane / C::KCH;                 // row within the group (0..15)
    const int c = (lane % C::KCH) ^ (r & (C::KCH - 1));
    k_voff[jj] = (key_perm(r) * D + 8 * c) * 2;
  }
  // V tile in LDS: [group][dim][16 keys], the two 8-key halves of a dim row
  // swapped when bit 2 xor bit 3 of the dim is set, so that the 16-byte
  // reads of any 16 consecutive dims (one half each) fall in 16 distinct
  // bank groups.  A DMA instruction fills 32 dims of one group.
  int v_dim[C::NDMA], v_kh[C::NDMA];
#pragma unroll
  for (int jj = 0; jj < C::NDMA; ++jj) {
    v_dim[jj] = 32 * jj + (lane >> 1);
    v_kh[jj] = (lane & 1) ^ (((v_dim[jj] >> 2) ^ (v_dim[jj] >> 3)) & 1);
  }
  // ---- block ids, 64 key tiles at a time.  Lane j of idv[P & 1] holds the
  // block of this wave's 16-key group in tile 64P + j (-1 when the group
  // lies past the request or its table entry is not a block of the pool);
  // lane j of absv[P & 1] holds the bits of that tile's absent groups.  The
  // table entries of period P+1 are read while period P is in use and
  // turned into these vectors one step later, after the wait that ends
  // every step's loads, so no step waits on the table. ----
  const int nkt = (kend + C::BN - 1) / C::BN;
  const int nper = (nkt + 63) >> 6;
  const int nbt = max((kv_len + bs - 1) >> pool.bs_shift, 1);   // table entries in use
  int raw[4];
  int idv0 = -1, idv1 = -1, absv0 = 0, absv1 = 0;
  auto load_raw = [&](int period) {
    const int t = 64 * period + lane;
#pragma unroll
    for (int r = 0; r < 4; ++r) raw[r] = table[min((t * C::BN + 16 * r) >> pool.bs_shift, nbt - 1)];
  };
  auto convert = [&](int period) {
    const int t = 64 * period + lane;
    int own = -1, absent = 0;
    bool bad = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool in = t * C::BN + 16 * r < kv_len;
      const bool valid = (unsigned)raw[r] < (unsigned)pool.num_blocks;
      if (!(in && valid)) absent |= 1 << r;
      if (r == wave) {
        own = in && valid ? raw[r] : -1;
        bad = in && !valid && t < nkt;
      }
    }
    if (__builtin_amdgcn_ballot_w64(bad) && lane == 0) flag_error(pool.err, PKV_ERRBIT_BLOCK_ID);
    if (period & 1) {
      idv1 = own;
      absv1 = absent;
    } else {
      idv0 = own;
      absv0 = absent;
    }
  };
  int have = 1;        // periods [0, have) are in idv/absv
  bool pend = false;   // raw holds the entries of period `have`
  load_raw(0);
  convert(0);
  if (nper > 1) {
    load_raw(1);
    pend = true;
  }
  // tile u's absent-group bits; this wave's block id in *blk_own
  auto tile_ids = [&](int u, int* blk_own) -> uint32_t {
    const bool odd = (u >> 6) & 1;
    *blk_own = __builtin_amdgcn_readlane(odd ? idv1 : idv0, u & 63);
    return __builtin_amdgcn_readlane(odd ? absv1 : absv0, u & 63);
  };
  auto dma_k = [&](int kt, char* kbuf, int blk) {
    const int key16 = kt * C::BN + 16 * wave;
    const bool ok = blk >= 0;
    const buffer_rsrc_t rs = buffer_rsrc(kpool + (ok ? (size_t)blk * block_stride + head_off : 0), ok ? tile_bytes : 0);
    const int soff = (key16 & (bs - 1)) * D * 2;
    char* dst = kbuf + (16 * wave) * 2 * D;
#pragma unroll
    for (int jj = 0; jj < C::NDMA; ++jj) lds_dma16(rs, dst + jj * 1024, k_voff[jj], soff);
  };
  auto dma_v = [&](int kt, char* vbuf, int blk) {
    const int key16 = kt * C::BN + 16 * wave;
    const bool ok = blk >= 0;
    const buffer_rsrc_t rs = buffer_rsrc(vpool + (ok ? (size_t)blk * block_stride + head_off : 0), ok ? tile_bytes : 0);
    const int soff = (key16 & (bs - 1)) * 2;
    char* dst = vbuf + wave * C::VGRP;
#pragma unroll
    for (int jj = 0; jj < C::NDMA; ++jj) {
      // an 8-key half wholly past the request reads zeros (out of range)
      const bool past = key16 + 8 * v_kh[jj] >= kv_len;
      lds_dma16(rs, dst + jj * 1024, past ? 0x40000000 : (v_dim[jj] * bs + 8 * v_kh[jj]) * 2, soff);
    }
  };
  // the request's last tile: V entries of keys in [kv_len, next multiple of
  // 8) sit in the same 16 bytes as valid keys and hold arbitrary bits; the
  // wave that loaded them zeroes them (p = 0 times a NaN pattern is NaN)
  auto fix_tail = [&](int kt, char* vbuf) {
    const int rel = kv_len - kt * C::BN;                        // valid keys in this tile
    if (rel >= C::BN || (rel & 7) == 0 || (rel >> 4) != wave) return;
    const int kh = (rel >> 3) & 1, e0 = rel & 7;
    char* base = vbuf + wave * C::VGRP;
    for (int d = lane; d < D; d += 64) {
      uint4* p = reinterpret_cast<uint4*>(base + d * 32 + ((kh ^ ((d >> 2) ^ (d >> 3)) & 1) << 4));
      uint4 v = *p;
      uint32_t* w = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e >= e0) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
      *p = v;
    }
  };

  // ---- LDS read addresses ----
  // K: row 32i + l32, chunk 2s + half at position (2s + half) ^ (l32 % KCH):
  // address = kx ^ 32s ^ (32 rows * i), XORs of disjoint bits with a
  // per-lane constant
  const int kx = l32 * 2 * D + (((half ^ (l32 & (C::KCH - 1))) & 1) << 4) + (((l32 & (C::KCH - 1)) >> 1) << 5);
  // V: dim 32t + l32, keys 32i + 16sp + 8half -> group 2i + sp, half `half`
  const int vx = l32 * 32 + (((half ^ (l32 >> 2) ^ (l32 >> 3)) & 1) << 4);

  f32x16_t o[C::DT];
#pragma unroll
  for (int t = 0; t < C::DT; ++t) o[t] = f32x16_t{};
  // Softmax state, in log2 units.  Q carries scale * log2(e), and the S
  // MFMA chain subtracts the running max m itself: its first MFMA per
  // 32-key half multiplies a constant A (1.0 in head-dim slot 0 of every
  // key row: aones) by B = -m (bf16, slot 0 of the lane's query: mq), so
  // the accumulator starts at -m and p = exp2(S) needs no multiply-add.  m
  // is kept bf16-representable, so the MFMA subtracts exactly the m used
  // in every rescale.  It is 0 until the first tile with a valid key sets
  // it (mset).
  float m = 0.f;
  bool mset = false;
  const uint4 aones = make_uint4(half == 0 ? 0x3F80u : 0u, 0u, 0u, 0u);
  uint4 mq = make_uint4(0u, 0u, 0u, 0u);
  // Row sums of P on the matrix cores: one 16x16x32 MFMA per 16 keys whose
  // B operand is the P register quad as laid out for the 32x32x16 product
  // (lane l: query l%32, keys 8(l/32)..+7) and whose constant A has row 0
  // selecting the lanes of queries 0..15 (lanes 0, 32: K groups 0, 2) and
  // row 1 those of queries 16..31 (lanes 17, 49: K groups 1, 3); so lanes
  // 0..15 accumulate the sums of queries lane (rs[0]) and lane + 16 (rs[1]).
  f32x4_t rs = f32x4_t{};
  const uint32_t ones_row = (lane == 0 || lane == 32 || lane == 17 || lane == 49) ? 0x3F803F80u : 0u;
  const uint4 arow = make_uint4(ones_row, ones_row, ones_row, ones_row);

  // row max of a score tile over both lane halves
  auto rowmax = [&](const f32x16x2& st) -> float {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(st.v[i][r], st.v[i][r + 1]));
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  };
  // the first tile's S (m = 0 then, so no -m term)
  auto qk = [&](const char* kbuf) -> f32x16x2 {
    f32x16x2 st;
    uint4 kf[2][C::KS];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int s = 0; s < C::KS; ++s)
        kf[i][s] = *reinterpret_cast<const uint4*>(kbuf + (kx ^ (32 * s) ^ (i * 32 * 2 * D)));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      st.v[i] = f32x16_t{};
#pragma unroll
      for (int s = 0; s < C::KS; ++s) st.v[i] = mfma32(kf[i][s], qf[s], st.v[i]);
    }
    return st;
  };
  // fragment qi of the S MFMAs (32-key half qi / KS, k-step qi % KS) and
  // fragment t of quarter c of the V tile
  auto ldk = [&](const char* kbuf, int qi) -> uint4 {
    return *reinterpret_cast<const uint4*>(kbuf + (kx ^ (32 * (qi % C::KS)) ^ ((qi / C::KS) * 32 * 2 * D)));
  };
  auto ldv = [&](const char* vbuf, int c, int t) -> uint4 {
    return *reinterpret_cast<const uint4*>(vbuf + vx + c * C::VGRP + t * 1024);
  };

  char* const k0b = kb0[grp];
  char* const k1b = kb1[grp];
  char* const v0b = vb0[grp];
  char* const v1b = vb1[grp];
  // prologue: this group's first two K tiles and first V tile; its first S
  int blk0 = -1, blk1 = -1;
  uint32_t absent_cur = 0, absent_next = 0;
  int blk_next = -1;
  if (grp < nkt) {
    absent_cur = tile_ids(grp, &blk0);
    dma_k(grp, k0b, blk0);
    dma_v(grp, v0b, blk0);
  }
  if (grp + NG < nkt) {
    absent_next = tile_ids(grp + NG, &blk1);
    dma_k(grp + NG, k1b, blk1);
    blk_next = blk1;
  }
  wait_dma();
  __syncthreads();
  f32x16x2 sa = qk(k0b), sb;

  // A step of this group on key tile kt has three phases:
  //  * stats(kt): softmax statistics of S(kt) in registers: masks for
  //    causality (tiles reaching past this wave's first query) and for
  //    absent groups, the row max, the rare move of m with the rescale of O
  //    and the row sums (the tile's scores then shifted by the same amount);
  //  * sync(kt): K(kt+NG) and V(kt) have arrived (this wave's loads, one
  //    step old); after the workgroup barrier every wave is past step
  //    kt-NG, so K(kt)'s buffer (kcur) and the buffer of V(kt-NG) (vnext)
  //    take the loads of K(kt+2NG) and V(kt+NG);
  //  * block(kt): S(kt+NG) = K Q^T - m into stn with the exponentials of
  //    P(kt) between its MFMAs, each quarter of P followed by its
  //    O^T += V^T P^T and row-sum MFMAs, in an order fixed by scheduling
  //    fences, every LDS fragment read a few MFMAs before its use, at raised
  //    wave priority so that the matrix cores go to the wave that has work
  //    for them.
  // Group 0 runs sync, block, stats of the next tile; group 1 (NG = 2) runs
  // sync, stats, block, so that between two barriers one group's softmax
  // work overlaps the other's MFMAs.  A step past the group's last tile only
  // keeps the barrier count equal across the groups.
  // O and the row sums times alpha (this lane's query)
  auto rescale = [&](float alpha) {
    const float a0 = __shfl(alpha, lane & 15), a1 = __shfl(alpha, (lane & 15) + 16);
    rs[0] *= a0;
    rs[1] *= a1;
#pragma unroll
    for (int t = 0; t < C::DT; ++t) o[t] *= alpha;
  };
  auto stats = [&](int kt, f32x16x2& st, uint32_t absent, float mx_block) {
    if (kt >= nkt) return;
    bool masked = false;
    const int kbase = kt * C::BN;
    if (kbase + C::BN - 1 > wave_first_q) {                    // wave-uniform
      // an opaque copy keeps the compares inside this branch (hoisted, they
      // would run on every tile)
      int d;
      asm volatile("v_mov_b32 %0, %1" : "=v"(d) : "v"(qpos - kbase - 8 * half));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * i + 16 * (r >> 3) + (r & 7) > d) st.v[i][r] = -INFINITY;
      masked = true;
    }
    if (absent) {                                               // wave-uniform, rare
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if ((absent >> (2 * i + (r >> 3))) & 1) st.v[i][r] = -INFINITY;
      masked = true;
    }
    // the block that computed S took its max; a masked tile takes it again
    const float mx = masked ? rowmax(st) : mx_block;
    // S already has m subtracted: move m when this tile exceeds it by the
    // slack, or to the first finite tile max of the row
    const bool grow = mset ? mx > kRescaleSlack : mx > -INFINITY;
    if (__builtin_amdgcn_ballot_w64(grow)) {                    // wave-uniform, rare
      const float delta = grow ? round_bf16(m + mx) - m : 0.f;
      m += delta;
      mset = mset || grow;
      mq.x = half == 0 ? (uint32_t)f32_to_bf16(-m) : 0u;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.v[i][r] -= delta;
      rescale(__builtin_amdgcn_exp2f(-delta));
    }
  };
  uint32_t absent_after = 0;
  int blk_after = -1;
  auto sync = [&](int kt, char* kcur, const char* vcur, char* vnext) {
    wait_dma();
    if (pend) {
      convert(have);
      ++have;
      pend = false;
    }
    if (kt < nkt) fix_tail(kt, const_cast<char*>(vcur));
    __syncthreads();
    absent_after = 0;
    blk_after = -1;
    const int u = kt + 2 * NG;
    if (u < nkt) {
      absent_after = tile_ids(u, &blk_after);
      dma_k(u, kcur, blk_after);
      // entering the last period read so far: read the next one's entries
      if (!pend && have < nper && (u >> 6) + 1 >= have) {
        load_raw(have);
        pend = true;
      }
    }
    if (kt + NG < nkt) dma_v(kt + NG, vnext, blk_next);
  };
  auto rotate = [&]() {
    absent_cur = absent_next;
    absent_next = absent_after;
    blk_next = blk_after;
  };
  auto block = [&](int kt, const char* knext, const char* vcur, const f32x16x2& st, f32x16x2& stn, float& mx_stn) {
    if (kt >= nkt) return;
    using BP = BlockPlan<D>;
    constexpr int R = 4;                                        // LDS fragments in flight
    // A operand (K or V fragment from LDS) of the MFMA in slot s
    auto frag = [&](int s) -> uint4 {
      const int g = BP::group_of(s), j = s - BP::gstart(g);
      return BP::gtype(g) == 0 ? ldk(knext, BP::gq(g) * BP::QPG + j) : ldv(vcur, BP::gq(g), j);
    };
    uint4 fr[R];
#pragma unroll
    for (int s = 0; s < R; ++s) fr[s] = frag(s);
    uint32_t pw[4][4];                                          // P in bf16 pairs, by quarter
    float mh[2] = {-INFINITY, -INFINITY};
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < BP::NS; ++s) {
      const int g = BP::group_of(s), j = s - BP::gstart(g), c = BP::gq(g);
      if (BP::gtype(g) == 0) {
        const int qi = c * BP::QPG + j, hs = qi / C::KS, ks = qi % C::KS;
        if (ks == 0) stn.v[hs] = mfma32(aones, mq, f32x16_t{});   // the -m term
        stn.v[hs] = mfma32(fr[s % R], qf[ks], stn.v[hs]);
      } else {
        const uint4 pc = make_uint4(pw[c][0], pw[c][1], pw[c][2], pw[c][3]);
        o[j] = mfma32(fr[s % R], pc, o[j]);
        if (j == 0) rs = mfma16x32(arow, pc, rs);                 // row sums of this quarter
      }
      if (s + R < BP::NS) fr[s % R] = frag(s + R);
      // the pairs of P placed in this slot: p = 2^S in bf16 for the MFMAs
#pragma unroll
      for (int pj = 0; pj < 16; ++pj) {
        if (BP::pair_slot(pj) != s) continue;
        const int pc = pj >> 2, w = pj & 3;
        const int i = pc >> 1, r = 8 * (pc & 1) + 2 * w;
        const float p0 = __builtin_amdgcn_exp2f(st.v[i][r]);
        const float p1 = __builtin_amdgcn_exp2f(st.v[i][r + 1]);
        pw[pc][w] = pack_bf16x2(p0, p1);
      }
      // the row max of S(kt+NG), a few registers per slot once each half
      // is complete
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (BP::max_slot(h, k) == s) mh[h] = fmaxf(fmaxf(mh[h], stn.v[h][2 * k]), stn.v[h][2 * k + 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    float mx = fmaxf(mh[0], mh[1]);
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx_stn = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  };

  // every group takes the same number of steps (one barrier each); st is
  // S(kt) on entry to a step, stn receives S(kt+NG); kcur holds K(kt),
  // knext K(kt+NG), vcur V(kt), vnext the buffer V(kt+NG) goes to
  const int nsteps = (nkt + NG - 1) / NG;
  const bool lead = NG == 1 || grp == 0;
  auto step = [&](int kt, char* kcur, const char* knext, const char* vcur, char* vnext, f32x16x2& st,
                  f32x16x2& stn, float mx_st, float& mx_stn) {
    sync(kt, kcur, vcur, vnext);
    if (!lead) stats(kt, st, absent_cur, mx_st);
    block(kt, knext, vcur, st, stn, mx_stn);
    rotate();
    if (lead) stats(kt + NG, stn, absent_cur, mx_stn);
  };
  float mxa = rowmax(sa), mxb = -INFINITY;
  if (lead) stats(grp, sa, absent_cur, mxa);
  for (int u = 0; u < nsteps; u += 2) {
    step(grp + NG * u, k0b, k1b, v0b, v1b, sa, sb, mxa, mxb);
    if (u + 1 < nsteps) step(grp + NG * (u + 1), k1b, k0b, v1b, v0b, sb, sa, mxb, mxa);
  }

  // the row sum of this lane's query over all keys of this group
  float ltot;
  {
    const int qq = lane & 31;
    const float t0 = __shfl(rs[0], qq & 15), t1 = __shfl(rs[1], qq & 15);
    ltot = qq < 16 ? t0 : t1;
  }
  // a row that never saw a valid key contributes nothing to the merge
  if (!mset) m = -1e30f;
  if constexpr (NG == 2) {
    // ---- merge group 1's (m, l, O) into group 0's, lane by lane (both
    // groups hold the same queries in the same layout) ----
    float* const ox = reinterpret_cast<float*>(wave < 2 ? &kb0[0][0] : &kb1[0][0]) + (wave & 1) * (16 * C::DT * 64);
    float* const mlx = reinterpret_cast<float*>(&vb0[0][0]) + wave * 128;
    __syncthreads();                                            // all buffers free
    if (grp == 1) {
#pragma unroll
      for (int t = 0; t < C::DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) ox[(16 * t + r) * 64 + lane] = o[t][r];
      mlx[lane] = m;
      mlx[64 + lane] = ltot;
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = mlx[lane], l1 = mlx[64 + lane];
    const float mn = fmaxf(m, m1);
    const float a0 = __builtin_amdgcn_exp2f(m - mn), a1 = __builtin_amdgcn_exp2f(m1 - mn);
    ltot = ltot * a0 + l1 * a1;
#pragma unroll
    for (int t = 0; t < C::DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[t][r] = o[t][r] * a0 + ox[(16 * t + r) * 64 + lane] * a1;
  }

  // ---- normalise and store: lane holds dims 32t + 8a + 4*half + 0..3 of its query ----
  if (qrel < T) {
    const float inv = 1.f / ltot;
    bf16_t* orow = out + ((size_t)(q0 + qrel) * num_q_heads + h) * D;
#pragma unroll
    for (int t = 0; t < C::DT; ++t)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const uint2 w = make_uint2(pack_bf16x2(o[t][4 * a] * inv, o[t][4 * a + 1] * inv),
                                   pack_bf16x2(o[t][4 * a + 2] * inv, o[t][4 * a + 3] * inv));
        *reinterpret_cast<uint2*>(orow + 32 * t + 8 * a + 4 * half) = w;
      }
  }
}

}  // namespace prefill_impl
}  // namespace pkv
