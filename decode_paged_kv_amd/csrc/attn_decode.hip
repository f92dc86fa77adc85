// Paged GQA decode attention: split-KV, wavefront-parallel, HBM-bound.
//
// Pages: "Lecture 7 · Prefill 与 Decode" section 1.1 (a decode step adds one
// token per request and reads all of its KV, so it is bound by memory
// traffic); "PD multiplexing: splitting prefill and decode by SM on one GPU"
// section "Green contexts: carving out SMs for a stream" (decode reaches
// the bandwidth limit once enough compute units issue loads at once).
//
// Work decomposition: one workgroup of 4 waves per (split, KV head,
// request).  A split covers `split_tokens` consecutive keys of the request.
// The G = Hq/Hkv q-heads of the KV head share every K/V byte the workgroup
// reads, so K and V are each read from HBM once per step.
//
// Inside a workgroup each wave walks 64-key tiles (tile i of the split goes
// to wave i % 4):
//   q.k   lane l owns key l of the tile and reads its K row (16-byte loads
//         of a block's contiguous rows); the G query rows are broadcast
//         from LDS; bf16 pairs use v_dot2_f32_bf16 with fp32 accumulation.
//   soft  online softmax per wave in the exp2 domain (scores pre-scaled by
//         scale*log2 e): running max m, per-lane partial sums.
//   p.v   p goes through the wave's own LDS slice; lane l owns head-dim
//         columns and reads the dim-major V tile (16 keys of one dim are
//         32 contiguous bytes), multiplying bf16 key pairs with v_dot2.
// The 4 waves' (m, l, acc) are merged in LDS.  A request whose context
// fits one split writes its output there; otherwise the split partials go
// to the workspace and a second kernel merges them.
#include <cstdlib>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTile = 64;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
// Orders one wave's LDS writes before its later LDS reads (no cross-wave sync).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T, int D, int G>
struct DecodeSmem {
  static constexpr int QW = (sizeof(T) == 2) ? D / 2 : D;            // q words per head
  uint32_t q[G][QW];                                                  // bf16 pairs or fp32 bits
  // p of the current tile per wave: bf16 (packed pairs) or fp32
  uint32_t p[kWaves][G][(sizeof(T) == 2) ? kTile / 2 : kTile];
  float red_acc[kWaves][G][D];
  float red_m[kWaves][G];
  float red_l[kWaves][G];
};

template <typename T, int D, int G>
__global__ void __launch_bounds__(kThreads)
attn_decode_kernel(PoolDev pool, const T* __restrict__ q, T* __restrict__ out, const int32_t* __restrict__ bt,
                   int bt_stride, const int32_t* __restrict__ ctx, int num_q_heads, float scale_log2,
                   int split_tokens, int num_splits, float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int DPL = D / 64;                  // head-dim columns per lane in p.v
  constexpr int VEC = 16 / sizeof(T);          // elements per 16-byte load
  using Smem = DecodeSmem<T, D, G>;
  __shared__ Smem sm;

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int L = ctx[b];
  if (L > (bt_stride << pool.bs_shift)) {        // never index past the request's table
    if (threadIdx.x == 0 && split == 0 && kvh == 0) flag_error(pool.err, PKV_ERRBIT_TABLE);
    L = bt_stride << pool.bs_shift;
  }
  const int start = split * split_tokens;
  if (start >= L) return;
  const int end = min(L, start + split_tokens);

  const int hl = pool.heads_per_shard;
  const int sh = kvh / hl, lh = kvh - sh * hl;
  const T* kpool = reinterpret_cast<const T*>(pool.k[sh]);
  const T* vpool = reinterpret_cast<const T*>(pool.v[sh]);
  const int bs = pool.block_size;
  const int32_t* table = bt + (size_t)b * bt_stride;

  // q rows of this KV head's group -> LDS
  {
    const uint32_t* qsrc = reinterpret_cast<const uint32_t*>(q + ((size_t)b * num_q_heads + (size_t)kvh * G) * D);
    uint32_t* qdst = &sm.q[0][0];
    for (int i = threadIdx.x; i < G * Smem::QW; i += kThreads) qdst[i] = qsrc[i];
  }
  __syncthreads();

  float m[G], lsum[G], acc[G][DPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    lsum[g] = 0.f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) acc[g][j] = 0.f;
  }

  const int ntiles = (end - start + kTile - 1) / kTile;
  for (int t = wave; t < ntiles; t += kWaves) {
    const int k0 = start + t * kTile;
    // ---- q.k: lane owns key k0 + lane ----
    const int key = k0 + lane;
    bool valid = key < end;
    const T* krow = nullptr;
    if (valid) {
      const int blk = table[key >> pool.bs_shift];
      if (blk < 0 || blk >= pool.num_blocks) {
        flag_error(pool.err, PKV_ERRBIT_BLOCK_ID);
        valid = false;
      } else {
        krow = kpool + tile_elems(pool, blk, lh) + (size_t)(key & (bs - 1)) * D;
      }
    }
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = 0.f;
    if (valid) {
#pragma unroll 4
      for (int c = 0; c < D / VEC; ++c) {
        const uint4 kv = *reinterpret_cast<const uint4*>(krow + c * VEC);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const uint4 qv = *reinterpret_cast<const uint4*>(&sm.q[g][c * 4]);
          if constexpr (kBf16) {
            s[g] = dot2_bf16(kv.x, qv.x, s[g]);
            s[g] = dot2_bf16(kv.y, qv.y, s[g]);
            s[g] = dot2_bf16(kv.z, qv.z, s[g]);
            s[g] = dot2_bf16(kv.w, qv.w, s[g]);
          } else {
            s[g] = fmaf(__uint_as_float(kv.x), __uint_as_float(qv.x), s[g]);
            s[g] = fmaf(__uint_as_float(kv.y), __uint_as_float(qv.y), s[g]);
            s[g] = fmaf(__uint_as_float(kv.z), __uint_as_float(qv.z), s[g]);
            s[g] = fmaf(__uint_as_float(kv.w), __uint_as_float(qv.w), s[g]);
          }
        }
      }
    }
    // ---- online softmax (exp2 domain) ----
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float sc = valid ? s[g] * scale_log2 : -INFINITY;
      const float mn = fmaxf(m[g], wave_max(sc));
      const float alpha = __builtin_amdgcn_exp2f(m[g] - mn);
      const float p = __builtin_amdgcn_exp2f(sc - mn);
      m[g] = mn;
      lsum[g] = lsum[g] * alpha + p;
#pragma unroll
      for (int j = 0; j < DPL; ++j) acc[g][j] *= alpha;
      if constexpr (kBf16) {
        reinterpret_cast<bf16_t*>(&sm.p[wave][g][0])[lane] = f32_to_bf16(p);
      } else {
        sm.p[wave][g][lane] = __float_as_uint(p);
      }
    }
    wave_lds_sync();
    // ---- p.v: lane owns head-dim columns lane*DPL .. +DPL ----
#pragma unroll
    for (int kk = 0; kk < kTile; kk += 16) {
      const int key16 = k0 + kk;
      if (key16 >= end) break;
      const int blk = table[key16 >> pool.bs_shift];
      if (blk < 0 || blk >= pool.num_blocks) continue;     // its keys already have p = 0
      const int nvalid = min(16, end - key16);
      const T* vtile = vpool + tile_elems(pool, blk, lh) + (key16 & (bs - 1));
#pragma unroll
      for (int j = 0; j < DPL; ++j) {
        const int d = lane * DPL + j;
        const T* vrow = vtile + (size_t)d * bs;          // 16 keys of dim d
        uint4 vv[16 / VEC];
#pragma unroll
        for (int u = 0; u < 16 / VEC; ++u) vv[u] = *reinterpret_cast<const uint4*>(vrow + u * VEC);
        uint32_t* vw = reinterpret_cast<uint32_t*>(vv);
        if (nvalid < 16) {            // keys past the context hold arbitrary bits: zero them
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            if (e >= nvalid) {
              if constexpr (kBf16) vw[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
              else vw[e] = 0u;
            }
          }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          if constexpr (kBf16) {
            const uint4 p0 = *reinterpret_cast<const uint4*>(&sm.p[wave][g][kk / 2]);
            const uint4 p1 = *reinterpret_cast<const uint4*>(&sm.p[wave][g][kk / 2 + 4]);
            float a = acc[g][j];
            a = dot2_bf16(p0.x, vw[0], a);
            a = dot2_bf16(p0.y, vw[1], a);
            a = dot2_bf16(p0.z, vw[2], a);
            a = dot2_bf16(p0.w, vw[3], a);
            a = dot2_bf16(p1.x, vw[4], a);
            a = dot2_bf16(p1.y, vw[5], a);
            a = dot2_bf16(p1.z, vw[6], a);
            a = dot2_bf16(p1.w, vw[7], a);
            acc[g][j] = a;
          } else {
            float a = acc[g][j];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const uint4 pp = *reinterpret_cast<const uint4*>(&sm.p[wave][g][kk + u * 4]);
              a = fmaf(__uint_as_float(pp.x), __uint_as_float(vw[u * 4 + 0]), a);
              a = fmaf(__uint_as_float(pp.y), __uint_as_float(vw[u * 4 + 1]), a);
              a = fmaf(__uint_as_float(pp.z), __uint_as_float(vw[u * 4 + 2]), a);
              a = fmaf(__uint_as_float(pp.w), __uint_as_float(vw[u * 4 + 3]), a);
            }
            acc[g][j] = a;
          }
        }
      }
    }
    wave_lds_sync();
  }

  // ---- merge the 4 waves ----
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float l = wave_sum(lsum[g]);
    if (lane == 0) {
      sm.red_m[wave][g] = m[g];
      sm.red_l[wave][g] = l;
    }
#pragma unroll
    for (int j = 0; j < DPL; ++j) sm.red_acc[wave][g][lane * DPL + j] = acc[g][j];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int g = i / D, d = i - g * D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm.red_m[w][g]);
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(sm.red_m[w][g] - mx);   // waves without keys: m = -inf -> 0
      l += sm.red_l[w][g] * f;
      o += sm.red_acc[w][g][d] * f;
    }
    const int h = kvh * G + g;
    if (L <= split_tokens) {                   // the request's only split: final output
      const float r = o / l;
      if constexpr (kBf16) out[((size_t)b * num_q_heads + h) * D + d] = f32_to_bf16(r);
      else out[((size_t)b * num_q_heads + h) * D + d] = r;
    } else {
      const size_t row = ((size_t)b * num_q_heads + h) * num_splits + split;
      part_o[row * D + d] = o;
      if (d == 0) {
        part_ml[row * 2 + 0] = mx;
        part_ml[row * 2 + 1] = l;
      }
    }
  }
}

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
// they are consumed: K right after S^T, V right after P V.  Three waves per
// SIMD keep about 16 KB each in flight.
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
};

// Running max update rule (log2 units): the max used for exp2 moves only
// when a tile's max exceeds it by more than this, so p <= 2^8.
constexpr float kDecodeSlack = 8.0f;

// Stream split bookkeeping.  Request b holds Hkv * ceil(L_b / 32) pair-tiles
// (L_b clamped to what its table addresses), laid out by request, then KV
// head, then key.  scan_tiles returns the total, the request holding pair-
// tile `target` (-1: none) with the index of its first pair-tile, and the
// index of request rb's first pair-tile; every lane of the wave gets the
// same values (a wave-wide prefix sum, 64 requests per pass).
struct TileScan {
  long long total;
  int b;
  long long base;
  long long base_rb;
  bool over;                                    // some context exceeds its table
};
__device__ __forceinline__ long long uniform64(long long x) {
  const int lo = __builtin_amdgcn_readfirstlane((int)(unsigned)(unsigned long long)x);
  const int hi = __builtin_amdgcn_readfirstlane((int)(unsigned)((unsigned long long)x >> 32));
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}
__device__ TileScan scan_tiles(const int32_t* __restrict__ ctx, int batch, int cap, int hkv, long long target, int rb) {
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

template <int D, int G, bool STREAM>
__global__ void __launch_bounds__(kThreads, 2)
attn_decode_bf16_kernel(PoolDev pool, const bf16_t* __restrict__ q, bf16_t* __restrict__ out,
                        const int32_t* __restrict__ bt, int bt_stride, const int32_t* __restrict__ ctx, int batch,
                        int num_q_heads, float scale_log2, int split_tokens, int num_splits,
                        float* __restrict__ part_o, float* __restrict__ part_ml) {
  static_assert(G >= 1 && G <= 16, "the q-heads of a KV head are the 16 MFMA columns");
  constexpr int KC = D / 32, DT = D / 16, TK = 32;
  __shared__ DecodeBf16Smem<D, G> sm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, j4 = lane >> 4;
  const int cap = bt_stride << pool.bs_shift;                   // keys the table can address
  const int hl = pool.heads_per_shard;
  const int bs = pool.block_size;
  const size_t block_stride = (size_t)hl * bs * D;
  const int tile_bytes = bs * D * 2;

  // keys [start, end) of request b (context L) and KV head kvh; the result
  // goes to out when final_out, else to the partial rows prow + g * pstride
  auto segment = [&](int b, int kvh, int L, int start, int end, bool final_out, size_t prow, int pstride) {
  const int sh = kvh / hl, lh = kvh - sh * hl;
  const bf16_t* kpool = reinterpret_cast<const bf16_t*>(pool.k[sh]);
  const bf16_t* vpool = reinterpret_cast<const bf16_t*>(pool.v[sh]);
  const size_t head_off = (size_t)lh * bs * D;                  // elements
  const int32_t* table = bt + (size_t)b * bt_stride;

  // q as the B operand of S^T: head l16 (zero columns past G), dims 32c + 8 j4
  uint4 qf[KC];
  {
    const bool hv = l16 < G;
    const bf16_t* qrow = q + ((size_t)b * num_q_heads + (size_t)kvh * G + (hv ? l16 : 0)) * D + 8 * j4;
#pragma unroll
    for (int c = 0; c < KC; ++c) qf[c] = hv ? *reinterpret_cast<const uint4*>(qrow + 32 * c) : make_uint4(0, 0, 0, 0);
  }

  const int k_voff = (l16 * D + 8 * j4) * 2;                    // bytes within a half's 16 K rows
  const int v_voff = (l16 * bs + 4 * j4) * 2;                   // dim l16 of a 16-dim slab, 4 keys
  // block ids of the tile at k0 (-1: past the split or out of range)
  auto fetch_ids = [&](int k0, int (&ids)[2]) {
    bool bad = false;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int key16 = k0 + 16 * h;
      const int blk = key16 < end ? table[key16 >> pool.bs_shift] : -1;
      const bool ok = blk >= 0 && blk < pool.num_blocks;
      bad |= key16 < end && !ok;
      // the id is wave-uniform; saying so keeps the descriptors built from
      // it in scalar registers
      ids[h] = __builtin_amdgcn_readfirstlane(ok ? blk : -1);
    }
    if (bad && lane == 0) flag_error(pool.err, PKV_ERRBIT_BLOCK_ID);
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
#pragma unroll
  for (int mm = 0; mm < DT; ++mm) o[mm] = f32x4_t{0.f, 0.f, 0.f, 0.f};
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

  const int ntiles = (end - start + TK - 1) / TK;
  // two tiles in flight per wave: ra holds tiles wave + 8i, rb tiles wave + 8i + 4
  DecodeTile<D> ra, rb;
  constexpr int W = kWaves;
  if (wave < ntiles) {
    fetch_ids(start + wave * TK, ra.blk);
    issue_k(start + wave * TK, ra);
    issue_v(start + wave * TK, ra);
  }
  if (wave + W < ntiles) {
    fetch_ids(start + (wave + W) * TK, rb.blk);
    issue_k(start + (wave + W) * TK, rb);
    issue_v(start + (wave + W) * TK, rb);
  }
  if (wave + 2 * W < ntiles) fetch_ids(start + (wave + 2 * W) * TK, ids_next);
  auto at = [&](int t) { return t < ntiles ? start + t * TK : -1; };
  for (int t = wave; t < ntiles; t += 2 * W) {
    process(start + t * TK, ra, at(t + 2 * W), at(t + 3 * W));
    if (t + W < ntiles) process(start + (t + W) * TK, rb, at(t + 3 * W), at(t + 4 * W));
  }

  // ---- merge the 4 waves ----
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
    const int h = kvh * G + g;
    if (final_out) {
      out[((size_t)b * num_q_heads + h) * D + d] = f32_to_bf16(acc / l);
    } else {
      const size_t row = prow + (size_t)g * pstride;
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
    // one segment: split blockIdx.x of (request blockIdx.z, KV head blockIdx.y)
    const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    int L = ctx[b];
    if (L > cap) {                              // never index past the request's table
      if (threadIdx.x == 0 && split == 0 && kvh == 0) flag_error(pool.err, PKV_ERRBIT_TABLE);
      L = cap;
    }
    const int start = split * split_tokens;
    if (start >= L) return;
    segment(b, kvh, L, start, min(L, start + split_tokens), L <= split_tokens,
            ((size_t)b * num_q_heads + (size_t)kvh * G) * num_splits + split, num_splits);
  } else {
    // stream split: workgroup w takes the pair-tiles [w W / NW, (w+1) W / NW)
    // of the W = Hkv * sum_b ceil(L_b / 32) tiles of the batch, ordered by
    // request, KV head, key; a pair met by several workgroups leaves one
    // partial per workgroup, in row (w + pair index) * G + g
    const int hkv = num_q_heads / G;
    const long long NW = gridDim.x, w = blockIdx.x;
    const TileScan tot = scan_tiles(ctx, batch, cap, hkv, -1, 0);
    if (tot.over && w == 0 && threadIdx.x == 0) flag_error(pool.err, PKV_ERRBIT_TABLE);
    const long long W = tot.total;
    long long t = w * W / NW;
    const long long t1 = (w + 1) * W / NW;
    if (t >= t1) return;
    const TileScan at = scan_tiles(ctx, batch, cap, hkv, t, 0);
    int b = at.b;
    long long base = at.base;
    while (t < t1) {
      const int L = min(ctx[b], cap);
      const int ntb = (L + TK - 1) / TK;
      if (ntb == 0) {                           // an empty request holds no tiles
        ++b;
        continue;
      }
      const int kvh = (int)((t - base) / ntb);
      const long long pstart = base + (long long)kvh * ntb;
      const long long seg_end = min(t1, pstart + ntb);
      const bool final_out = stream_owner(pstart, NW, W) == stream_owner(pstart + ntb - 1, NW, W);
      segment(b, kvh, L, (int)(t - pstart) * TK, min(L, (int)(seg_end - pstart) * TK), final_out,
              (size_t)(w + (long long)b * hkv + kvh) * G, 1);
      t = seg_end;
      if (t == base + (long long)hkv * ntb) {
        base = t;
        ++b;
      }
    }
  }
}

// Merge the split partials of each (request, q-head): rescale each split's
// (m, l, acc) to the common max and normalise, in one pass with a running
// max (the loads of four splits at a time are in flight together).
// Requests with one split were finished by the attention kernel.
template <typename T, int D>
__global__ void __launch_bounds__(D)
attn_decode_merge_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                         const int32_t* __restrict__ ctx, T* __restrict__ out, int num_q_heads, int split_tokens,
                         int num_splits, int max_len) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int L = min(ctx[b], max_len);
  const int ns = min(num_splits, (L + split_tokens - 1) / split_tokens);
  if (ns <= 1) return;                         // written by the attention kernel itself
  const size_t row0 = ((size_t)b * num_q_heads + h) * num_splits;
  const float2* ml = reinterpret_cast<const float2*>(part_ml) + row0;
  float mx = -INFINITY, l = 0.f, o = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 4) {
    float2 v[4];
    float a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool in = s0 + j < ns;
      v[j] = in ? ml[s0 + j] : make_float2(-INFINITY, 0.f);
      a[j] = in ? part_o[(row0 + s0 + j) * D + d] : 0.f;
    }
    float mn = mx;
#pragma unroll
    for (int j = 0; j < 4; ++j) mn = fmaxf(mn, v[j].x);
    const float f = __builtin_amdgcn_exp2f(mx - mn);    // 0 on the first pass
    l *= f;
    o *= f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e = __builtin_amdgcn_exp2f(v[j].x - mn);   // 0 for the padding entries
      l += v[j].y * e;
      o += a[j] * e;
    }
    mx = mn;
  }
  const float r = o / l;
  if constexpr (sizeof(T) == 2) out[((size_t)b * num_q_heads + h) * D + d] = f32_to_bf16(r);
  else out[((size_t)b * num_q_heads + h) * D + d] = r;
}

// Merge of the stream split: pair (b, h / G) has one partial per workgroup
// that met it, rows (w + pair index) * G + g for w in [owner of its first
// tile, owner of its last]; a pair met by one workgroup is already final.
template <int D>
__global__ void __launch_bounds__(D)
attn_decode_stream_merge_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                const int32_t* __restrict__ ctx, bf16_t* __restrict__ out, int batch,
                                int num_q_heads, int hkv, int cap, int nwg) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int G = num_q_heads / hkv, kvh = h / G, g = h - kvh * G;
  const TileScan sc = scan_tiles(ctx, batch, cap, hkv, -1, b);
  const int L = min(ctx[b], cap);
  const int ntb = (max(L, 0) + 31) >> 5;
  if (ntb == 0) return;
  const long long pstart = sc.base_rb + (long long)kvh * ntb;
  const long long wlo = stream_owner(pstart, nwg, sc.total), whi = stream_owner(pstart + ntb - 1, nwg, sc.total);
  if (wlo == whi) return;
  const size_t row0 = (size_t)(wlo + (long long)b * hkv + kvh) * G + g;
  const int ns = (int)(whi - wlo + 1);
  float mx = -INFINITY, l = 0.f, o = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 4) {
    float2 v[4];
    float a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool in = s0 + j < ns;
      const size_t row = row0 + (size_t)(s0 + j) * G;
      v[j] = in ? reinterpret_cast<const float2*>(part_ml)[row] : make_float2(-INFINITY, 0.f);
      a[j] = in ? part_o[row * D + d] : 0.f;
    }
    float mn = mx;
#pragma unroll
    for (int j = 0; j < 4; ++j) mn = fmaxf(mn, v[j].x);
    const float f = __builtin_amdgcn_exp2f(mx - mn);    // 0 on the first pass
    l *= f;
    o *= f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e = __builtin_amdgcn_exp2f(v[j].x - mn);   // 0 for the padding entries
      l += v[j].y * e;
      o += a[j] * e;
    }
    mx = mn;
  }
  out[((size_t)b * num_q_heads + h) * D + d] = f32_to_bf16(o / l);
}

template <typename T, int D, int G>
hipError_t launch_typed(const PoolDev& pool, const void* q, void* out, const int32_t* bt, int bt_stride,
                        const int32_t* ctx, int batch, int num_q_heads, float scale_log2, const DecodePlan& plan,
                        void* ws, hipStream_t s) {
  float* part_o = static_cast<float*>(ws);
  float* part_ml = part_o ? part_o + (size_t)batch * num_q_heads * plan.num_splits * D : nullptr;
  if constexpr (sizeof(T) == 2) {
    if (plan.stream_wgs > 0) {
      float* ml = static_cast<float*>(ws) + (size_t)(plan.stream_wgs + batch * (num_q_heads / G)) * G * D;
      hipLaunchKernelGGL((attn_decode_bf16_kernel<D, G, true>), dim3(plan.stream_wgs), dim3(kThreads), 0, s, pool,
                         static_cast<const bf16_t*>(q), static_cast<bf16_t*>(out), bt, bt_stride, ctx, batch,
                         num_q_heads, scale_log2, 0, 0, part_o, ml);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((attn_decode_stream_merge_kernel<D>), dim3(num_q_heads, batch), dim3(D), 0, s, part_o, ml,
                         ctx, static_cast<bf16_t*>(out), batch, num_q_heads, num_q_heads / G,
                         bt_stride << pool.bs_shift, plan.stream_wgs);
      return hipGetLastError();
    }
  }
  const dim3 grid(plan.num_splits, num_q_heads / G, batch);
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((attn_decode_bf16_kernel<D, G, false>), grid, dim3(kThreads), 0, s, pool,
                       static_cast<const bf16_t*>(q), static_cast<bf16_t*>(out), bt, bt_stride, ctx, batch,
                       num_q_heads, scale_log2, plan.split_tokens, plan.num_splits, part_o, part_ml);
  else
    hipLaunchKernelGGL((attn_decode_kernel<T, D, G>), grid, dim3(kThreads), 0, s, pool, static_cast<const T*>(q),
                       static_cast<T*>(out), bt, bt_stride, ctx, num_q_heads, scale_log2, plan.split_tokens,
                       plan.num_splits, part_o, part_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.num_splits == 1) return e;
  hipLaunchKernelGGL((attn_decode_merge_kernel<T, D>), dim3(num_q_heads, batch), dim3(D), 0, s, part_o, part_ml,
                     ctx, static_cast<T*>(out), num_q_heads, plan.split_tokens, plan.num_splits,
                     bt_stride << pool.bs_shift);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(int group, const PoolDev& pool, const void* q, void* out, const int32_t* bt, int bt_stride,
                    const int32_t* ctx, int batch, int num_q_heads, float scale_log2, const DecodePlan& plan,
                    void* ws, hipStream_t s) {
  switch (group) {
    case 1: return launch_typed<T, D, 1>(pool, q, out, bt, bt_stride, ctx, batch, num_q_heads, scale_log2, plan, ws, s);
    case 2: return launch_typed<T, D, 2>(pool, q, out, bt, bt_stride, ctx, batch, num_q_heads, scale_log2, plan, ws, s);
    case 4: return launch_typed<T, D, 4>(pool, q, out, bt, bt_stride, ctx, batch, num_q_heads, scale_log2, plan, ws, s);
    case 8: return launch_typed<T, D, 8>(pool, q, out, bt, bt_stride, ctx, batch, num_q_heads, scale_log2, plan, ws, s);
    case 16: return launch_typed<T, D, 16>(pool, q, out, bt, bt_stride, ctx, batch, num_q_heads, scale_log2, plan, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

DecodePlan plan_decode(int batch, int num_q_heads, int num_kv_heads, int max_context_len, int head_dim, int dtype) {
  // Two workgroups per CU (256 CUs) already keep enough loads in flight to
  // saturate HBM, so a batch with that many (request, KV head) pairs runs
  // one split per pair and needs no merge.  Below that a pair is cut into
  // splits of at most 512 keys (short workgroups balance uneven contexts as
  // they finish), shorter still until there are about three workgroups per
  // CU (the bf16 kernel's occupancy), but no shorter than 128 keys.  Splits
  // are whole 32-key tiles.
  const long pairs = (long)batch * num_kv_heads;
  long split = max_context_len;
  if (pairs < 512) {
    split = ((long)max_context_len * pairs + 767) / 768;
    split = split < 128 ? 128 : (split > 512 ? 512 : split);
  }
  split = (split + 31) / 32 * 32;
  // tuning override (keys per split, a multiple of 32)
  static const int forced = [] {
    const char* e = getenv("PKV_DECODE_SPLIT_TOKENS");
    const int v = e ? atoi(e) : 0;
    return (v >= 32 && v % 32 == 0) ? v : 0;
  }();
  if (forced) split = forced;
  DecodePlan p;
  p.split_tokens = (int)split;
  p.num_splits = (int)((max_context_len + split - 1) / split);
  p.stream_wgs = 0;
  // partial (acc, m, l) per (request, q-head, split)
  p.workspace = p.num_splits > 1 ? (size_t)batch * num_q_heads * p.num_splits * (head_dim + 2) * sizeof(float) : 0;
  // bf16 with fewer pairs than resident workgroups and contexts long
  // enough to need splits: the stream split instead (one resident round of
  // two workgroups per CU, each taking an equal run of 32-key tiles, so
  // uneven contexts cost no idle tail; partial rows (workgroups + pairs) * G)
  static const int stream_wgs = [] {
    const char* e = getenv("PKV_DECODE_STREAM_WGS");
    const int v = e ? atoi(e) : 0;
    return v > 0 ? v : 512;
  }();
  if (dtype == PKV_BF16 && pairs < 512 && p.num_splits > 1 && !forced) {
    const long tiles = pairs * (((long)max_context_len + 31) / 32);
    p.stream_wgs = (int)(tiles < stream_wgs ? tiles : stream_wgs);
    p.split_tokens = 0;
    p.num_splits = 0;
    p.workspace = (size_t)(p.stream_wgs + pairs) * (num_q_heads / num_kv_heads) * (head_dim + 2) * sizeof(float);
  }
  return p;
}

hipError_t launch_attn_decode(const PoolDev& pool, int dtype, const void* q, void* out, const int32_t* bt,
                              int bt_stride, const int32_t* ctx, int batch, int num_q_heads, float scale,
                              const DecodePlan& plan, void* workspace, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  const int group = num_q_heads / pool.num_kv_heads;
  const float sl2 = scale * kLog2e;
  if (dtype == PKV_BF16) {
    if (pool.head_dim == 128) return launch_d<bf16_t, 128>(group, pool, q, out, bt, bt_stride, ctx, batch, num_q_heads, sl2, plan, workspace, s);
    return launch_d<bf16_t, 64>(group, pool, q, out, bt, bt_stride, ctx, batch, num_q_heads, sl2, plan, workspace, s);
  }
  if (pool.head_dim == 128) return launch_d<float, 128>(group, pool, q, out, bt, bt_stride, ctx, batch, num_q_heads, sl2, plan, workspace, s);
  return launch_d<float, 64>(group, pool, q, out, bt, bt_stride, ctx, batch, num_q_heads, sl2, plan, workspace, s);
}

}  // namespace pkv
