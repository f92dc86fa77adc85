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
// split to wave i % 4).  A tile is two 16-key groups, each inside one block,
// so a group's block id is wave-uniform: it is read with a scalar load and
// the group's (block, head) K and V tiles are addressed through buffer
// descriptors in scalar registers; a lane adds only a fixed offset.  Every
// load instruction reads 1 KB of consecutive bytes:
//   K     one instruction takes 64 lanes x 16 B = 1024/(2D) whole rows of
//         the block's contiguous K rows.  The rows go to the wave's LDS
//         slice (rows padded by 16 B so the row-per-lane reads below hit
//         distinct banks).
//   q.k   lanes l and l+32 own key l%32, each half of the head dim; the
//         wave's q rows are broadcast from LDS (two addresses per read);
//         partial dots of the two halves meet through v_permlane32_swap.
//   soft  per-tile max over the 32 keys with DPP row steps and one
//         v_permlane16_swap; exp2 domain; p stored to LDS as bf16 pairs.
//   V     the dim-major V tile gives 16 keys of one dim as 32 contiguous
//         bytes; two lanes split those, one instruction covers 32 dims
//         (1 KB).  p.v multiplies bf16 key pairs with v_dot2.
// Loads run one tile ahead: the next tile's K is issued as soon as this
// tile's K sits in LDS, its V as soon as this tile's p.v has consumed the
// V registers, so HBM latency overlaps the arithmetic.
// A request whose context fits one split writes its output directly;
// otherwise each split writes its partial (m, l, acc) and the merge kernel
// combines them (a device-wide handoff inside the kernel would need L2
// write-back and invalidation on this multi-XCD part, costlier than a
// second launch).
// ------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// v[l] + v[l ^ 32]
__device__ __forceinline__ float sum_halves(float v) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
// max over the 32 lanes of each half-wave
__device__ __forceinline__ float max_half(float v) {
  v = fmaxf(v, dpp<0xB1>(v));     // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp<0x4E>(v));     // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp<0x141>(v));    // row_half_mirror
  v = fmaxf(v, dpp<0x140>(v));    // row_mirror
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

template <int D, int G>
struct DecodeBf16Smem {
  static constexpr int TK = 32, KROW = D + 8;
  uint32_t q[G][D / 2];                         // bf16 pairs
  union {
    struct {
      bf16_t k[kWaves][TK * KROW];              // per-wave K tile
      uint32_t p[kWaves][G][TK / 2];            // per-wave p, bf16 pairs
    } t;
    struct {
      float acc[kWaves][G][D];
      float m[kWaves][G];
      float l[kWaves][G];
    } r;
  } u;
};

template <int D, int G>
__global__ void __launch_bounds__(kThreads)
attn_decode_bf16_kernel(PoolDev pool, const bf16_t* __restrict__ q, bf16_t* __restrict__ out,
                        const int32_t* __restrict__ bt, int bt_stride, const int32_t* __restrict__ ctx,
                        int num_q_heads, float scale_log2, int split_tokens, int num_splits,
                        float* __restrict__ part_o, float* __restrict__ part_ml) {
  using Smem = DecodeBf16Smem<D, G>;
  constexpr int TK = Smem::TK, KROW = Smem::KROW;
  constexpr int LPR = D / 8;            // lanes per K row in a coalesced load
  constexpr int KPI = 64 / LPR;         // K rows per load instruction
  constexpr int KPG = 16 / KPI;         // K load instructions per 16-key group
  constexpr int HALF = D / 2;
  constexpr int DPL = D / 32;           // V dims per lane
  __shared__ Smem sm;

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int L = ctx[b];
  if (L > (bt_stride << pool.bs_shift)) {
    if (threadIdx.x == 0 && split == 0 && kvh == 0) flag_error(pool.err, PKV_ERRBIT_TABLE);
    L = bt_stride << pool.bs_shift;
  }
  const int start = split * split_tokens;
  if (start >= L) return;
  const int end = min(L, start + split_tokens);
  const int nsplit = (L + split_tokens - 1) / split_tokens;   // splits holding keys of this request
  const int hl = pool.heads_per_shard;
  const int sh = kvh / hl, lh = kvh - sh * hl;
  const bf16_t* kpool = reinterpret_cast<const bf16_t*>(pool.k[sh]);
  const bf16_t* vpool = reinterpret_cast<const bf16_t*>(pool.v[sh]);
  const int bs = pool.block_size;
  const size_t head_off = (size_t)lh * bs * D;                  // elements
  const size_t block_stride = (size_t)hl * bs * D;
  const int tile_bytes = bs * D * 2;
  const int32_t* table = bt + (size_t)b * bt_stride;

  {
    const uint32_t* qsrc = reinterpret_cast<const uint32_t*>(q + ((size_t)b * num_q_heads + (size_t)kvh * G) * D);
    uint32_t* qdst = &sm.q[0][0];
    for (int i = threadIdx.x; i < G * D / 2; i += kThreads) qdst[i] = qsrc[i];
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
  const int kk = lane & 31, hh = lane >> 5;
  bf16_t* ktile = sm.u.t.k[wave];

  // ---- loads of one tile (two 16-key groups, uniform block ids) ----
  const int k_voff = ((lane / LPR) * D + (lane % LPR) * 8) * 2;        // bytes within a group's rows
  const int v_voff = ((lane >> 1) * bs + (lane & 1) * 8) * 2;          // dim lane/2, keys (lane&1)*8
  uint4 kr[2][KPG], vr[2][DPL];
  int nblk[2];                                  // block ids of the tile in flight (-1: absent)
  auto fetch_ids = [&](int k0) {
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      const int key16 = k0 + 16 * grp;
      int blk = key16 < end ? table[key16 >> pool.bs_shift] : -1;
      blk = __builtin_amdgcn_readfirstlane(blk);
      if (key16 < end && (blk < 0 || blk >= pool.num_blocks)) {
        if (lane == 0) flag_error(pool.err, PKV_ERRBIT_BLOCK_ID);
        blk = -1;
      }
      nblk[grp] = blk;
    }
  };
  auto issue_k = [&](int k0) {
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      const bool ok = nblk[grp] >= 0;
      const buffer_rsrc_t rs = buffer_rsrc(kpool + (ok ? (size_t)nblk[grp] * block_stride + head_off : 0),
                                           ok ? tile_bytes : 0);
      const int soff = ((k0 + 16 * grp) & (bs - 1)) * D * 2;
#pragma unroll
      for (int j = 0; j < KPG; ++j) kr[grp][j] = buffer_load16(rs, k_voff + j * KPI * D * 2, soff);
    }
  };
  auto issue_v = [&](int k0) {
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      const bool ok = nblk[grp] >= 0;
      const buffer_rsrc_t rs = buffer_rsrc(vpool + (ok ? (size_t)nblk[grp] * block_stride + head_off : 0),
                                           ok ? tile_bytes : 0);
      const int soff = ((k0 + 16 * grp) & (bs - 1)) * 2;
#pragma unroll
      for (int i = 0; i < DPL; ++i) vr[grp][i] = buffer_load16(rs, v_voff, soff + i * 64 * bs);
    }
  };

  const int ntiles = (end - start + TK - 1) / TK;
  if (wave < ntiles) {
    fetch_ids(start + wave * TK);
    issue_k(start + wave * TK);
    issue_v(start + wave * TK);
  }
  for (int t = wave; t < ntiles; t += kWaves) {
    const int k0 = start + t * TK;
    const bool grp_ok[2] = {nblk[0] >= 0, nblk[1] >= 0};
    // ---- K -> LDS, then the next tile's K loads ----
#pragma unroll
    for (int grp = 0; grp < 2; ++grp)
#pragma unroll
      for (int j = 0; j < KPG; ++j)
        *reinterpret_cast<uint4*>(&ktile[(16 * grp + j * KPI + lane / LPR) * KROW + (lane % LPR) * 8]) = kr[grp][j];
    wave_lds_sync();
    const int tn = t + kWaves;
    if (tn < ntiles) {
      fetch_ids(start + tn * TK);
      issue_k(start + tn * TK);
    }
    // ---- q.k: key kk, head-dim half hh ----
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = 0.f;
    {
      // the key's half row stays in registers; q rows stream from LDS one
      // head at a time (the empty asm keeps the compiler from hoisting the
      // reads of every head at once, which would cost G*HALF/2 registers)
      uint4 kv[HALF / 8];
      const bf16_t* krow = &ktile[kk * KROW + hh * HALF];
#pragma unroll
      for (int c = 0; c < HALF / 8; ++c) kv[c] = *reinterpret_cast<const uint4*>(krow + c * 8);
      int zero = 0;     // opaque 0 tied to the previous head's score (orders the q reads)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint32_t* qrow = &sm.q[g][hh * HALF / 2] + zero;
#pragma unroll
        for (int c = 0; c < HALF / 8; ++c) {
          const uint4 qv = *reinterpret_cast<const uint4*>(qrow + c * 4);
          s[g] = dot2_bf16(kv[c].x, qv.x, s[g]);
          s[g] = dot2_bf16(kv[c].y, qv.y, s[g]);
          s[g] = dot2_bf16(kv[c].z, qv.z, s[g]);
          s[g] = dot2_bf16(kv[c].w, qv.w, s[g]);
        }
        asm volatile("v_mov_b32 %0, 0" : "=v"(zero) : "v"(s[g]));
      }
    }
    const bool valid = k0 + kk < end && grp_ok[kk >> 4];
    // ---- online softmax over the tile's 32 keys ----
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float sc = valid ? sum_halves(s[g]) * scale_log2 : -INFINITY;
      const float mn = fmaxf(m[g], max_half(sc));
      const float alpha = __builtin_amdgcn_exp2f(m[g] - mn);
      const float p = __builtin_amdgcn_exp2f(sc - mn);
      m[g] = mn;
      lsum[g] = lsum[g] * alpha + (hh == 0 ? p : 0.f);
#pragma unroll
      for (int j = 0; j < DPL; ++j) acc[g][j] *= alpha;
      const float pn = dpp<0xB1>(p);                    // the odd neighbour's p
      if ((kk & 1) == 0 && hh == (g & 1)) sm.u.t.p[wave][g][kk >> 1] = pack_bf16x2(p, pn);
    }
    wave_lds_sync();
    // ---- the request's last tile: V entries of keys past the context hold
    // arbitrary bits and must be zero (p = 0 times a NaN pattern is NaN) ----
    if (k0 + TK > end) {
#pragma unroll
      for (int grp = 0; grp < 2; ++grp) {
        const int nvalid = end - (k0 + 16 * grp) - (lane & 1) * 8;
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
          uint32_t* w = reinterpret_cast<uint32_t*>(&vr[grp][i]);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e >= nvalid) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
        }
      }
    }
    // ---- p.v: lane holds dims lane/2 + 32i of keys 16grp + (lane&1)*8 .. +8 ----
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      int zero = 0;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint4 pp = *reinterpret_cast<const uint4*>(&sm.u.t.p[wave][g][grp * 8 + (lane & 1) * 4] + zero);
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
          float a = acc[g][i];
          a = dot2_bf16(pp.x, vr[grp][i].x, a);
          a = dot2_bf16(pp.y, vr[grp][i].y, a);
          a = dot2_bf16(pp.z, vr[grp][i].z, a);
          a = dot2_bf16(pp.w, vr[grp][i].w, a);
          acc[g][i] = a;
        }
        if (g % 4 == 3) asm volatile("v_mov_b32 %0, 0" : "=v"(zero) : "v"(acc[g][0]));
      }
    }
    if (tn < ntiles) issue_v(start + tn * TK);
    wave_lds_sync();
  }

  // ---- merge the lane pairs (two key halves), then the 4 waves ----
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[g][i] += dpp<0xB1>(acc[g][i]);
  __syncthreads();              // the tile buffers are reused for the reduction below
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float l = wave_sum(lsum[g]);
    if (lane == 0) {
      sm.u.r.m[wave][g] = m[g];
      sm.u.r.l[wave][g] = l;
    }
    if ((lane & 1) == 0) {
#pragma unroll
      for (int i = 0; i < DPL; ++i) sm.u.r.acc[wave][g][lane / 2 + 32 * i] = acc[g][i];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int g = i / D, d = i - g * D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm.u.r.m[w][g]);
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(sm.u.r.m[w][g] - mx);
      l += sm.u.r.l[w][g] * f;
      o += sm.u.r.acc[w][g][d] * f;
    }
    const int h = kvh * G + g;
    if (nsplit == 1) {
      out[((size_t)b * num_q_heads + h) * D + d] = f32_to_bf16(o / l);
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

// Merge the split partials of each (request, q-head): rescale each split's
// (m, l, acc) to the common max and normalise.  Requests with one split
// were finished by the attention kernel.
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
  float mx = -INFINITY;
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, part_ml[(row0 + s) * 2]);
  float l = 0.f, o = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float f = __builtin_amdgcn_exp2f(part_ml[(row0 + s) * 2] - mx);
    l += part_ml[(row0 + s) * 2 + 1] * f;
    o += part_o[(row0 + s) * D + d] * f;
  }
  const float r = o / l;
  if constexpr (sizeof(T) == 2) out[((size_t)b * num_q_heads + h) * D + d] = f32_to_bf16(r);
  else out[((size_t)b * num_q_heads + h) * D + d] = r;
}

template <typename T, int D, int G>
hipError_t launch_typed(const PoolDev& pool, const void* q, void* out, const int32_t* bt, int bt_stride,
                        const int32_t* ctx, int batch, int num_q_heads, float scale_log2, const DecodePlan& plan,
                        void* ws, hipStream_t s) {
  float* part_o = static_cast<float*>(ws);
  float* part_ml = part_o ? part_o + (size_t)batch * num_q_heads * plan.num_splits * D : nullptr;
  const dim3 grid(plan.num_splits, num_q_heads / G, batch);
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((attn_decode_bf16_kernel<D, G>), grid, dim3(kThreads), 0, s, pool,
                       static_cast<const bf16_t*>(q), static_cast<bf16_t*>(out), bt, bt_stride, ctx, num_q_heads,
                       scale_log2, plan.split_tokens, plan.num_splits, part_o, part_ml);
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

DecodePlan plan_decode(int batch, int num_q_heads, int num_kv_heads, int max_context_len, int head_dim) {
  // About two workgroups per CU (256 CUs) keep enough loads in flight to
  // saturate HBM; below that a (request, KV head) is split into more
  // workgroups, each split at least 256 keys so its fixed cost stays small.
  // Splits are whole 32-key tiles.
  const long pairs = (long)batch * num_kv_heads;
  const long splits = pairs >= 512 ? 1 : (512 + pairs - 1) / pairs;
  long split = (max_context_len + splits - 1) / splits;
  split = split < 256 ? 256 : split;
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
  // partial (acc, m, l) per (request, q-head, split)
  p.workspace = p.num_splits > 1 ? (size_t)batch * num_q_heads * p.num_splits * (head_dim + 2) * sizeof(float) : 0;
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
