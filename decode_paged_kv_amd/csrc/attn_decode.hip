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
// bf16 (the measured path): the MFMA kernel of decode_bf16.h, with the
// equal-splits plan or, for batches with fewer (request, KV head) pairs
// than resident workgroups, the stream split (plans below).  A plan made
// for a launch on part of the device's CUs (the decode stream of a PD
// multiplexing level) with one split per (request, KV head) runs the
// whole-line form of decode_line.h instead.
//
// fp32 (small checks): the kernel in this file.  Inside a workgroup each
// wave walks 64-key tiles (tile i of the split goes to wave i % 4):
//   q.k   lane l owns key l of the tile and reads its K row (16-byte loads
//         of a block's contiguous rows); the G query rows are broadcast
//         from LDS; fp32 fma accumulation.
//   soft  online softmax per wave in the exp2 domain (scores pre-scaled by
//         scale*log2 e): running max m, per-lane partial sums.
//   p.v   p goes through the wave's own LDS slice; lane l owns head-dim
//         columns and reads the dim-major V tile (16 keys of one dim are
//         contiguous).
// The 4 waves' (m, l, acc) are merged in LDS.  A request whose context
// fits one split writes its output there; otherwise the split partials go
// to the workspace and a second kernel merges them.
#include <cstdlib>

#include "decode_bf16.h"
#include "decode_line.h"

namespace pkv {
namespace {

using namespace decode_impl;

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

template <int D, int G>
struct DecodeSmem {
  float q[G][D];
  float p[kWaves][G][kTile];     // p of the current tile, per wave
  float red_acc[kWaves][G][D];
  float red_m[kWaves][G];
  float red_l[kWaves][G];
};

// fp32 kernel (bf16 runs the MFMA kernel of decode_bf16.h).
template <int D, int G>
__global__ void __launch_bounds__(kThreads)
attn_decode_f32_kernel(PoolDev pool, const float* __restrict__ q, float* __restrict__ out,
                       const int32_t* __restrict__ bt, int bt_stride, const int32_t* __restrict__ ctx,
                       int num_q_heads, float scale_log2, int split_tokens, int num_splits, int max_len,
                       float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int DPL = D / 64;                  // head-dim columns per lane in p.v
  using Smem = DecodeSmem<D, G>;
  __shared__ Smem sm;

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int L = ctx[b];
  if (L > max_len) {                             // past max_context_len: cut, flagged
    if (threadIdx.x == 0 && split == 0 && kvh == 0) flag_error(pool.err, PKV_ERRBIT_CONTEXT);
    L = max_len;
  }
  const int start = split * split_tokens;
  if (start >= L) return;
  const int end = min(L, start + split_tokens);

  const int hl = pool.heads_per_shard;
  const int sh = kvh / hl, lh = kvh - sh * hl;
  const float* kpool = reinterpret_cast<const float*>(pool.k[sh]);
  const float* vpool = reinterpret_cast<const float*>(pool.v[sh]);
  const int bs = pool.block_size;
  const int32_t* table = bt + (size_t)b * bt_stride;

  // q rows of this KV head's group -> LDS
  {
    const float* qsrc = q + ((size_t)b * num_q_heads + (size_t)kvh * G) * D;
    float* qdst = &sm.q[0][0];
    for (int i = threadIdx.x; i < G * D; i += kThreads) qdst[i] = qsrc[i];
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
    const float* krow = nullptr;
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
      for (int c = 0; c < D / 4; ++c) {
        const float4 kv = *reinterpret_cast<const float4*>(krow + c * 4);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float4 qv = *reinterpret_cast<const float4*>(&sm.q[g][c * 4]);
          s[g] = fmaf(kv.x, qv.x, s[g]);
          s[g] = fmaf(kv.y, qv.y, s[g]);
          s[g] = fmaf(kv.z, qv.z, s[g]);
          s[g] = fmaf(kv.w, qv.w, s[g]);
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
      sm.p[wave][g][lane] = p;
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
      const float* vtile = vpool + tile_elems(pool, blk, lh) + (key16 & (bs - 1));
#pragma unroll
      for (int j = 0; j < DPL; ++j) {
        const int d = lane * DPL + j;
        const float* vrow = vtile + (size_t)d * bs;      // 16 keys of dim d
        float vv[16];
#pragma unroll
        for (int u = 0; u < 4; ++u) *reinterpret_cast<float4*>(&vv[4 * u]) = *reinterpret_cast<const float4*>(vrow + 4 * u);
        // keys past the context hold arbitrary bits: zero them (0 * NaN is NaN)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (e >= nvalid) vv[e] = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float a = acc[g][j];
#pragma unroll
          for (int e = 0; e < 16; ++e) a = fmaf(sm.p[wave][g][kk + e], vv[e], a);
          acc[g][j] = a;
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
      out[((size_t)b * num_q_heads + h) * D + d] = o / l;
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

template <int D, int G, bool STREAM, bool APPEND>
__global__ void __launch_bounds__(kThreads, 2)
attn_decode_bf16_kernel(PoolDev pool, const bf16_t* __restrict__ q, bf16_t* __restrict__ out,
                        const int32_t* __restrict__ bt, int bt_stride, const int32_t* __restrict__ ctx, int batch,
                        int num_q_heads, float scale_log2, int split_tokens, int num_splits, int max_len,
                        float* __restrict__ part_o, float* __restrict__ part_ml, const bf16_t* __restrict__ k_new,
                        const bf16_t* __restrict__ v_new) {
  __shared__ DecodeBf16Smem<D, G> sm;
  decode_bf16_block<D, G, STREAM, APPEND>(pool, q, out, bt, bt_stride, ctx, batch, num_q_heads, scale_log2,
                                          split_tokens, num_splits, max_len, part_o, part_ml, k_new, v_new,
                                          blockIdx.x, blockIdx.y, blockIdx.z, gridDim.x, sm);
}

// grid (1, KV heads, requests): one workgroup per (request, KV head)
template <int D, int G, bool APPEND>
__global__ void __launch_bounds__(kThreads, 2)
attn_decode_line_kernel(PoolDev pool, const bf16_t* __restrict__ q, bf16_t* __restrict__ out,
                        const int32_t* __restrict__ bt, int bt_stride, const int32_t* __restrict__ ctx,
                        int num_q_heads, float scale_log2, int max_len, const bf16_t* __restrict__ k_new,
                        const bf16_t* __restrict__ v_new) {
  __shared__ __attribute__((aligned(1024))) char ktiles[decode_line::LineKCfg<D>::REGION];
  __shared__ decode_line::LineSmem<D, G> sm;
  decode_line::decode_line_block<D, G, APPEND>(pool, q, out, bt, bt_stride, ctx, num_q_heads, scale_log2, max_len,
                                               k_new, v_new, blockIdx.y, blockIdx.z, ktiles, sm);
}

// The new token's K/V row of each (request, KV head) written at position
// L-1 of the request (the fp32 path of attn_decode_append; the bf16 kernel
// writes it itself).  One workgroup per (KV head, request), a thread per dim.
template <typename T>
__global__ void __launch_bounds__(128)
kv_append_kernel(PoolDev pool, const T* __restrict__ k_new, const T* __restrict__ v_new,
                 const int32_t* __restrict__ bt, int bt_stride, const int32_t* __restrict__ ctx, int max_len) {
  const int kvh = blockIdx.x, b = blockIdx.y, D = pool.head_dim;
  const int L = ctx[b];
  if (L <= 0) return;
  if (L > max_len) {                              // past max_context_len: nothing written, flagged
    if (threadIdx.x == 0 && kvh == 0) flag_error(pool.err, PKV_ERRBIT_CONTEXT);
    return;
  }
  const int blk = bt[(size_t)b * bt_stride + ((L - 1) >> pool.bs_shift)];
  if (blk < 0 || blk >= pool.num_blocks) {
    if (threadIdx.x == 0) flag_error(pool.err, PKV_ERRBIT_BLOCK_ID);
    return;
  }
  const int hl = pool.heads_per_shard, sh = kvh / hl, lh = kvh - sh * hl;
  const size_t tile = tile_elems(pool, blk, lh);
  const int off = (L - 1) & (pool.block_size - 1);
  const T* kn = k_new + ((size_t)b * pool.num_kv_heads + kvh) * D;
  const T* vn = v_new + ((size_t)b * pool.num_kv_heads + kvh) * D;
  T* kp = reinterpret_cast<T*>(pool.k[sh]) + tile + (size_t)off * D;
  T* vp = reinterpret_cast<T*>(pool.v[sh]) + tile + off;
  for (int d = threadIdx.x; d < D; d += 128) {
    kp[d] = kn[d];
    vp[(size_t)d * pool.block_size] = vn[d];
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
// The owners are computed over the same NW = min(grid, tiles) workgroups as
// in the attention kernel, every one of which has tiles, so each row read
// here was written by this launch (never a stale row of a reused workspace).
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
  const long long nw = min((long long)nwg, sc.total);
  const long long pstart = sc.base_rb + (long long)kvh * ntb;
  const long long wlo = stream_owner(pstart, nw, sc.total), whi = stream_owner(pstart + ntb - 1, nw, sc.total);
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
                        void* ws, hipStream_t s, const void* k_new, const void* v_new) {
  float* part_o = static_cast<float*>(ws);
  float* part_ml = part_o ? part_o + (size_t)batch * num_q_heads * plan.num_splits * D : nullptr;
  // append mode with the stream split or in fp32: the new rows are written
  // by a small kernel first (in the stream-split bf16 kernel the fused form
  // would push it past its registers)
  const bool append_first = k_new && (sizeof(T) == 4 || plan.stream_wgs > 0);
  if (append_first) {
    hipLaunchKernelGGL(kv_append_kernel<T>, dim3(pool.num_kv_heads, batch), dim3(128), 0, s, pool,
                       static_cast<const T*>(k_new), static_cast<const T*>(v_new), bt, bt_stride, ctx, plan.max_len);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if constexpr (sizeof(T) == 2) {
    if (plan.stream_wgs > 0) {
      float* ml = static_cast<float*>(ws) + (size_t)(plan.stream_wgs + batch * (num_q_heads / G)) * G * D;
      hipLaunchKernelGGL((attn_decode_bf16_kernel<D, G, true, false>), dim3(plan.stream_wgs), dim3(kThreads), 0, s,
                         pool, static_cast<const bf16_t*>(q), static_cast<bf16_t*>(out), bt, bt_stride, ctx, batch,
                         num_q_heads, scale_log2, 0, 0, plan.max_len, part_o, ml, nullptr, nullptr);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((attn_decode_stream_merge_kernel<D>), dim3(num_q_heads, batch), dim3(D), 0, s, part_o, ml,
                         ctx, static_cast<bf16_t*>(out), batch, num_q_heads, num_q_heads / G, plan.max_len,
                         plan.stream_wgs);
      return hipGetLastError();
    }
  }
  const dim3 grid(plan.num_splits, num_q_heads / G, batch);
  if constexpr (sizeof(T) == 2) {
#define PKV_SPLIT_LAUNCH(AP)                                                                                       \
    hipLaunchKernelGGL((attn_decode_bf16_kernel<D, G, false, AP>), grid, dim3(kThreads), 0, s, pool,               \
                       static_cast<const bf16_t*>(q), static_cast<bf16_t*>(out), bt, bt_stride, ctx, batch,       \
                       num_q_heads, scale_log2, plan.split_tokens, plan.num_splits, plan.max_len, part_o, part_ml, \
                       static_cast<const bf16_t*>(k_new), static_cast<const bf16_t*>(v_new))
#define PKV_LINE_LAUNCH(AP)                                                                                        \
    hipLaunchKernelGGL((attn_decode_line_kernel<D, G, AP>), grid, dim3(kThreads), 0, s, pool,                      \
                       static_cast<const bf16_t*>(q), static_cast<bf16_t*>(out), bt, bt_stride, ctx, num_q_heads, \
                       scale_log2, plan.max_len, static_cast<const bf16_t*>(k_new),                               \
                       static_cast<const bf16_t*>(v_new))
    if (plan.line_k && plan.num_splits == 1) {
      if (k_new) PKV_LINE_LAUNCH(true);
      else PKV_LINE_LAUNCH(false);
    } else {
      if (k_new) PKV_SPLIT_LAUNCH(true);
      else PKV_SPLIT_LAUNCH(false);
    }
#undef PKV_LINE_LAUNCH
#undef PKV_SPLIT_LAUNCH
  } else {
    hipLaunchKernelGGL((attn_decode_f32_kernel<D, G>), grid, dim3(kThreads), 0, s, pool, static_cast<const float*>(q),
                       static_cast<float*>(out), bt, bt_stride, ctx, num_q_heads, scale_log2, plan.split_tokens,
                       plan.num_splits, plan.max_len, part_o, part_ml);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.num_splits == 1) return e;
  hipLaunchKernelGGL((attn_decode_merge_kernel<T, D>), dim3(num_q_heads, batch), dim3(D), 0, s, part_o, part_ml,
                     ctx, static_cast<T*>(out), num_q_heads, plan.split_tokens, plan.num_splits, plan.max_len);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(int group, const PoolDev& pool, const void* q, void* out, const int32_t* bt, int bt_stride,
                    const int32_t* ctx, int batch, int num_q_heads, float scale_log2, const DecodePlan& plan,
                    void* ws, hipStream_t s, const void* k_new, const void* v_new) {
  switch (group) {
    case 1: return launch_typed<T, D, 1>(pool, q, out, bt, bt_stride, ctx, batch, num_q_heads, scale_log2, plan, ws, s, k_new, v_new);
    case 2: return launch_typed<T, D, 2>(pool, q, out, bt, bt_stride, ctx, batch, num_q_heads, scale_log2, plan, ws, s, k_new, v_new);
    case 4: return launch_typed<T, D, 4>(pool, q, out, bt, bt_stride, ctx, batch, num_q_heads, scale_log2, plan, ws, s, k_new, v_new);
    case 8: return launch_typed<T, D, 8>(pool, q, out, bt, bt_stride, ctx, batch, num_q_heads, scale_log2, plan, ws, s, k_new, v_new);
    case 16: return launch_typed<T, D, 16>(pool, q, out, bt, bt_stride, ctx, batch, num_q_heads, scale_log2, plan, ws, s, k_new, v_new);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_split_merge(const PoolDev& pool, int dtype, void* out, const int32_t* ctx, int bt_stride,
                                     int batch, int num_q_heads, const DecodePlan& plan, void* workspace,
                                     hipStream_t s) {
  if (batch == 0 || plan.stream_wgs > 0 || plan.num_splits <= 1) return hipSuccess;
  const float* part_o = static_cast<const float*>(workspace);
  const float* part_ml = part_o + (size_t)batch * num_q_heads * plan.num_splits * pool.head_dim;
#define PKV_MERGE(T, DD)                                                                                           \
  hipLaunchKernelGGL((attn_decode_merge_kernel<T, DD>), dim3(num_q_heads, batch), dim3(DD), 0, s, part_o, part_ml, \
                     ctx, static_cast<T*>(out), num_q_heads, plan.split_tokens, plan.num_splits, plan.max_len)
  if (dtype == PKV_BF16) {
    if (pool.head_dim == 128) PKV_MERGE(bf16_t, 128);
    else PKV_MERGE(bf16_t, 64);
  } else {
    if (pool.head_dim == 128) PKV_MERGE(float, 128);
    else PKV_MERGE(float, 64);
  }
#undef PKV_MERGE
  return hipGetLastError();
}

DecodePlan plan_decode(int batch, int num_q_heads, int num_kv_heads, int max_context_len, int head_dim, int dtype,
                       bool stream_ok) {
  // Two workgroups per CU (256 CUs) already keep enough loads in flight to
  // saturate HBM, so a batch with that many (request, KV head) pairs runs
  // one split per pair and needs no merge.  Below that a pair is cut into
  // splits of at most 512 keys (short workgroups balance uneven contexts as
  // they finish), shorter still until there are about three workgroups per
  // CU (more than are resident at once at head dim 128, so short and long
  // splits even out), but no shorter than 128 keys.  Splits
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
  p.max_len = max_context_len;
  p.split_tokens = (int)split;
  p.num_splits = (int)((max_context_len + split - 1) / split);
  p.stream_wgs = 0;
  p.line_k = false;
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
  if (stream_ok && dtype == PKV_BF16 && pairs < 512 && p.num_splits > 1 && !forced) {
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
                              const DecodePlan& plan, void* workspace, hipStream_t s, const void* k_new,
                              const void* v_new) {
  if (batch == 0) return hipSuccess;
  const int group = num_q_heads / pool.num_kv_heads;
  const float sl2 = scale * kLog2e;
  if (dtype == PKV_BF16) {
    if (pool.head_dim == 128) return launch_d<bf16_t, 128>(group, pool, q, out, bt, bt_stride, ctx, batch, num_q_heads, sl2, plan, workspace, s, k_new, v_new);
    return launch_d<bf16_t, 64>(group, pool, q, out, bt, bt_stride, ctx, batch, num_q_heads, sl2, plan, workspace, s, k_new, v_new);
  }
  if (pool.head_dim == 128) return launch_d<float, 128>(group, pool, q, out, bt, bt_stride, ctx, batch, num_q_heads, sl2, plan, workspace, s, k_new, v_new);
  return launch_d<float, 64>(group, pool, q, out, bt, bt_stride, ctx, batch, num_q_heads, sl2, plan, workspace, s, k_new, v_new);
}

}  // namespace pkv
