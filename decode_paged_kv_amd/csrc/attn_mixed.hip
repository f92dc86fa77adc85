// Stall-free mixed batch: the decode attention of every decoding request
// and the prefill attention of a chunk, one layer, in a single launch.
//
// Pages: "Lecture 7 · Prefill 与 Decode" section 2.4 (a batch takes every
// decoding request first, one token each, then prefill chunks that use only
// what is left of a per-step token budget, so decode never stalls and the
// decode step's idle compute is filled with prefill work) and section 2.3
// (a chunk attends to everything before it plus the causal part of itself).
//
// One grid holds both kinds of workgroup, so on the whole device the
// bandwidth-bound decode work runs beside the matrix-core-bound prefill work
// instead of after it.  Decode first is the rule for what enters the batch;
// inside the launch the step ends when its last workgroup does, so the
// prefill workgroups (the long ones: a query tile walks every earlier key)
// take the low block ids and are dispatched first, and the decode
// workgroups fill the compute units around them.  Each workgroup runs the
// same per-workgroup code as the separate decode and prefill kernels
// (equal-splits decode plan; prefill with one key-tile group), so results
// are those of the two kernels.  The prefill block count is a multiple of
// the XCD count, so the prefill blocks keep their XCD mapping.
#include <algorithm>

#include "decode_bf16.h"
#include "prefill_bf16.h"

namespace pkv {
namespace {

// A workgroup is either kind, so the two kinds' LDS share one allocation
// (their sum would leave room for only one workgroup per CU at G >= 8).
template <int D, int G>
union MixedSmem {
  prefill_impl::PrefillSmem<D, 1> prefill;
  decode_impl::DecodeBf16Smem<D, G> decode;
};

template <int D, int G>
__global__ void __launch_bounds__(256, 2)
attn_mixed_bf16_kernel(PoolDev pool,
                       // decode part: equal splits, blocks (split, KV head, request) flattened split-fastest,
                       // after the prefill blocks
                       const bf16_t* __restrict__ dq, bf16_t* __restrict__ dout, const int32_t* __restrict__ dbt,
                       int dbt_stride, const int32_t* __restrict__ ctx, int dbatch, int split_tokens,
                       int num_splits, int max_len, float* __restrict__ part_o, float* __restrict__ part_ml,
                       int dec_blocks,
                       // prefill part
                       const bf16_t* __restrict__ pq, bf16_t* __restrict__ pout, const int32_t* __restrict__ pbt,
                       int pbt_stride, const int32_t* __restrict__ start_loc, const int32_t* __restrict__ chunk_start,
                       int pbatch, int ntiles, int pf_items, int pf_blocks, int pf_max_total, int num_q_heads,
                       float scale_log2) {
  __shared__ MixedSmem<D, G> sm;
  if ((int)blockIdx.x < pf_blocks) {
    prefill_impl::prefill_bf16_block<D, 1>(pool, pq, pout, pbt, pbt_stride, start_loc, chunk_start, pbatch, ntiles,
                                           num_q_heads, G, scale_log2, pf_items, pf_max_total, blockIdx.x,
                                           pf_blocks, sm.prefill.kb0, sm.prefill.kb1, sm.prefill.vb0,
                                           sm.prefill.vb1);
  } else {
    const int bid = blockIdx.x - pf_blocks;
    const int hkv = num_q_heads / G;
    const int per_b = num_splits * hkv;
    const int b = bid / per_b;
    const int rem = bid - b * per_b;
    const int kvh = rem / num_splits, split = rem - kvh * num_splits;
    decode_impl::decode_bf16_block<D, G, false>(pool, dq, dout, dbt, dbt_stride, ctx, dbatch, num_q_heads,
                                                scale_log2, split_tokens, num_splits, max_len, part_o, part_ml, nullptr,
                                                nullptr, split, kvh, b, 0, sm.decode);
  }
}

constexpr int kXcdCount = 8;
constexpr float kLog2eMixed = 1.4426950408889634f;

template <int D, int G>
hipError_t launch_mixed_dg(const PoolDev& pool, const MixedDecode& d, const MixedPrefill& p, int num_q_heads,
                           float scale, hipStream_t s) {
  const int hkv = num_q_heads / G;
  const int dec_blocks = d.batch > 0 ? d.plan.num_splits * hkv * d.batch : 0;
  constexpr int BM = 128;
  const int ntiles = p.batch > 0 && p.max_chunk_len > 0 ? (p.max_chunk_len + BM - 1) / BM : 0;
  const int pf_items = hkv * ntiles * G * p.batch;
  const int pf_blocks = (pf_items + kXcdCount - 1) / kXcdCount * kXcdCount;
  const int pf_max_total =
      p.batch > 0 ? (int)std::min<long long>(p.max_total_len, (long long)p.bt_stride << pool.bs_shift) : 0;
  if (dec_blocks + pf_blocks == 0) return hipSuccess;
  float* part_o = static_cast<float*>(d.workspace);
  float* part_ml = part_o ? part_o + (size_t)d.batch * num_q_heads * d.plan.num_splits * D : nullptr;
  hipLaunchKernelGGL((attn_mixed_bf16_kernel<D, G>), dim3(dec_blocks + pf_blocks), dim3(256), 0, s, pool,
                     static_cast<const bf16_t*>(d.q), static_cast<bf16_t*>(d.out), d.bt, d.bt_stride, d.ctx, d.batch,
                     d.plan.split_tokens, d.plan.num_splits, d.plan.max_len, part_o, part_ml, dec_blocks,
                     static_cast<const bf16_t*>(p.q), static_cast<bf16_t*>(p.out), p.bt, p.bt_stride, p.start_loc,
                     p.chunk_start, p.batch, ntiles, pf_items, pf_blocks, pf_max_total, num_q_heads,
                     scale * kLog2eMixed);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_split_merge(pool, PKV_BF16, d.out, d.ctx, d.bt_stride, d.batch, num_q_heads, d.plan,
                                   d.workspace, s);
}

template <int D>
hipError_t launch_mixed_d(int group, const PoolDev& pool, const MixedDecode& d, const MixedPrefill& p,
                          int num_q_heads, float scale, hipStream_t s) {
  switch (group) {
    case 1: return launch_mixed_dg<D, 1>(pool, d, p, num_q_heads, scale, s);
    case 2: return launch_mixed_dg<D, 2>(pool, d, p, num_q_heads, scale, s);
    case 4: return launch_mixed_dg<D, 4>(pool, d, p, num_q_heads, scale, s);
    case 8: return launch_mixed_dg<D, 8>(pool, d, p, num_q_heads, scale, s);
    case 16: return launch_mixed_dg<D, 16>(pool, d, p, num_q_heads, scale, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_mixed(const PoolDev& pool, int dtype, const MixedDecode& d, const MixedPrefill& p,
                             int num_q_heads, float scale, hipStream_t s) {
  if (dtype != PKV_BF16) {
    // fp32 (checks only): the two kernels back to back, decode first
    hipError_t e = launch_attn_decode(pool, dtype, d.q, d.out, d.bt, d.bt_stride, d.ctx, d.batch, num_q_heads, scale,
                                      d.plan, d.workspace, s);
    if (e != hipSuccess) return e;
    return launch_attn_prefill(pool, dtype, p.q, p.out, p.bt, p.bt_stride, p.start_loc, p.chunk_start, p.batch,
                               p.max_chunk_len, p.max_total_len, num_q_heads, scale, s);
  }
  const int group = num_q_heads / pool.num_kv_heads;
  if (pool.head_dim == 128) return launch_mixed_d<128>(group, pool, d, p, num_q_heads, scale, s);
  return launch_mixed_d<64>(group, pool, d, p, num_q_heads, scale, s);
}

}  // namespace pkv
