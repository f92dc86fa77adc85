// Paged causal GQA prefill attention for one chunk per request.
//
// Pages: "Lecture 7 · Prefill 与 Decode" section 2.3 (a chunk's queries see
// every earlier chunk plus the causal part of their own chunk, so chunked
// prefill equals one-shot prefill; the cost is re-reading earlier KV, and
// prefill attention stays compute-bound); "PD multiplexing: splitting
// prefill and decode by SM on one GPU" section "Is it worth it: an
// estimate" (the attention flop count 4*Hq*D*(T*S + T^2/2) per layer).
//
// bf16 path (the dense contraction, on MFMA):
//   One workgroup = 128 query rows of one q-head (4 waves x 32 rows).  It
//   walks 64-key tiles of the request's KV through the block table; each
//   tile's K rows and dim-major V rows are staged in LDS (padded rows, no
//   bank conflicts on 16-byte reads) with the next tile's global loads in
//   flight while the current tile is computed.
//   Both products run transposed on v_mfma_f32_32x32x16_bf16 so that one
//   lane ends up owning one query:
//     S^T = K Q^T   (A = K rows from LDS, B = the wave's Q held in VGPRs)
//     O^T += V^T P^T (A = dim-major V rows from LDS, B = P from registers)
//   With the C layout of the 32x32 MFMA, lane l holds 16 keys of query
//   l%32 per 32-key half tile, so the softmax max/sum need one cross-lane
//   step (lanes l and l^32).  The K rows fed to the first MFMA are
//   permuted so that the 8 consecutive accumulator registers a lane
//   converts to bf16 are 8 consecutive keys; the second MFMA's A operand
//   then reads those same 8 keys as one 16-byte run of the dim-major V
//   tile.  The permutation is applied when K rows are written to LDS, so
//   the MFMA reads consecutive LDS rows (bank-conflict free with the
//   16-byte row padding).  Online softmax in the exp2 domain, fp32 accumulation.
//   Work items are ordered (KV head, query tile from the heaviest, q-head
//   in the group) and dealt out so that each XCD (consecutive workgroup ids
//   go round-robin over the 8 XCDs) gets one contiguous run: the q-heads of
//   one KV head then stream the same K/V through the same L2.
//
// fp32 path: a plain wave-per-(query, head) kernel for small checks.
#include <algorithm>

#include "prefill_bf16.h"

namespace pkv {
namespace {

using namespace prefill_impl;

template <int D, int NG>
__global__ void __launch_bounds__(256 * NG, 2 / NG)
attn_prefill_bf16_kernel(PoolDev pool, const bf16_t* __restrict__ q, bf16_t* __restrict__ out,
                         const int32_t* __restrict__ bt, int bt_stride, const int32_t* __restrict__ start_loc,
                         const int32_t* __restrict__ chunk_start, int batch, int ntiles, int num_q_heads,
                         int group, float scale_log2, int total_items, int max_total) {
  __shared__ __attribute__((aligned(1024))) PrefillTiles<D, NG> kb0, kb1, vb0, vb1;
  prefill_bf16_block<D, NG>(pool, q, out, bt, bt_stride, start_loc, chunk_start, batch, ntiles, num_q_heads, group,
                            scale_log2, total_items, max_total, blockIdx.x, gridDim.x, kb0, kb1, vb0, vb1);
}

// fp32: one wave per (query row, q-head); lane owns head-dim columns.
template <int D>
__global__ void __launch_bounds__(256)
attn_prefill_f32_kernel(PoolDev pool, const float* __restrict__ q, float* __restrict__ out,
                        const int32_t* __restrict__ bt, int bt_stride, const int32_t* __restrict__ start_loc,
                        const int32_t* __restrict__ chunk_start, int max_chunk_len, int num_q_heads, int group,
                        float scale_log2, int max_total) {
  constexpr int DPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);     // query row within the chunk
  const int h = blockIdx.y, b = blockIdx.z;
  const int q0 = start_loc[b];
  const int T = start_loc[b + 1] - q0;
  if (row >= T || row >= max_chunk_len) return;
  const int S = chunk_start[b];
  const int pos = S + row;
  // keys [0, pos], cut to max_total_len (checked against the table's
  // capacity on the host) and flagged if the chunk reaches past it
  if (row == 0 && lane == 0 && S + T > max_total) flag_error(pool.err, PKV_ERRBIT_CONTEXT);
  const int kend = min(pos + 1, max_total);
  const int kvh = h / group;
  const int hl = pool.heads_per_shard;
  const int sh = kvh / hl, lh = kvh - sh * hl;
  const float* kpool = reinterpret_cast<const float*>(pool.k[sh]);
  const float* vpool = reinterpret_cast<const float*>(pool.v[sh]);
  const int bs = pool.block_size;
  const int32_t* table = bt + (size_t)b * bt_stride;
  float qv[DPL], acc[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) {
    qv[j] = q[((size_t)(q0 + row) * num_q_heads + h) * D + lane * DPL + j];
    acc[j] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int key = 0; key < kend; ++key) {
    const int blk = table[key >> pool.bs_shift];
    if (blk < 0 || blk >= pool.num_blocks) {
      if (lane == 0) flag_error(pool.err, PKV_ERRBIT_BLOCK_ID);
      continue;
    }
    const size_t tile = tile_elems(pool, blk, lh);
    const int off = key & (bs - 1);
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) part = fmaf(qv[j], kpool[tile + (size_t)off * D + lane * DPL + j], part);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o);
    const float s = part * scale_log2;
    const float mn = fmaxf(m, s);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    const float p = __builtin_amdgcn_exp2f(s - mn);
    l = l * alpha + p;
#pragma unroll
    for (int j = 0; j < DPL; ++j) acc[j] = fmaf(p, vpool[tile + (size_t)(lane * DPL + j) * bs + off], acc[j] * alpha);
    m = mn;
  }
#pragma unroll
  for (int j = 0; j < DPL; ++j) out[((size_t)(q0 + row) * num_q_heads + h) * D + lane * DPL + j] = acc[j] / l;
}

}  // namespace

hipError_t launch_attn_prefill(const PoolDev& pool, int dtype, const void* q, void* out, const int32_t* bt,
                               int bt_stride, const int32_t* start_loc, const int32_t* chunk_start, int batch,
                               int max_chunk_len, int max_total_len, int num_q_heads, float scale, hipStream_t s) {
  if (batch == 0 || max_chunk_len == 0) return hipSuccess;
  // never past what the table addresses (the ABI has checked max_total_len
  // against it already)
  const int max_total = (int)std::min<long long>(max_total_len, (long long)bt_stride << pool.bs_shift);
  const int group = num_q_heads / pool.num_kv_heads;
  const float sl2 = scale * kLog2e;
  if (dtype == PKV_BF16) {
    constexpr int BM = 128;
    const int ntiles = (max_chunk_len + BM - 1) / BM;
    const int items = pool.num_kv_heads * ntiles * group * batch;
    const int grid = (items + kXcds - 1) / kXcds * kXcds;
    // fewer than two 4-wave workgroups per CU (256 CUs): split each
    // workgroup's key tiles over two groups of 4 waves instead
    const bool split = items < 512;
#define PKV_PREFILL_LAUNCH(DD, NG)                                                                               \
    hipLaunchKernelGGL((attn_prefill_bf16_kernel<DD, NG>), dim3(grid), dim3(256 * NG), 0, s, pool,                \
                       static_cast<const bf16_t*>(q), static_cast<bf16_t*>(out), bt, bt_stride, start_loc,       \
                       chunk_start, batch, ntiles, num_q_heads, group, sl2, items, max_total)
    if (pool.head_dim == 128) {
      if (split) PKV_PREFILL_LAUNCH(128, 2);
      else PKV_PREFILL_LAUNCH(128, 1);
    } else {
      if (split) PKV_PREFILL_LAUNCH(64, 2);
      else PKV_PREFILL_LAUNCH(64, 1);
    }
#undef PKV_PREFILL_LAUNCH
    return hipGetLastError();
  }
  const dim3 grid((max_chunk_len + 3) / 4, num_q_heads, batch);
  if (pool.head_dim == 128)
    hipLaunchKernelGGL(attn_prefill_f32_kernel<128>, grid, dim3(256), 0, s, pool, static_cast<const float*>(q),
                       static_cast<float*>(out), bt, bt_stride, start_loc, chunk_start, max_chunk_len, num_q_heads,
                       group, sl2, max_total);
  else
    hipLaunchKernelGGL(attn_prefill_f32_kernel<64>, grid, dim3(256), 0, s, pool, static_cast<const float*>(q),
                       static_cast<float*>(out), bt, bt_stride, start_loc, chunk_start, max_chunk_len, num_q_heads,
                       group, sl2, max_total);
  return hipGetLastError();
}

}  // namespace pkv
