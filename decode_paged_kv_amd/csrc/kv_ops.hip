// Slot mapping, KV write and KV relayout kernels (bit copies, HBM-bound).
//
// Pages: "PD 分离与 KV 传输" (PD disaggregation and KV transfer), sections
// "实现" (slots built from the block table, per-layer write and gather) and
// "布局转换" (block size and TP head-split conversion on the GPU).
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- slots ----
__global__ void __launch_bounds__(kThreads)
slot_mapping_kernel(const int32_t* __restrict__ bt, int bt_stride, const int32_t* __restrict__ start_loc,
                    const int32_t* __restrict__ pos_start, int batch, int num_tokens, int block_size,
                    int num_blocks, int32_t* __restrict__ slots, int32_t* err) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= num_tokens) return;
  // request b with start_loc[b] <= i < start_loc[b+1] (binary search)
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (start_loc[mid] <= i) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int pos = pos_start[b] + (i - start_loc[b]);
  const int idx = pos / block_size;
  if (pos < 0 || idx >= bt_stride) {
    slots[i] = -1;
    flag_error(err, PKV_ERRBIT_TABLE);
    return;
  }
  const int blk = bt[(size_t)b * bt_stride + idx];
  if (blk < 0 || blk >= num_blocks) {
    slots[i] = -1;
    flag_error(err, PKV_ERRBIT_BLOCK_ID);
    return;
  }
  slots[i] = blk * block_size + (pos - idx * block_size);
}

// ---------------------------------------------------------------- write ----
// blockIdx.y == 0: K rows, one 16-byte vector per thread, rows contiguous on
// both sides.  blockIdx.y == 1: V, whose pool tile is dim-major, so a thread
// takes one 16-byte vector of one token's row and scatters its elements
// down the block's dim rows; consecutive threads take consecutive tokens so
// that each scattered store lands next to its neighbour's.
template <typename T>
__global__ void __launch_bounds__(kThreads)
kv_write_kernel(PoolDev pool, const T* __restrict__ k, const T* __restrict__ v,
                const int32_t* __restrict__ slots, int n_tokens) {
  constexpr int VEC = 16 / sizeof(T);
  const int H = pool.num_kv_heads, D = pool.head_dim;
  const int cpr = D / VEC;                        // vectors per row
  const size_t total = (size_t)n_tokens * H * cpr;
  const size_t cap = (size_t)pool.num_blocks << pool.bs_shift;
  const int hl = pool.heads_per_shard;
  for (size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x; idx < total; idx += (size_t)gridDim.x * kThreads) {
    int i, h, c;
    if (blockIdx.y == 0) {             // token-major, vector fastest
      c = idx % cpr;
      h = (idx / cpr) % H;
      i = idx / ((size_t)cpr * H);
    } else {                            // token fastest
      i = idx % n_tokens;
      c = (idx / n_tokens) % cpr;
      h = idx / ((size_t)n_tokens * cpr);
    }
    const int slot = slots[i];
    if (slot < 0) continue;
    if ((size_t)slot >= cap) {
      flag_error(pool.err, PKV_ERRBIT_SLOT);
      continue;
    }
    const int blk = slot >> pool.bs_shift;
    const int off = slot & (pool.block_size - 1);
    const int shard = h / hl, lh = h - shard * hl;
    const size_t tile = tile_elems(pool, blk, lh);
    const size_t src = ((size_t)i * H + h) * D + c * VEC;
    if (blockIdx.y == 0) {
      T* dst = reinterpret_cast<T*>(pool.k[shard]) + tile + (size_t)off * D + c * VEC;
      *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(k + src);
    } else {
      union { uint4 u; T e[VEC]; } val;
      val.u = *reinterpret_cast<const uint4*>(v + src);
      T* dst = reinterpret_cast<T*>(pool.v[shard]) + tile + (size_t)(c * VEC) * pool.block_size + off;
#pragma unroll
      for (int j = 0; j < VEC; ++j) dst[(size_t)j * pool.block_size] = val.e[j];
    }
  }
}

// ------------------------------------------------------------- relayout ----
// One workgroup per (destination block j of the request, head).  The
// destination (block, head) K tile and V tile are each one contiguous run
// of block_size * head_dim elements; every thread fills 16-byte vectors of
// both from the matching 16 bytes of the source tiles.  The source block ids
// of the tokens in this destination block are read from the table once, into
// LDS; the shard base pointers are uniform per workgroup; each thread issues
// all its loads (K and V) before its non-temporal stores.  Block sizes are
// powers of two >= 16, so a 16-byte run of keys of one dim (V) never
// straddles a source block.  Tokens at or past n_tokens are not written.
constexpr int kRelayoutVpt = 2;    // vectors per thread per tile and round

template <typename T>
__global__ void __launch_bounds__(kThreads)
kv_relayout_kernel(PoolDev src, const int32_t* __restrict__ src_bt, PoolDev dst,
                   const int32_t* __restrict__ dst_bt, int n_tokens) {
  constexpr int VEC = 16 / sizeof(T);
  __shared__ int sblk[128 / 16];           // source blocks covering one destination block
  const int j = blockIdx.x;                // destination block index within the request
  const int h = blockIdx.y;
  const int D = dst.head_dim;
  const int bsd = dst.block_size, bss = src.block_size;
  const int p0 = j * bsd;
  const int valid = min(bsd, n_tokens - p0);     // tokens of this block that exist
  const int dblk = dst_bt[j];
  if (dblk < 0 || dblk >= dst.num_blocks) {
    if (threadIdx.x == 0) flag_error(dst.err, PKV_ERRBIT_BLOCK_ID);
    return;
  }
  const int first = p0 >> src.bs_shift;
  const int nsrc = ((p0 + valid - 1) >> src.bs_shift) - first + 1;
  if ((int)threadIdx.x < nsrc) {
    int b = src_bt[first + threadIdx.x];
    if (b < 0 || b >= src.num_blocks) {
      flag_error(src.err, PKV_ERRBIT_BLOCK_ID);
      b = -1;
    }
    sblk[threadIdx.x] = b;
  }
  __syncthreads();
  const int dsh = h / dst.heads_per_shard, dlh = h - dsh * dst.heads_per_shard;
  const int ssh = h / src.heads_per_shard, slh = h - ssh * src.heads_per_shard;
  const T* sk = reinterpret_cast<const T*>(src.k[ssh]);
  const T* sv = reinterpret_cast<const T*>(src.v[ssh]);
  T* dk = reinterpret_cast<T*>(dst.k[dsh]) + tile_elems(dst, dblk, dlh);
  T* dv = reinterpret_cast<T*>(dst.v[dsh]) + tile_elems(dst, dblk, dlh);
  const int off0 = p0 & (bss - 1);               // p0's offset in its source block (bss > bsd only)
  const int vpr_shift = __builtin_ctz(D / VEC);  // K: vectors per row
  const int vpk_shift = __builtin_ctz(bsd / VEC);// V: vectors per dim row
  const int nv = (bsd * D) / VEC;                // vectors per tile
  const size_t stile = (size_t)bss * D;
  for (int base = threadIdx.x; base < nv; base += kThreads * kRelayoutVpt) {
    uint4 kv[kRelayoutVpt], vv[kRelayoutVpt];
    bool kok[kRelayoutVpt], vok[kRelayoutVpt];
    int kdo[kRelayoutVpt], vdo[kRelayoutVpt];
#pragma unroll
    for (int u = 0; u < kRelayoutVpt; ++u) {
      const int e = base + u * kThreads;
      // K vector e: token o, dims d..d+VEC
      {
        const int o = e >> vpr_shift, d = (e & ((1 << vpr_shift) - 1)) * VEC;
        const int r = off0 + o;
        const int b = (e < nv && o < valid) ? sblk[r >> src.bs_shift] : -1;
        kok[u] = b >= 0;
        kdo[u] = o * D + d;
        kv[u] = kok[u] ? load_nt16(sk + ((size_t)b * src.heads_per_shard + slh) * stile +
                                   (size_t)(r & (bss - 1)) * D + d)
                       : make_uint4(0, 0, 0, 0);
      }
      // V vector e: dim d, tokens o..o+VEC
      {
        const int d = e >> vpk_shift, o = (e & ((1 << vpk_shift) - 1)) * VEC;
        const int r = off0 + o;
        const int b = (e < nv && o + VEC <= valid) ? sblk[r >> src.bs_shift] : -1;
        vok[u] = b >= 0;
        vdo[u] = d * bsd + o;
        vv[u] = vok[u] ? load_nt16(sv + ((size_t)b * src.heads_per_shard + slh) * stile + (size_t)d * bss +
                                   (r & (bss - 1)))
                       : make_uint4(0, 0, 0, 0);
        if (!vok[u] && e < nv && o < valid) {        // ragged tail of the request: element copies
          const int sb = sblk[r >> src.bs_shift];
          if (sb >= 0) {
            const T* sp = sv + ((size_t)sb * src.heads_per_shard + slh) * stile + (size_t)d * bss + (r & (bss - 1));
            for (int t = 0; t < valid - o; ++t) dv[d * bsd + o + t] = sp[t];
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kRelayoutVpt; ++u) {
      if (kok[u]) store_nt16(dk + kdo[u], kv[u]);
      if (vok[u]) store_nt16(dv + vdo[u], vv[u]);
    }
  }
}

}  // namespace

hipError_t launch_slot_mapping(const int32_t* bt, int bt_stride, const int32_t* start_loc, const int32_t* pos_start,
                               int batch, int num_tokens, int block_size, int num_blocks, int32_t* slots,
                               int32_t* err, hipStream_t s) {
  if (num_tokens == 0) return hipSuccess;
  const int grid = (num_tokens + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(grid), dim3(kThreads), 0, s, bt, bt_stride, start_loc, pos_start,
                     batch, num_tokens, block_size, num_blocks, slots, err);
  return hipGetLastError();
}

hipError_t launch_kv_write(const PoolDev& pool, int dtype, const void* k, const void* v, const int32_t* slots,
                           int n_tokens, hipStream_t s) {
  if (n_tokens == 0) return hipSuccess;
  const int esz = dtype == PKV_BF16 ? 2 : 4;
  const size_t total = (size_t)n_tokens * pool.num_kv_heads * (pool.head_dim * esz / 16);
  const int grid = (int)std::min<size_t>((total + kThreads - 1) / kThreads, 8192);
  if (dtype == PKV_BF16)
    hipLaunchKernelGGL(kv_write_kernel<bf16_t>, dim3(grid, 2), dim3(kThreads), 0, s, pool,
                       static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), slots, n_tokens);
  else
    hipLaunchKernelGGL(kv_write_kernel<float>, dim3(grid, 2), dim3(kThreads), 0, s, pool,
                       static_cast<const float*>(k), static_cast<const float*>(v), slots, n_tokens);
  return hipGetLastError();
}

hipError_t launch_kv_relayout(const PoolDev& src, const int32_t* src_bt, const PoolDev& dst, const int32_t* dst_bt,
                              int dtype, int n_tokens, hipStream_t s) {
  if (n_tokens == 0) return hipSuccess;
  const dim3 grid((n_tokens + dst.block_size - 1) / dst.block_size, dst.num_kv_heads);
  if (dtype == PKV_BF16)
    hipLaunchKernelGGL(kv_relayout_kernel<bf16_t>, grid, dim3(kThreads), 0, s, src, src_bt, dst, dst_bt, n_tokens);
  else
    hipLaunchKernelGGL(kv_relayout_kernel<float>, grid, dim3(kThreads), 0, s, src, src_bt, dst, dst_bt, n_tokens);
  return hipGetLastError();
}

}  // namespace pkv
