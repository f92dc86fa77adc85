// Calibration of what HBM delivers to the access patterns of the attention
// library's memory-bound kernels (measurement infrastructure of the
// benchmark; not part of the attention library):
//
//   * tiled read: every workgroup reads `tiles_per_wg` 4 KiB tiles at
//     positions taken from an index array (a permutation of a pool's
//     tiles), the way a decode workgroup reads the K and V tiles of one
//     (request, KV head) pair of a paged pool.  Nothing is written but one
//     word per thread.
//   * tiled copy: every workgroup copies `tiles_per_wg` 4 KiB tiles from
//     permuted source positions to permuted destination positions, the
//     traffic of a relayout between two paged pools.
//   * contiguous copy of the same byte count.
//
// Loads carry the non-temporal hint (each byte is read once); all of a
// thread's loads of a round are issued before any is consumed.  Stores are
// vector stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kTile = 4096;                      // bytes
constexpr int kThreads = 256;                    // one 16-byte vector per thread per tile

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld_nt(const void* p) {
  return __builtin_nontemporal_load(static_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st_nt(u32x4 v, void* p) { __builtin_nontemporal_store(v, static_cast<u32x4*>(p)); }

template <int U>
__global__ void __launch_bounds__(kThreads)
tiled_read_kernel(const char* __restrict__ pool, const int32_t* __restrict__ ids, int tiles_per_wg,
                  uint32_t* __restrict__ sink) {
  const int32_t* my = ids + (size_t)blockIdx.x * tiles_per_wg;
  const int off = threadIdx.x * 16;
  uint32_t acc = 0;
  for (int t = 0; t < tiles_per_wg; t += U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = t + u < tiles_per_wg ? ld_nt(pool + (size_t)my[t + u] * kTile + off) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

template <int U>
__global__ void __launch_bounds__(kThreads)
tiled_copy_kernel(const char* __restrict__ src, const int32_t* __restrict__ sids, char* __restrict__ dst,
                  const int32_t* __restrict__ dids, int tiles_per_wg) {
  const size_t base = (size_t)blockIdx.x * tiles_per_wg;
  const int off = threadIdx.x * 16;
  for (int t = 0; t < tiles_per_wg; t += U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (t + u < tiles_per_wg) v[u] = ld_nt(src + (size_t)sids[base + t + u] * kTile + off);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (t + u < tiles_per_wg) st_nt(v[u], dst + (size_t)dids[base + t + u] * kTile + off);
  }
}

__global__ void __launch_bounds__(kThreads)
contiguous_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += (size_t)gridDim.x * kThreads)
    st_nt(ld_nt(src + i), dst + i);
}

}  // namespace

extern "C" {

// Tiled read: `wgs` workgroups of 256 threads, workgroup w reads the 4 KiB
// tiles ids[w * tiles_per_wg .. +tiles_per_wg) of `pool` (device; every id
// must lie inside the pool: the caller builds them), `unroll` (4, 8 or 16)
// tiles per round.  sink: device uint32 [wgs * 256].  Returns 0 or the HIP
// error (hipErrorInvalidValue for a bad argument).
int pkv_calib_tiled_read(const void* pool, const int32_t* ids, int wgs, int tiles_per_wg, int unroll, uint32_t* sink,
                         hipStream_t stream) {
  if (!pool || !ids || !sink || wgs <= 0 || tiles_per_wg <= 0) return (int)hipErrorInvalidValue;
  const dim3 g(wgs), b(kThreads);
  const char* p = static_cast<const char*>(pool);
  switch (unroll) {
    case 4: hipLaunchKernelGGL(tiled_read_kernel<4>, g, b, 0, stream, p, ids, tiles_per_wg, sink); break;
    case 8: hipLaunchKernelGGL(tiled_read_kernel<8>, g, b, 0, stream, p, ids, tiles_per_wg, sink); break;
    case 16: hipLaunchKernelGGL(tiled_read_kernel<16>, g, b, 0, stream, p, ids, tiles_per_wg, sink); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

// Tiled copy: workgroup w copies tile sids[i] of src to tile dids[i] of dst
// for i in [w * tiles_per_wg, +tiles_per_wg), `unroll` (2 or 4) tiles per
// round.  Ids must lie inside their buffers and dids must not repeat.
int pkv_calib_tiled_copy(const void* src, const int32_t* sids, void* dst, const int32_t* dids, int wgs,
                         int tiles_per_wg, int unroll, hipStream_t stream) {
  if (!src || !sids || !dst || !dids || wgs <= 0 || tiles_per_wg <= 0) return (int)hipErrorInvalidValue;
  const dim3 g(wgs), b(kThreads);
  const char* s = static_cast<const char*>(src);
  char* d = static_cast<char*>(dst);
  switch (unroll) {
    case 2: hipLaunchKernelGGL(tiled_copy_kernel<2>, g, b, 0, stream, s, sids, d, dids, tiles_per_wg); break;
    case 4: hipLaunchKernelGGL(tiled_copy_kernel<4>, g, b, 0, stream, s, sids, d, dids, tiles_per_wg); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

// Contiguous copy of `bytes` (a multiple of 16; both pointers 16-byte
// aligned) with `wgs` workgroups of 256 threads in a grid-stride loop.
int pkv_calib_copy(const void* src, void* dst, size_t bytes, int wgs, hipStream_t stream) {
  if (!src || !dst || wgs <= 0 || bytes % 16 != 0 || ((uintptr_t)src | (uintptr_t)dst) % 16 != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(contiguous_copy_kernel, dim3(wgs), dim3(kThreads), 0, stream, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), bytes / 16);
  return (int)hipGetLastError();
}

}  // extern "C"
