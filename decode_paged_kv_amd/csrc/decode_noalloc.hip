// attn_decode without a caller workspace: the split-KV partial results go
// to a fixed device array of this library instead, so the call allocates
// nothing (for callers that cannot: code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, at its own address, until the process ends.  In
// host code its name is only a stand-in for the symbol, so the device
// address is looked up once per device (hipGetSymbolAddress, with that
// device current) and that address is what the kernels receive.
//
// Nothing in the array needs clearing between calls: every partial row a
// launch's merge kernel reads is written earlier in the same launch
// sequence.  All calls on one GPU share the array, so calls that can
// overlap on one GPU (other streams, graph replays) race with each other.
#include <mutex>

#include "pkv_internal.h"

namespace pkv {
int fail(int code, const char* fmt, ...);
int hip_fail(hipError_t e, const char* where);
int check_pool(const pkv_pool_layer* p, const char* name, PoolDev* out);
int check_heads(const PoolDev& pool, int num_q_heads);
bool scale_ok(float x);
bool aligned16(const void* p);
float resolve_scale(float scale, int head_dim);
void clear_error();
}  // namespace pkv

using namespace pkv;

namespace {

constexpr size_t kScratchBytes = PKV_DECODE_NOALLOC_SCRATCH_BYTES;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up on the
// first call made with that device current, then kept).
int scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "attn_decode_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PKV_EUNSUPPORTED, "attn_decode_noalloc: device %d (at most %d devices)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "attn_decode_noalloc: hipGetSymbolAddress(scratch)");
    if (!p) return fail(PKV_EHIP, "attn_decode_noalloc: hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

int attn_decode_noalloc(const pkv_pool_layer* pool, const void* q, void* out, const int32_t* block_tables,
                        int32_t bt_stride, const int32_t* context_lens, int32_t batch, int32_t max_context_len,
                        int32_t num_q_heads, float scale, hipStream_t stream) {
  clear_error();
  PoolDev pd;
  if (int rc = check_pool(pool, "attn_decode_noalloc", &pd)) return rc;
  if (int rc = check_heads(pd, num_q_heads)) return rc;
  if (batch < 0) return fail(PKV_EINVAL, "attn_decode_noalloc: batch %d", batch);
  if (batch == 0) return PKV_OK;
  if (max_context_len <= 0) return fail(PKV_EINVAL, "attn_decode_noalloc: max_context_len %d", max_context_len);
  if (!q || !out || !block_tables || !context_lens) return fail(PKV_EINVAL, "attn_decode_noalloc: NULL device array");
  if (!aligned16(q) || !aligned16(out)) return fail(PKV_EINVAL, "attn_decode_noalloc: q/out must be 16-byte aligned");
  if (bt_stride <= 0 || (int64_t)bt_stride * pd.block_size < max_context_len)
    return fail(PKV_EINVAL, "attn_decode_noalloc: bt_stride %d blocks cannot hold %d tokens", bt_stride,
                max_context_len);
  if (!scale_ok(scale)) return fail(PKV_EINVAL, "attn_decode_noalloc: scale must be finite and >= 0");
  const DecodePlan plan = plan_decode(batch, num_q_heads, pd.num_kv_heads, max_context_len, pd.head_dim, pool->dtype);
  if (plan.workspace > kScratchBytes)
    return fail(PKV_ERANGE, "attn_decode_noalloc: the split plan needs %zu bytes of partial results, more than the "
                "%zu-byte scratch (use attn_decode with a workspace)", plan.workspace, kScratchBytes);
  void* ws = nullptr;
  if (plan.workspace > 0)
    if (int rc = scratch_on_current_device(&ws)) return rc;
  hipError_t e = launch_attn_decode(pd, pool->dtype, q, out, block_tables, bt_stride, context_lens, batch,
                                    num_q_heads, resolve_scale(scale, pd.head_dim), plan, ws, stream);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "attn_decode_noalloc");
}

}  // extern "C"
