// C-ABI entry points of libpkv: host-side argument validation, then the
// kernel launchers.  Every check here runs before any HIP call, so a
// rejected call enqueues nothing.  See include/pkv.h for the contracts.
#include <cmath>
#include <cstring>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "pkv_internal.h"

namespace pkv {

thread_local std::string g_last_error;

void clear_error() { g_last_error.clear(); }

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(PKV_EHIP, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static int log2_exact(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return (1 << s) == x ? s : -1;
}

// Validates one pool layer and fills the kernel-side descriptor.
int check_pool(const pkv_pool_layer* p, const char* name, PoolDev* out) {
  if (!p) return fail(PKV_EINVAL, "%s: pool is NULL", name);
  if (p->dtype != PKV_F32 && p->dtype != PKV_BF16) return fail(PKV_EUNSUPPORTED, "%s: dtype %d", name, p->dtype);
  if (p->num_blocks <= 0) return fail(PKV_EINVAL, "%s: num_blocks %d", name, p->num_blocks);
  if (p->block_size != 16 && p->block_size != 32 && p->block_size != 64 && p->block_size != 128)
    return fail(PKV_EUNSUPPORTED, "%s: block_size %d (supported: 16, 32, 64, 128)", name, p->block_size);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(PKV_EUNSUPPORTED, "%s: head_dim %d (supported: 64, 128)", name, p->head_dim);
  if (p->num_kv_heads <= 0) return fail(PKV_EINVAL, "%s: num_kv_heads %d", name, p->num_kv_heads);
  if (p->num_shards <= 0 || p->num_shards > PKV_MAX_SHARDS)
    return fail(PKV_EINVAL, "%s: num_shards %d (1..%d)", name, p->num_shards, PKV_MAX_SHARDS);
  if (p->num_kv_heads % p->num_shards)
    return fail(PKV_EUNSUPPORTED, "%s: %d shards do not divide %d kv heads", name, p->num_shards, p->num_kv_heads);
  const size_t elems = (size_t)p->num_blocks * (p->num_kv_heads / p->num_shards) * p->block_size * p->head_dim;
  if (elems > (size_t)1 << 40) return fail(PKV_ERANGE, "%s: shard of %zu elements is too large", name, elems);
  for (int s = 0; s < p->num_shards; ++s) {
    if (!p->k[s] || !p->v[s]) return fail(PKV_EINVAL, "%s: shard %d has a NULL K or V pointer", name, s);
    if (!aligned16(p->k[s]) || !aligned16(p->v[s]))
      return fail(PKV_EINVAL, "%s: shard %d K/V pointers must be 16-byte aligned", name, s);
  }
  for (int s = 0; s < PKV_MAX_SHARDS; ++s) {
    out->k[s] = s < p->num_shards ? static_cast<char*>(p->k[s]) : nullptr;
    out->v[s] = s < p->num_shards ? static_cast<char*>(p->v[s]) : nullptr;
  }
  out->num_blocks = p->num_blocks;
  out->block_size = p->block_size;
  out->bs_shift = log2_exact(p->block_size);
  out->heads_per_shard = p->num_kv_heads / p->num_shards;
  out->num_kv_heads = p->num_kv_heads;
  out->head_dim = p->head_dim;
  out->err = p->err_word;
  return PKV_OK;
}

int check_heads(const PoolDev& pool, int num_q_heads) {
  if (num_q_heads <= 0 || num_q_heads % pool.num_kv_heads)
    return fail(PKV_EINVAL, "num_q_heads %d is not a positive multiple of %d kv heads", num_q_heads,
                pool.num_kv_heads);
  const int g = num_q_heads / pool.num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16)
    return fail(PKV_EUNSUPPORTED, "%d q-heads per kv head (supported: 1, 2, 4, 8, 16)", g);
  return PKV_OK;
}

// Finite and >= 0 (0 selects the default scale), tested on the bits: the
// library is built without NaN semantics for comparisons, so a NaN compare
// would be folded away.
bool scale_ok(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  return (u & 0x7f800000u) != 0x7f800000u && !(u >> 31 && (u & 0x7fffffffu));
}
// finite and > 0
bool positive_finite(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  return (u & 0x7f800000u) != 0x7f800000u && !(u >> 31) && (u & 0x7fffffffu);
}

float resolve_scale(float scale, int head_dim) {
  return scale > 0.f ? scale : 1.0f / std::sqrt((float)head_dim);
}

}  // namespace pkv

using namespace pkv;

extern "C" {

const char* pkv_last_error(void) { return g_last_error.c_str(); }

int pkv_version(void) { return PKV_VERSION; }

int pkv_slot_mapping(const int32_t* block_tables, int32_t bt_stride, const int32_t* start_loc,
                     const int32_t* pos_start, int32_t batch, int32_t num_tokens, int32_t block_size,
                     int32_t num_blocks, int32_t* slots_out, int32_t* err_word, hipStream_t stream) {
  g_last_error.clear();
  if (num_tokens < 0 || batch < 0) return fail(PKV_EINVAL, "pkv_slot_mapping: negative batch or token count");
  if (num_tokens == 0) return PKV_OK;
  if (batch == 0) return fail(PKV_EINVAL, "pkv_slot_mapping: tokens but no requests");
  if (!block_tables || !start_loc || !pos_start || !slots_out)
    return fail(PKV_EINVAL, "pkv_slot_mapping: NULL device array");
  if (bt_stride <= 0) return fail(PKV_EINVAL, "pkv_slot_mapping: bt_stride %d", bt_stride);
  if (log2_exact(block_size) < 4 || block_size > 128)
    return fail(PKV_EUNSUPPORTED, "pkv_slot_mapping: block_size %d", block_size);
  if (num_blocks <= 0) return fail(PKV_EINVAL, "pkv_slot_mapping: num_blocks %d", num_blocks);
  if ((int64_t)num_blocks * block_size > INT32_MAX) return fail(PKV_ERANGE, "pkv_slot_mapping: pool too large");
  hipError_t e = launch_slot_mapping(block_tables, bt_stride, start_loc, pos_start, batch, num_tokens, block_size,
                                     num_blocks, slots_out, err_word, stream);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "pkv_slot_mapping");
}

int kv_write(const pkv_pool_layer* pool, const void* k, const void* v, const int32_t* slots, int32_t n_tokens,
             hipStream_t stream) {
  g_last_error.clear();
  PoolDev pd;
  if (int rc = check_pool(pool, "kv_write", &pd)) return rc;
  if (n_tokens < 0) return fail(PKV_EINVAL, "kv_write: n_tokens %d", n_tokens);
  if (n_tokens == 0) return PKV_OK;
  if (!k || !v || !slots) return fail(PKV_EINVAL, "kv_write: NULL k, v or slots");
  if (!aligned16(k) || !aligned16(v)) return fail(PKV_EINVAL, "kv_write: k and v must be 16-byte aligned");
  if ((int64_t)pd.num_blocks * pd.block_size > INT32_MAX) return fail(PKV_ERANGE, "kv_write: pool too large");
  hipError_t e = launch_kv_write(pd, pool->dtype, k, v, slots, n_tokens, stream);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "kv_write");
}

int kv_relayout(const pkv_pool_layer* src, const int32_t* src_bt, const pkv_pool_layer* dst, const int32_t* dst_bt,
                int32_t n_tokens, hipStream_t stream) {
  g_last_error.clear();
  PoolDev ps, pd;
  if (int rc = check_pool(src, "kv_relayout(src)", &ps)) return rc;
  if (int rc = check_pool(dst, "kv_relayout(dst)", &pd)) return rc;
  if (src->num_kv_heads != dst->num_kv_heads || src->head_dim != dst->head_dim)
    return fail(PKV_EINVAL, "kv_relayout: heads/head_dim differ (%d/%d vs %d/%d)", src->num_kv_heads,
                src->head_dim, dst->num_kv_heads, dst->head_dim);
  if (src->dtype != dst->dtype) return fail(PKV_EUNSUPPORTED, "kv_relayout: dtype conversion is not supported");
  if (n_tokens < 0) return fail(PKV_EINVAL, "kv_relayout: n_tokens %d", n_tokens);
  if (n_tokens == 0) return PKV_OK;
  if (!src_bt || !dst_bt) return fail(PKV_EINVAL, "kv_relayout: NULL block table");
  if ((int64_t)src->num_blocks * src->block_size < n_tokens || (int64_t)dst->num_blocks * dst->block_size < n_tokens)
    return fail(PKV_EINVAL, "kv_relayout: %d tokens do not fit a pool", n_tokens);
  for (int s = 0; s < src->num_shards; ++s)
    for (int t = 0; t < dst->num_shards; ++t)
      if (src->k[s] == dst->k[t] || src->v[s] == dst->v[t])
        return fail(PKV_EINVAL, "kv_relayout: source and destination share a shard buffer");
  hipError_t e = launch_kv_relayout(ps, src_bt, pd, dst_bt, src->dtype, n_tokens, stream);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "kv_relayout");
}

int kv_relayout_convert(const pkv_pool_layer* src, const int32_t* src_bt, const pkv_kv_dest* dst,
                        const int32_t* dst_bt, int32_t n_tokens, hipStream_t stream) {
  g_last_error.clear();
  PoolDev ps;
  if (int rc = check_pool(src, "kv_relayout_convert(src)", &ps)) return rc;
  if (!dst) return fail(PKV_EINVAL, "kv_relayout_convert: dst is NULL");
  if (dst->num_kv_heads != src->num_kv_heads || dst->head_dim != src->head_dim)
    return fail(PKV_EINVAL, "kv_relayout_convert: heads/head_dim differ (%d/%d vs %d/%d)", src->num_kv_heads,
                src->head_dim, dst->num_kv_heads, dst->head_dim);
  if (dst->num_blocks <= 0) return fail(PKV_EINVAL, "kv_relayout_convert: dst num_blocks %d", dst->num_blocks);
  if (log2_exact(dst->block_size) < 4 || dst->block_size > 128)
    return fail(PKV_EUNSUPPORTED, "kv_relayout_convert: dst block_size %d (supported: 16, 32, 64, 128)",
                dst->block_size);
  if (dst->num_shards <= 0 || dst->num_shards > PKV_MAX_SHARDS || dst->num_kv_heads % dst->num_shards)
    return fail(PKV_EUNSUPPORTED, "kv_relayout_convert: %d dst shards for %d kv heads", dst->num_shards,
                dst->num_kv_heads);
  if (dst->layout != PKV_LAYOUT_POOL && dst->layout != PKV_LAYOUT_TOKEN_MAJOR && dst->layout != PKV_LAYOUT_KV_FUSED)
    return fail(PKV_EINVAL, "kv_relayout_convert: layout %d", dst->layout);
  const bool fp8 = dst->dtype == PKV_FP8_E4M3;
  if (!(dst->dtype == src->dtype || (fp8 && src->dtype == PKV_BF16)))
    return fail(PKV_EUNSUPPORTED, "kv_relayout_convert: dtype %d -> %d", src->dtype, dst->dtype);
  if (fp8 && !positive_finite(dst->scale))
    return fail(PKV_EINVAL, "kv_relayout_convert: FP8 scale must be finite and > 0");
  const size_t esize = fp8 ? 1 : (src->dtype == PKV_BF16 ? 2 : 4);
  const size_t per_shard = (size_t)dst->num_blocks * (dst->num_kv_heads / dst->num_shards) * dst->block_size *
                           dst->head_dim * esize * (dst->layout == PKV_LAYOUT_KV_FUSED ? 2 : 1);
  if (per_shard > ((size_t)1 << 42)) return fail(PKV_ERANGE, "kv_relayout_convert: dst shard too large");
  for (int t = 0; t < dst->num_shards; ++t) {
    const bool need_v = dst->layout != PKV_LAYOUT_KV_FUSED;
    if (!dst->k[t] || (need_v && !dst->v[t]))
      return fail(PKV_EINVAL, "kv_relayout_convert: dst shard %d has a NULL buffer", t);
    if (!aligned16(dst->k[t]) || (need_v && !aligned16(dst->v[t])))
      return fail(PKV_EINVAL, "kv_relayout_convert: dst shard %d buffers must be 16-byte aligned", t);
    for (int s = 0; s < src->num_shards; ++s)
      if (dst->k[t] == src->k[s] || dst->k[t] == src->v[s] || (need_v && (dst->v[t] == src->k[s] || dst->v[t] == src->v[s])))
        return fail(PKV_EINVAL, "kv_relayout_convert: source and destination share a buffer");
  }
  if (n_tokens < 0) return fail(PKV_EINVAL, "kv_relayout_convert: n_tokens %d", n_tokens);
  if (n_tokens == 0) return PKV_OK;
  if (!src_bt || !dst_bt) return fail(PKV_EINVAL, "kv_relayout_convert: NULL block table");
  if ((int64_t)src->num_blocks * src->block_size < n_tokens || (int64_t)dst->num_blocks * dst->block_size < n_tokens)
    return fail(PKV_EINVAL, "kv_relayout_convert: %d tokens do not fit a pool", n_tokens);
  hipError_t e = launch_kv_relayout_convert(ps, src_bt, *dst, dst->num_kv_heads / dst->num_shards, dst_bt,
                                            src->dtype, n_tokens, ps.err, stream);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "kv_relayout_convert");
}

int attn_prefill_chunk(const pkv_pool_layer* pool, const void* q, void* out, const int32_t* block_tables,
                       int32_t bt_stride, const int32_t* start_loc, const int32_t* chunk_start, int32_t batch,
                       int32_t max_chunk_len, int32_t max_total_len, int32_t num_q_heads, float scale,
                       hipStream_t stream) {
  g_last_error.clear();
  PoolDev pd;
  if (int rc = check_pool(pool, "attn_prefill_chunk", &pd)) return rc;
  if (int rc = check_heads(pd, num_q_heads)) return rc;
  if (batch < 0 || max_chunk_len < 0) return fail(PKV_EINVAL, "attn_prefill_chunk: negative batch or chunk length");
  if (batch == 0 || max_chunk_len == 0) return PKV_OK;
  if (!q || !out || !block_tables || !start_loc || !chunk_start)
    return fail(PKV_EINVAL, "attn_prefill_chunk: NULL device array");
  if (!aligned16(q) || !aligned16(out)) return fail(PKV_EINVAL, "attn_prefill_chunk: q/out must be 16-byte aligned");
  if (bt_stride <= 0) return fail(PKV_EINVAL, "attn_prefill_chunk: bt_stride %d", bt_stride);
  if (max_total_len < max_chunk_len)
    return fail(PKV_EINVAL, "attn_prefill_chunk: max_total_len %d is below max_chunk_len %d", max_total_len,
                max_chunk_len);
  if ((int64_t)bt_stride * pd.block_size < max_total_len)
    return fail(PKV_EINVAL, "attn_prefill_chunk: bt_stride %d blocks cannot hold %d tokens", bt_stride,
                max_total_len);
  if (!scale_ok(scale)) return fail(PKV_EINVAL, "attn_prefill_chunk: scale must be finite and >= 0");
  if ((int64_t)max_chunk_len * 2 > INT32_MAX / 64) return fail(PKV_ERANGE, "attn_prefill_chunk: chunk too long");
  hipError_t e = launch_attn_prefill(pd, pool->dtype, q, out, block_tables, bt_stride, start_loc, chunk_start, batch,
                                     max_chunk_len, max_total_len, num_q_heads, resolve_scale(scale, pd.head_dim),
                                     stream);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "attn_prefill_chunk");
}

size_t pkv_attn_decode_workspace_size_for(const pkv_pool_layer* pool, int32_t batch, int32_t num_q_heads,
                                          int32_t max_context_len) {
  // the plan attn_decode, attn_decode_append and run_mux_round make for this
  // pool (KV heads, head dim, dtype); 0 for arguments those calls reject
  if (!pool || batch <= 0 || num_q_heads <= 0 || max_context_len <= 0) return 0;
  if (pool->num_kv_heads <= 0 || num_q_heads % pool->num_kv_heads) return 0;
  if (pool->dtype != PKV_F32 && pool->dtype != PKV_BF16) return 0;
  return plan_decode(batch, num_q_heads, pool->num_kv_heads, max_context_len, pool->head_dim, pool->dtype).workspace;
}

size_t pkv_attn_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t max_context_len,
                                      int32_t head_dim) {
  // the plan depends on the KV head count and the dtype, which are not
  // given: the largest need over the group sizes and both dtypes
  if (batch <= 0 || num_q_heads <= 0 || max_context_len <= 0 || head_dim <= 0) return 0;
  size_t worst = 0;
  for (int g = 1; g <= 16 && g <= num_q_heads; g *= 2) {
    if (num_q_heads % g) continue;
    for (int dt : {(int)PKV_F32, (int)PKV_BF16}) {
      const DecodePlan p = plan_decode(batch, num_q_heads, num_q_heads / g, max_context_len, head_dim, dt);
      if (p.workspace > worst) worst = p.workspace;
    }
  }
  return worst;
}

int attn_decode(const pkv_pool_layer* pool, const void* q, void* out, const int32_t* block_tables, int32_t bt_stride,
                const int32_t* context_lens, int32_t batch, int32_t max_context_len, int32_t num_q_heads,
                float scale, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  PoolDev pd;
  if (int rc = check_pool(pool, "attn_decode", &pd)) return rc;
  if (int rc = check_heads(pd, num_q_heads)) return rc;
  if (batch < 0) return fail(PKV_EINVAL, "attn_decode: batch %d", batch);
  if (batch == 0) return PKV_OK;
  if (max_context_len <= 0) return fail(PKV_EINVAL, "attn_decode: max_context_len %d", max_context_len);
  if (!q || !out || !block_tables || !context_lens) return fail(PKV_EINVAL, "attn_decode: NULL device array");
  if (!aligned16(q) || !aligned16(out)) return fail(PKV_EINVAL, "attn_decode: q/out must be 16-byte aligned");
  if (bt_stride <= 0 || (int64_t)bt_stride * pd.block_size < max_context_len)
    return fail(PKV_EINVAL, "attn_decode: bt_stride %d blocks cannot hold %d tokens", bt_stride, max_context_len);
  if (!scale_ok(scale)) return fail(PKV_EINVAL, "attn_decode: scale must be finite and >= 0");
  const DecodePlan plan = plan_decode(batch, num_q_heads, pd.num_kv_heads, max_context_len, pd.head_dim, pool->dtype);
  if (plan.workspace > 0) {
    if (!workspace || workspace_bytes < plan.workspace)
      return fail(PKV_EINVAL, "attn_decode: workspace of %zu bytes needed, %zu given", plan.workspace,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(PKV_EINVAL, "attn_decode: workspace must be 16-byte aligned");
  }
  hipError_t e = launch_attn_decode(pd, pool->dtype, q, out, block_tables, bt_stride, context_lens, batch, num_q_heads,
                                    resolve_scale(scale, pd.head_dim), plan, workspace, stream);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "attn_decode");
}

int attn_decode_append(const pkv_pool_layer* pool, const void* q, const void* k_new, const void* v_new, void* out,
                       const int32_t* block_tables, int32_t bt_stride, const int32_t* context_lens, int32_t batch,
                       int32_t max_context_len, int32_t num_q_heads, float scale, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  PoolDev pd;
  if (int rc = check_pool(pool, "attn_decode_append", &pd)) return rc;
  if (int rc = check_heads(pd, num_q_heads)) return rc;
  if (batch < 0) return fail(PKV_EINVAL, "attn_decode_append: batch %d", batch);
  if (batch == 0) return PKV_OK;
  if (max_context_len <= 0) return fail(PKV_EINVAL, "attn_decode_append: max_context_len %d", max_context_len);
  if (!q || !out || !block_tables || !context_lens || !k_new || !v_new)
    return fail(PKV_EINVAL, "attn_decode_append: NULL device array");
  if (!aligned16(q) || !aligned16(out) || !aligned16(k_new) || !aligned16(v_new))
    return fail(PKV_EINVAL, "attn_decode_append: q/k_new/v_new/out must be 16-byte aligned");
  if (bt_stride <= 0 || (int64_t)bt_stride * pd.block_size < max_context_len)
    return fail(PKV_EINVAL, "attn_decode_append: bt_stride %d blocks cannot hold %d tokens", bt_stride,
                max_context_len);
  if (!scale_ok(scale)) return fail(PKV_EINVAL, "attn_decode_append: scale must be finite and >= 0");
  const DecodePlan plan = plan_decode(batch, num_q_heads, pd.num_kv_heads, max_context_len, pd.head_dim, pool->dtype);
  if (plan.workspace > 0) {
    if (!workspace || workspace_bytes < plan.workspace)
      return fail(PKV_EINVAL, "attn_decode_append: workspace of %zu bytes needed, %zu given", plan.workspace,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(PKV_EINVAL, "attn_decode_append: workspace must be 16-byte aligned");
  }
  hipError_t e = launch_attn_decode(pd, pool->dtype, q, out, block_tables, bt_stride, context_lens, batch, num_q_heads,
                                    resolve_scale(scale, pd.head_dim), plan, workspace, stream, k_new, v_new);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "attn_decode_append");
}

int pkv_stall_free_chunk(int32_t token_budget, int32_t num_decode, int32_t prompt_remaining) {
  g_last_error.clear();
  if (token_budget < 0 || num_decode < 0 || prompt_remaining < 0)
    return fail(PKV_EINVAL, "pkv_stall_free_chunk: negative argument");
  const int32_t left = token_budget > num_decode ? token_budget - num_decode : 0;
  return prompt_remaining < left ? prompt_remaining : left;
}

int pkv_stall_free_batch(int32_t token_budget, int32_t num_decode, const int32_t* prompt_remaining,
                         int32_t num_prompts, int32_t* chunks_out) {
  g_last_error.clear();
  if (token_budget < 0 || num_decode < 0 || num_prompts < 0)
    return fail(PKV_EINVAL, "pkv_stall_free_batch: negative argument");
  if (num_prompts > 0 && (!prompt_remaining || !chunks_out))
    return fail(PKV_EINVAL, "pkv_stall_free_batch: NULL prompt or chunk array");
  for (int i = 0; i < num_prompts; ++i)
    if (prompt_remaining[i] < 0) return fail(PKV_EINVAL, "pkv_stall_free_batch: prompt %d has %d tokens left", i,
                                             prompt_remaining[i]);
  // decode first (one token each, never dropped); then each prompt in the
  // caller's order, the ongoing ones before the new, takes what is left
  int64_t left = token_budget > num_decode ? (int64_t)token_budget - num_decode : 0;
  int64_t total = 0;
  for (int i = 0; i < num_prompts; ++i) {
    const int64_t take = prompt_remaining[i] < left ? prompt_remaining[i] : left;
    chunks_out[i] = (int32_t)take;
    left -= take;
    total += take;
  }
  return (int)total;
}

int attn_mixed_batch(const pkv_pool_layer* pool, const void* q_dec, void* out_dec, const int32_t* dec_block_tables,
                     int32_t dec_bt_stride, const int32_t* context_lens, int32_t num_decode, int32_t max_context_len,
                     const void* q_pf, void* out_pf, const int32_t* pf_block_tables, int32_t pf_bt_stride,
                     const int32_t* start_loc, const int32_t* chunk_start, int32_t num_prefill,
                     int32_t max_chunk_len, int32_t max_total_len, int32_t num_q_heads, float scale,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  PoolDev pd;
  if (int rc = check_pool(pool, "attn_mixed_batch", &pd)) return rc;
  if (int rc = check_heads(pd, num_q_heads)) return rc;
  if (num_decode < 0 || num_prefill < 0 || max_chunk_len < 0)
    return fail(PKV_EINVAL, "attn_mixed_batch: negative batch or chunk length");
  if (!scale_ok(scale)) return fail(PKV_EINVAL, "attn_mixed_batch: scale must be finite and >= 0");
  MixedDecode d{};
  MixedPrefill p{};
  if (num_decode > 0) {
    if (max_context_len <= 0) return fail(PKV_EINVAL, "attn_mixed_batch: max_context_len %d", max_context_len);
    if (!q_dec || !out_dec || !dec_block_tables || !context_lens)
      return fail(PKV_EINVAL, "attn_mixed_batch: NULL decode array");
    if (!aligned16(q_dec) || !aligned16(out_dec))
      return fail(PKV_EINVAL, "attn_mixed_batch: decode q/out must be 16-byte aligned");
    if (dec_bt_stride <= 0 || (int64_t)dec_bt_stride * pd.block_size < max_context_len)
      return fail(PKV_EINVAL, "attn_mixed_batch: dec_bt_stride %d blocks cannot hold %d tokens", dec_bt_stride,
                  max_context_len);
    const DecodePlan plan =
        plan_decode(num_decode, num_q_heads, pd.num_kv_heads, max_context_len, pd.head_dim, pool->dtype, false);
    if (plan.workspace > 0) {
      if (!workspace || workspace_bytes < plan.workspace)
        return fail(PKV_EINVAL, "attn_mixed_batch: workspace of %zu bytes needed, %zu given", plan.workspace,
                    workspace ? workspace_bytes : (size_t)0);
      if (!aligned16(workspace)) return fail(PKV_EINVAL, "attn_mixed_batch: workspace must be 16-byte aligned");
    }
    d = MixedDecode{q_dec, out_dec, dec_block_tables, dec_bt_stride, context_lens, num_decode, plan, workspace};
  }
  if (num_prefill > 0 && max_chunk_len > 0) {
    if (!q_pf || !out_pf || !pf_block_tables || !start_loc || !chunk_start)
      return fail(PKV_EINVAL, "attn_mixed_batch: NULL prefill array");
    if (!aligned16(q_pf) || !aligned16(out_pf))
      return fail(PKV_EINVAL, "attn_mixed_batch: prefill q/out must be 16-byte aligned");
    if (pf_bt_stride <= 0) return fail(PKV_EINVAL, "attn_mixed_batch: pf_bt_stride %d", pf_bt_stride);
    if (max_total_len < max_chunk_len)
      return fail(PKV_EINVAL, "attn_mixed_batch: max_total_len %d is below max_chunk_len %d", max_total_len,
                  max_chunk_len);
    if ((int64_t)pf_bt_stride * pd.block_size < max_total_len)
      return fail(PKV_EINVAL, "attn_mixed_batch: pf_bt_stride %d blocks cannot hold %d tokens", pf_bt_stride,
                  max_total_len);
    if ((int64_t)max_chunk_len * 2 > INT32_MAX / 64) return fail(PKV_ERANGE, "attn_mixed_batch: chunk too long");
    p = MixedPrefill{q_pf,        out_pf,      pf_block_tables, pf_bt_stride, start_loc,
                     chunk_start, num_prefill, max_chunk_len,   max_total_len};
  }
  if (d.batch == 0 && p.batch == 0) return PKV_OK;
  hipError_t e = launch_attn_mixed(pd, pool->dtype, d, p, num_q_heads, resolve_scale(scale, pd.head_dim), stream);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "attn_mixed_batch");
}

}  // extern "C"
