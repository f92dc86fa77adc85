// Single-GPU PD multiplexing: CU-masked stream pairs per split level, the
// level / layers-per-round policy, and the round loop.
//
// Page: "PD multiplexing: splitting prefill and decode by SM on one GPU",
// sections "Green contexts: carving out SMs for a stream" (a stream bound
// to a subset of compute units; bandwidth and L2 stay shared) and "SGLang's
// PD multiplexing" (split levels on a granularity grid, the level picked
// from the decode batch size, prefill cut by layer, the main loop that syncs
// only the decode stream and changes level only when a prefill starts or
// ends).  On MI355X a split is a pair of streams created with
// hipExtStreamCreateWithCUMask over complementary CU masks.
#include <hip/hip_ext.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "pkv_internal.h"

namespace pkv {
int fail(int code, const char* fmt, ...);
int hip_fail(hipError_t e, const char* where);
int check_pool(const pkv_pool_layer* p, const char* name, PoolDev* out);
int check_heads(const PoolDev& pool, int num_q_heads);
bool scale_ok(float x);
bool aligned16(const void* p);
void clear_error();
}  // namespace pkv

using namespace pkv;

namespace {
constexpr int kMaskWords = 8;    // 256 CUs
constexpr int kXcds = 8;
}  // namespace

struct pkv_mux {
  int device = 0;
  int total_cus = 0;
  int granularity = 8, min_decode = 32, group_num = 8, divisor = 36, budget = 65536;
  std::vector<std::pair<int, int>> groups;                 // (prefill CUs, decode CUs)
  std::vector<std::array<uint32_t, kMaskWords>> pmask, dmask;
  std::vector<hipStream_t> pstream, dstream;               // created on first use
  hipStream_t whole = nullptr;                             // ordinary stream: the whole device
  hipEvent_t prefill_done = nullptr;
  int level = -1;
  int override_level = -1;       // fixed level while a prefill runs (-1: the batch-size rule)
  bool level_with_prefill = false;
  bool done_pending = false;     // event recorded, completion not yet seen
  bool prefill_finished = false; // completion seen; the level changes next round
  std::vector<int> used_levels;
  std::vector<int> manual;       // decode-batch threshold of each split level (empty: the divisor rule)
  // decode step as one HIP graph per level (opt-in): the captured launches
  // and the arguments they were captured with
  bool use_graphs = false;
  bool decode_append = false;
  std::vector<std::vector<uint64_t>> graph_sig;
  std::vector<hipGraphExec_t> graph_exec;
};

namespace {

// Split levels: prefill takes x CUs, x on the granularity grid from
// `granularity` to total - granularity, prefill at least half and decode at
// least min_decode; keep `levels` of them evenly spaced from the smallest,
// listed largest prefill first.
std::vector<std::pair<int, int>> split_levels(int total, int min_part, int granularity, int min_decode, int levels) {
  std::vector<int> cand;
  for (int x = min_part; x <= total - min_part; x += granularity)
    if (2 * x >= total && total - x >= min_decode) cand.push_back(x);
  if ((int)cand.size() >= levels) {
    const int stride = std::max<int>(1, (int)cand.size() / levels);
    std::vector<int> kept;
    for (size_t i = 0; i < cand.size() && (int)kept.size() < levels; i += stride) kept.push_back(cand[i]);
    cand = kept;
  }
  std::sort(cand.rbegin(), cand.rend());
  std::vector<std::pair<int, int>> out;
  for (int x : cand) out.emplace_back(x, total - x);
  return out;
}

int choose(int n, int decode_bs, bool has_prefill, int divisor) {
  if (decode_bs > 0 && has_prefill) return std::min(n - 2, std::max(1, decode_bs * (n - 2) / divisor));
  if (decode_bs > 0) return n - 1;
  return 0;
}

// Manual divisions: split level i (1 .. n-2) is used from thresholds[i-1]
// decode requests on (thresholds non-decreasing); below the first, level 1.
int choose_manual(int n, int decode_bs, bool has_prefill, const int* thresholds) {
  if (decode_bs > 0 && has_prefill) {
    int level = 1;
    for (int i = 1; i <= n - 2; ++i)
      if (decode_bs >= thresholds[i - 1]) level = i;
    return level;
  }
  if (decode_bs > 0) return n - 1;
  return 0;
}

bool valid_thresholds(const int32_t* t, int n) {
  for (int i = 0; i < n; ++i)
    if (t[i] < 1 || (i && t[i] < t[i - 1])) return false;
  return true;
}

int choose_m(const pkv_mux* m, int decode_bs, bool has_prefill) {
  const int n = (int)m->groups.size();
  if (!m->manual.empty()) return choose_manual(n, decode_bs, has_prefill, m->manual.data());
  return choose(n, decode_bs, has_prefill, m->divisor);
}

// CU masks: decode takes the same number of CUs on every XCD.  Mask bit i of
// a queue's CU mask selects CU i / kXcds of XCD i % kXcds (the runtime
// spreads consecutive mask bits over the XCDs), so decode takes the lowest
// decode_cus / kXcds CUs of each XCD and prefill the rest.
void build_masks(int total, int decode_cus, std::array<uint32_t, kMaskWords>& pm, std::array<uint32_t, kMaskWords>& dm) {
  pm.fill(0);
  dm.fill(0);
  const int dec_per_xcd = decode_cus / kXcds;
  for (int i = 0; i < total; ++i) {
    const int cu_in_xcd = i / kXcds;
    auto& m = cu_in_xcd < dec_per_xcd ? dm : pm;
    m[i / 32] |= 1u << (i % 32);
  }
}

// A queue whose mask leaves some XCD without a CU can never run the share of
// its workgroups dispatched there; every mask used must keep >= 1 CU per XCD.
bool every_xcd_has_a_cu(const uint32_t* m, int total) {
  int per[kXcds] = {0};
  for (int i = 0; i < total; ++i)
    if ((m[i / 32] >> (i % 32)) & 1u) per[i % kXcds]++;
  for (int x = 0; x < kXcds; ++x)
    if (per[x] == 0) return false;
  return true;
}

int ensure_streams(pkv_mux* m, int level) {
  const auto& g = m->groups[level];
  if (g.first == 0 || g.second == 0) return PKV_OK;      // whole-device groups use the ordinary stream
  if (m->pstream[level] && m->dstream[level]) return PKV_OK;
  if (!every_xcd_has_a_cu(m->pmask[level].data(), m->total_cus) ||
      !every_xcd_has_a_cu(m->dmask[level].data(), m->total_cus))
    return fail(PKV_EINVAL, "CU masks of level %d leave an XCD without a CU", level);
  hipError_t e = hipExtStreamCreateWithCUMask(&m->pstream[level], kMaskWords, m->pmask[level].data());
  if (e != hipSuccess) return hip_fail(e, "hipExtStreamCreateWithCUMask(prefill)");
  e = hipExtStreamCreateWithCUMask(&m->dstream[level], kMaskWords, m->dmask[level].data());
  if (e != hipSuccess) return hip_fail(e, "hipExtStreamCreateWithCUMask(decode)");
  m->used_levels.push_back(level);
  return PKV_OK;
}

hipStream_t stream_of(const pkv_mux* m, int level, int which) {
  const auto& g = m->groups[level];
  if (g.first == 0 || g.second == 0) return m->whole;
  return which == 0 ? m->pstream[level] : m->dstream[level];
}

int sync_level(pkv_mux* m, int level) {
  if (level < 0) return PKV_OK;
  for (int w = 0; w < 2; ++w) {
    hipStream_t s = stream_of(m, level, w);
    if (!s) continue;
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  }
  return PKV_OK;
}

// Every layer's pool must have layer 0's shape: the split plan, the
// workspace size and the table checks are made once, from layer 0.
int check_layer_pools(const pkv_pool_layer* pools, int n, std::vector<PoolDev>& out, const char* what) {
  out.resize(n);
  for (int l = 0; l < n; ++l) {
    if (int rc = check_pool(&pools[l], what, &out[l])) return rc;
    const pkv_pool_layer &a = pools[0], &b = pools[l];
    if (b.dtype != a.dtype || b.num_kv_heads != a.num_kv_heads || b.head_dim != a.head_dim ||
        b.block_size != a.block_size || b.num_shards != a.num_shards || b.num_blocks != a.num_blocks)
      return fail(PKV_EINVAL, "%s: layer %d's pool differs from layer 0's (dtype, heads, head_dim, block size, "
                  "shards or blocks)", what, l);
  }
  return PKV_OK;
}

int check_decode_step(const pkv_decode_step* d, std::vector<PoolDev>& pools, DecodePlan& plan) {
  if (!d) return fail(PKV_EINVAL, "run_mux_round: decode step is NULL");
  if (d->num_layers <= 0 || !d->pools || !d->q || !d->k_new || !d->v_new || !d->out)
    return fail(PKV_EINVAL, "run_mux_round: decode step needs layers and per-layer arrays");
  if (d->batch <= 0 || d->max_context_len <= 0 || !d->slots || !d->block_tables || !d->context_lens)
    return fail(PKV_EINVAL, "run_mux_round: decode step batch/context/tables");
  if (int rc = check_layer_pools(d->pools, d->num_layers, pools, "run_mux_round(decode pool)")) return rc;
  for (int l = 0; l < d->num_layers; ++l) {
    if (!d->q[l] || !d->k_new[l] || !d->v_new[l] || !d->out[l])
      return fail(PKV_EINVAL, "run_mux_round: decode layer %d has a NULL tensor", l);
    if (!aligned16(d->q[l]) || !aligned16(d->k_new[l]) || !aligned16(d->v_new[l]) || !aligned16(d->out[l]))
      return fail(PKV_EINVAL, "run_mux_round: decode layer %d q/k_new/v_new/out must be 16-byte aligned", l);
  }
  const PoolDev& p0 = pools[0];
  if (int rc = check_heads(p0, d->num_q_heads)) return rc;
  if (!scale_ok(d->scale)) return fail(PKV_EINVAL, "run_mux_round: decode scale must be finite and >= 0");
  if (d->bt_stride <= 0 || (int64_t)d->bt_stride * p0.block_size < d->max_context_len)
    return fail(PKV_EINVAL, "run_mux_round: decode bt_stride %d blocks cannot hold %d tokens", d->bt_stride,
                d->max_context_len);
  if ((int64_t)p0.num_blocks * p0.block_size > INT32_MAX) return fail(PKV_ERANGE, "run_mux_round: pool too large");
  plan = plan_decode(d->batch, d->num_q_heads, p0.num_kv_heads, d->max_context_len, p0.head_dim, d->pools[0].dtype);
  if (plan.workspace > 0) {
    if (!d->workspace || d->workspace_bytes < plan.workspace)
      return fail(PKV_EINVAL, "run_mux_round: decode workspace of %zu bytes needed, %zu given", plan.workspace,
                  d->workspace ? d->workspace_bytes : (size_t)0);
    if (!aligned16(d->workspace)) return fail(PKV_EINVAL, "run_mux_round: decode workspace must be 16-byte aligned");
  }
  return PKV_OK;
}

int check_prefill_job(const pkv_prefill_job* p, std::vector<PoolDev>& pools) {
  if (!p) return fail(PKV_EINVAL, "run_mux_round: prefill job is NULL");
  if (p->num_layers <= 0 || !p->pools || !p->q || !p->k || !p->v || !p->out)
    return fail(PKV_EINVAL, "run_mux_round: prefill job needs layers and per-layer arrays");
  if (p->num_tokens <= 0 || !p->slots || !p->block_table || !p->start_loc || !p->chunk_start)
    return fail(PKV_EINVAL, "run_mux_round: prefill job tokens/tables");
  if (p->next_layer < 0 || p->next_layer > p->num_layers) return fail(PKV_EINVAL, "run_mux_round: next_layer");
  if (int rc = check_layer_pools(p->pools, p->num_layers, pools, "run_mux_round(prefill pool)")) return rc;
  for (int l = 0; l < p->num_layers; ++l) {
    if (!p->q[l] || !p->k[l] || !p->v[l] || !p->out[l])
      return fail(PKV_EINVAL, "run_mux_round: prefill layer %d has a NULL tensor", l);
    if (!aligned16(p->q[l]) || !aligned16(p->k[l]) || !aligned16(p->v[l]) || !aligned16(p->out[l]))
      return fail(PKV_EINVAL, "run_mux_round: prefill layer %d q/k/v/out must be 16-byte aligned", l);
  }
  if (int rc = check_heads(pools[0], p->num_q_heads)) return rc;
  if (!scale_ok(p->scale)) return fail(PKV_EINVAL, "run_mux_round: prefill scale must be finite and >= 0");
  if (p->bt_stride <= 0 || (int64_t)p->bt_stride * pools[0].block_size < p->num_tokens)
    return fail(PKV_EINVAL, "run_mux_round: prefill bt_stride %d blocks cannot hold %d tokens", p->bt_stride,
                p->num_tokens);
  if ((int64_t)p->num_tokens * 2 > INT32_MAX / 64) return fail(PKV_ERANGE, "run_mux_round: prompt too long");
  if ((int64_t)pools[0].num_blocks * pools[0].block_size > INT32_MAX)
    return fail(PKV_ERANGE, "run_mux_round: pool too large");
  return PKV_OK;
}

float scale_or_default(float s, int d) { return s > 0.f ? s : 1.0f / std::sqrt((float)d); }

}  // namespace

extern "C" {

int pkv_mux_policy_groups_grid(int total_units, int min_part, int granularity, int min_decode, int group_num,
                               int32_t* prefill_units, int32_t* decode_units, int32_t cap, int32_t* n) {
  if (!n || total_units <= 0 || min_part <= 0 || granularity <= 0 || min_decode < 0 || group_num < 3)
    return fail(PKV_EINVAL, "pkv_mux_policy_groups_grid: bad argument");
  std::vector<std::pair<int, int>> g{{total_units, 0}};
  for (auto& x : split_levels(total_units, min_part, granularity, min_decode, group_num - 2)) g.push_back(x);
  g.emplace_back(0, total_units);
  *n = (int32_t)g.size();
  for (int i = 0; i < *n && i < cap; ++i) {
    if (prefill_units) prefill_units[i] = g[i].first;
    if (decode_units) decode_units[i] = g[i].second;
  }
  return PKV_OK;
}

int pkv_mux_policy_choose(int num_groups, int decode_bs, int has_prefill, int decode_bs_divisor) {
  if (num_groups < 3 || decode_bs < 0 || decode_bs_divisor <= 0) return fail(PKV_EINVAL, "pkv_mux_policy_choose");
  return choose(num_groups, decode_bs, has_prefill != 0, decode_bs_divisor);
}

int pkv_mux_check_decode_step(const pkv_decode_step* d) {
  clear_error();
  std::vector<PoolDev> pools;
  DecodePlan plan{};
  return check_decode_step(d, pools, plan);
}

int pkv_mux_check_prefill_job(const pkv_prefill_job* p) {
  clear_error();
  std::vector<PoolDev> pools;
  return check_prefill_job(p, pools);
}

int pkv_mux_policy_cu_masks(int total_cus, int decode_cus, uint32_t* prefill_words, uint32_t* decode_words,
                            int32_t cap_words) {
  clear_error();
  if (total_cus <= 0 || total_cus > kMaskWords * 32 || total_cus % kXcds)
    return fail(PKV_EUNSUPPORTED, "pkv_mux_policy_cu_masks: %d CUs (a multiple of %d, at most %d)", total_cus, kXcds,
                kMaskWords * 32);
  if (decode_cus <= 0 || decode_cus >= total_cus || decode_cus % kXcds)
    return fail(PKV_EINVAL, "pkv_mux_policy_cu_masks: %d decode CUs (a multiple of %d, 0 < n < %d)", decode_cus,
                kXcds, total_cus);
  if (cap_words < (total_cus + 31) / 32 || !prefill_words || !decode_words)
    return fail(PKV_EINVAL, "pkv_mux_policy_cu_masks: output arrays");
  std::array<uint32_t, kMaskWords> pm, dm;
  build_masks(total_cus, decode_cus, pm, dm);
  for (int i = 0; i < (total_cus + 31) / 32; ++i) {
    prefill_words[i] = pm[i];
    decode_words[i] = dm[i];
  }
  return PKV_OK;
}

int pkv_mux_policy_mask_ok(const uint32_t* words, int32_t nwords, int total_cus) {
  clear_error();
  if (!words || total_cus <= 0 || total_cus > kMaskWords * 32 || total_cus % kXcds || nwords < (total_cus + 31) / 32)
    return fail(PKV_EINVAL, "pkv_mux_policy_mask_ok: bad argument");
  std::array<uint32_t, kMaskWords> m{};
  for (int i = 0; i < (total_cus + 31) / 32; ++i) m[i] = words[i];
  return every_xcd_has_a_cu(m.data(), total_cus) ? 1 : 0;
}

int pkv_mux_policy_layers_per_round(int prefill_tokens, int num_layers, int token_budget) {
  if (prefill_tokens <= 0 || num_layers <= 0 || token_budget <= 0)
    return fail(PKV_EINVAL, "pkv_mux_policy_layers_per_round");
  return std::min(num_layers, std::max(1, token_budget / prefill_tokens));
}

int pkv_mux_create(int device, int cu_granularity, int min_decode_cus, int sm_group_num, int decode_bs_divisor,
                   int token_budget, pkv_mux** out) {
  if (!out) return fail(PKV_EINVAL, "pkv_mux_create: out is NULL");
  *out = nullptr;
  if (cu_granularity <= 0 || min_decode_cus < 0 || sm_group_num < 3 || decode_bs_divisor <= 0 || token_budget <= 0)
    return fail(PKV_EINVAL, "pkv_mux_create: bad policy parameter");
  int cus = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  if (cus > kMaskWords * 32 || cus % kXcds) return fail(PKV_EUNSUPPORTED, "pkv_mux_create: %d CUs", cus);
  if (cus % cu_granularity || cu_granularity % kXcds)
    return fail(PKV_EINVAL, "pkv_mux_create: granularity %d must divide %d CUs and be a multiple of %d", cu_granularity,
                cus, kXcds);
  e = hipSetDevice(device);
  if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  pkv_mux* m = new pkv_mux();
  m->device = device;
  m->total_cus = cus;
  m->granularity = cu_granularity;
  m->min_decode = min_decode_cus;
  m->group_num = sm_group_num;
  m->divisor = decode_bs_divisor;
  m->budget = token_budget;
  m->groups.emplace_back(cus, 0);
  for (auto& g : split_levels(cus, cu_granularity, cu_granularity, min_decode_cus, sm_group_num - 2))
    m->groups.push_back(g);
  m->groups.emplace_back(0, cus);
  const size_t n = m->groups.size();
  m->pmask.resize(n);
  m->dmask.resize(n);
  m->pstream.assign(n, nullptr);
  m->graph_sig.assign(n, {});
  m->graph_exec.assign(n, nullptr);
  m->dstream.assign(n, nullptr);
  for (size_t i = 0; i < n; ++i) build_masks(cus, m->groups[i].second, m->pmask[i], m->dmask[i]);
  e = hipStreamCreateWithFlags(&m->whole, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&m->prefill_done, hipEventDisableTiming);
  if (e != hipSuccess) {
    pkv_mux_destroy(m);
    return hip_fail(e, "pkv_mux_create");
  }
  *out = m;
  return PKV_OK;
}

void pkv_mux_destroy(pkv_mux* m) {
  if (!m) return;
  for (hipGraphExec_t g : m->graph_exec)
    if (g) (void)hipGraphExecDestroy(g);
  for (size_t i = 0; i < m->pstream.size(); ++i) {
    if (m->pstream[i]) { (void)hipStreamSynchronize(m->pstream[i]); (void)hipStreamDestroy(m->pstream[i]); }
    if (m->dstream[i]) { (void)hipStreamSynchronize(m->dstream[i]); (void)hipStreamDestroy(m->dstream[i]); }
  }
  if (m->whole) { (void)hipStreamSynchronize(m->whole); (void)hipStreamDestroy(m->whole); }
  if (m->prefill_done) (void)hipEventDestroy(m->prefill_done);
  delete m;
}

int pkv_mux_groups(const pkv_mux* m, int32_t* prefill_cus, int32_t* decode_cus, int32_t cap, int32_t* n) {
  if (!m || !n) return fail(PKV_EINVAL, "pkv_mux_groups: NULL argument");
  *n = (int32_t)m->groups.size();
  for (int i = 0; i < *n && i < cap; ++i) {
    if (prefill_cus) prefill_cus[i] = m->groups[i].first;
    if (decode_cus) decode_cus[i] = m->groups[i].second;
  }
  return PKV_OK;
}

int pkv_mux_choose(const pkv_mux* m, int decode_bs, int has_prefill) {
  if (!m) return fail(PKV_EINVAL, "pkv_mux_choose: NULL mux");
  return choose_m(m, decode_bs, has_prefill != 0);
}

int pkv_mux_policy_choose_manual(int num_groups, int decode_bs, int has_prefill, const int32_t* thresholds) {
  if (num_groups < 3 || decode_bs < 0 || !thresholds || !valid_thresholds(thresholds, num_groups - 2))
    return fail(PKV_EINVAL, "pkv_mux_policy_choose_manual");
  std::vector<int> t(thresholds, thresholds + num_groups - 2);
  return choose_manual(num_groups, decode_bs, has_prefill != 0, t.data());
}

int pkv_mux_set_manual_divisions(pkv_mux* m, const int32_t* thresholds, int32_t n) {
  if (!m) return fail(PKV_EINVAL, "pkv_mux_set_manual_divisions: NULL mux");
  if (n == 0) {
    m->manual.clear();
    return PKV_OK;
  }
  const int levels = (int)m->groups.size() - 2;
  if (n != levels || !thresholds || !valid_thresholds(thresholds, n))
    return fail(PKV_EINVAL, "pkv_mux_set_manual_divisions: need %d non-decreasing thresholds >= 1", levels);
  m->manual.assign(thresholds, thresholds + n);
  return PKV_OK;
}

int pkv_mux_set_level_override(pkv_mux* m, int level) {
  if (!m) return fail(PKV_EINVAL, "pkv_mux_set_level_override: NULL mux");
  if (level != -1 && (level < 1 || level > (int)m->groups.size() - 2))
    return fail(PKV_EINVAL, "pkv_mux_set_level_override: level %d outside 1..%d", level, (int)m->groups.size() - 2);
  m->override_level = level;
  return PKV_OK;
}

int pkv_mux_layers_per_round(const pkv_mux* m, int prefill_tokens, int num_layers) {
  if (!m || prefill_tokens <= 0 || num_layers <= 0) return fail(PKV_EINVAL, "pkv_mux_layers_per_round: bad argument");
  return std::min(num_layers, std::max(1, m->budget / prefill_tokens));
}

void* pkv_mux_stream(const pkv_mux* mc, int level, int which) {
  pkv_mux* m = const_cast<pkv_mux*>(mc);
  if (!m || level < 0 || level >= (int)m->groups.size() || (which != 0 && which != 1)) return nullptr;
  if (ensure_streams(m, level) != PKV_OK) return nullptr;
  return stream_of(m, level, which);
}

int pkv_mux_cu_mask(const pkv_mux* m, int level, int which, uint32_t* words, int32_t cap, int32_t* n) {
  if (!m || !n || level < 0 || level >= (int)m->groups.size() || (which != 0 && which != 1))
    return fail(PKV_EINVAL, "pkv_mux_cu_mask: bad argument");
  const auto& src = which == 0 ? m->pmask[level] : m->dmask[level];
  *n = kMaskWords;
  for (int i = 0; i < kMaskWords && i < cap; ++i) words[i] = src[i];
  return PKV_OK;
}

namespace {

// Every argument a captured decode step depends on.
std::vector<uint64_t> decode_signature(const pkv_decode_step* d) {
  std::vector<uint64_t> v;
  auto put = [&](uint64_t x) { v.push_back(x); };
  auto ptr = [&](const void* x) { put((uint64_t)(uintptr_t)x); };
  put((uint64_t)d->num_layers);
  for (int l = 0; l < d->num_layers; ++l) {
    const pkv_pool_layer& pl = d->pools[l];
    for (int s = 0; s < PKV_MAX_SHARDS; ++s) {
      ptr(pl.k[s]);
      ptr(pl.v[s]);
    }
    put((uint64_t)pl.num_blocks);
    put((uint64_t)pl.block_size);
    put((uint64_t)pl.num_kv_heads);
    put((uint64_t)pl.num_shards);
    put((uint64_t)pl.head_dim);
    put((uint64_t)pl.dtype);
    ptr(d->q[l]);
    ptr(d->k_new[l]);
    ptr(d->v_new[l]);
    ptr(d->out[l]);
  }
  ptr(d->slots);
  ptr(d->block_tables);
  ptr(d->context_lens);
  ptr(d->workspace);
  put((uint64_t)d->workspace_bytes);
  put((uint64_t)d->bt_stride);
  put((uint64_t)d->batch);
  put((uint64_t)d->max_context_len);
  put((uint64_t)d->num_q_heads);
  uint32_t sb;
  std::memcpy(&sb, &d->scale, sizeof(sb));
  put(sb);
  return v;
}

hipError_t launch_decode_step(const pkv_decode_step* d, const std::vector<PoolDev>& dpools, const DecodePlan& plan,
                              hipStream_t ds, bool append) {
  const float sc = scale_or_default(d->scale, dpools[0].head_dim);
  for (int l = 0; l < d->num_layers; ++l) {
    if (append) {
      // the write and the attention of each layer in one launch (slots unused)
      const hipError_t e = launch_attn_decode(dpools[l], d->pools[l].dtype, d->q[l], d->out[l], d->block_tables,
                                              d->bt_stride, d->context_lens, d->batch, d->num_q_heads, sc, plan,
                                              d->workspace, ds, d->k_new[l], d->v_new[l]);
      if (e != hipSuccess) return e;
      continue;
    }
    hipError_t e = launch_kv_write(dpools[l], d->pools[l].dtype, d->k_new[l], d->v_new[l], d->slots, d->batch, ds);
    if (e == hipSuccess)
      e = launch_attn_decode(dpools[l], d->pools[l].dtype, d->q[l], d->out[l], d->block_tables, d->bt_stride,
                             d->context_lens, d->batch, d->num_q_heads, sc, plan, d->workspace, ds);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Runs the decode step on `ds` as the level's graph, capturing it first when
// there is none or the arguments changed.
hipError_t run_decode_graph(pkv_mux* m, int level, const pkv_decode_step* d, const std::vector<PoolDev>& dpools,
                            const DecodePlan& plan, hipStream_t ds) {
  std::vector<uint64_t> sig = decode_signature(d);
  hipGraphExec_t& exec = m->graph_exec[level];
  if (!exec || m->graph_sig[level] != sig) {
    if (exec) {
      (void)hipGraphExecDestroy(exec);
      exec = nullptr;
    }
    hipError_t e = hipStreamBeginCapture(ds, hipStreamCaptureModeRelaxed);
    if (e != hipSuccess) return e;
    const hipError_t el = launch_decode_step(d, dpools, plan, ds, m->decode_append);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(ds, &graph);
    if (el != hipSuccess || e != hipSuccess) {
      if (graph) (void)hipGraphDestroy(graph);
      return el != hipSuccess ? el : e;
    }
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) {
      exec = nullptr;
      return e;
    }
    m->graph_sig[level] = std::move(sig);
  }
  return hipGraphLaunch(exec, ds);
}

}  // namespace

int pkv_mux_set_decode_graphs(pkv_mux* m, int enable) {
  if (!m) return fail(PKV_EINVAL, "pkv_mux_set_decode_graphs: NULL mux");
  m->use_graphs = enable != 0;
  return PKV_OK;
}

int pkv_mux_set_decode_append(pkv_mux* m, int enable) {
  if (!m) return fail(PKV_EINVAL, "pkv_mux_set_decode_append: NULL mux");
  m->decode_append = enable != 0;
  for (auto& sig : m->graph_sig) sig.clear();   // captured steps hold the other form: capture again
  return PKV_OK;
}

int run_mux_round(pkv_mux* m, const pkv_decode_step* d, pkv_prefill_job* p, int32_t* level_out,
                  int32_t* prefill_done_out) {
  clear_error();
  if (!m) return fail(PKV_EINVAL, "run_mux_round: NULL mux");
  std::vector<PoolDev> dpools, ppools;
  DecodePlan plan{};
  if (d)
    if (int rc = check_decode_step(d, dpools, plan)) return rc;
  if (p)
    if (int rc = check_prefill_job(p, ppools)) return rc;
  const int ng = (int)m->groups.size();
  const int decode_bs = d ? d->batch : 0;
  const bool starting = p && p->next_layer == 0 && !p->submitted_all;
  const bool want_prefill = p && !p->submitted_all;
  hipError_t e = hipSetDevice(m->device);
  if (e != hipSuccess) return hip_fail(e, "hipSetDevice");

  // ---- level: while a prefill is in flight it changes only when the prefill
  // starts or has finished; with no prefill it follows the decode batch ----
  bool rechoose = m->level < 0;
  if (starting && !m->level_with_prefill) rechoose = true;
  if (m->prefill_finished && !want_prefill) rechoose = true;
  if (!want_prefill && !m->level_with_prefill) rechoose = true;
  if (rechoose) {
    int next = choose_m(m, decode_bs, want_prefill);
    if (want_prefill && decode_bs > 0 && m->override_level > 0) next = m->override_level;
    if (next != m->level)
      if (int rc = sync_level(m, m->level)) return rc;    // both streams of the old level drain first
    m->level = next;
    m->level_with_prefill = want_prefill;
    m->prefill_finished = false;
  }
  const int level = m->level;
  if (int rc = ensure_streams(m, level)) return rc;
  hipStream_t ds = stream_of(m, level, 1), ps = stream_of(m, level, 0);

  // ---- decode step on the decode stream (as the level's graph when on) ----
  // on a CU-masked stream a plan of one split per (request, KV head) runs
  // the whole-line kernel: with part of the CUs, half-line K reads and
  // 8-byte V reads limit the bandwidth
  plan.line_k = ds != m->whole && plan.stream_wgs == 0 && plan.num_splits == 1;
  if (d) {
    e = m->use_graphs ? run_decode_graph(m, level, d, dpools, plan, ds)
                      : launch_decode_step(d, dpools, plan, ds, m->decode_append);
    if (e != hipSuccess) return hip_fail(e, "run_mux_round(decode)");
  }
  // ---- next layers of the prefill on the prefill stream ----
  if (want_prefill) {
    const int per_round = std::min(p->num_layers, std::max(1, m->budget / p->num_tokens));
    const int end = std::min(p->num_layers, p->next_layer + per_round);
    const float sc = scale_or_default(p->scale, ppools[0].head_dim);
    for (int l = p->next_layer; l < end; ++l) {
      e = launch_kv_write(ppools[l], p->pools[l].dtype, p->k[l], p->v[l], p->slots, p->num_tokens, ps);
      if (e == hipSuccess)
        e = launch_attn_prefill(ppools[l], p->pools[l].dtype, p->q[l], p->out[l], p->block_table, p->bt_stride,
                                p->start_loc, p->chunk_start, 1, p->num_tokens, p->num_tokens, p->num_q_heads, sc,
                                ps);
      if (e != hipSuccess) return hip_fail(e, "run_mux_round(prefill)");
    }
    p->next_layer = end;
    if (end == p->num_layers) {
      e = hipEventRecord(m->prefill_done, ps);
      if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
      p->submitted_all = 1;
      m->done_pending = true;
    }
  }
  // ---- block on the decode stream only ----
  if (d) {
    e = hipStreamSynchronize(ds);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize(decode)");
  }
  int done = 0;
  if (p && p->submitted_all) {
    if (m->done_pending) {
      e = hipEventQuery(m->prefill_done);
      if (e == hipSuccess) {
        m->done_pending = false;
        m->prefill_finished = true;
        done = 1;
      } else if (e != hipErrorNotReady) {
        return hip_fail(e, "hipEventQuery");
      }
    } else {
      done = 1;
    }
  }
  if (level_out) *level_out = level;
  if (prefill_done_out) *prefill_done_out = done;
  return PKV_OK;
}

int pkv_mux_wait_prefill(pkv_mux* m) {
  if (!m) return fail(PKV_EINVAL, "pkv_mux_wait_prefill: NULL mux");
  if (m->done_pending) {
    hipError_t e = hipEventSynchronize(m->prefill_done);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    m->done_pending = false;
    m->prefill_finished = true;
  }
  return PKV_OK;
}

}  // extern "C"
