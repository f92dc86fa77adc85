/*
 * pkv.h - C ABI of libpkv: paged-KV GQA attention, KV relayout and
 * single-GPU PD multiplexing for AMD Instinct MI355X (gfx950).
 *
 * Pages cited (titles as on the pages):
 *   [MUX]    "PD multiplexing: splitting prefill and decode by SM on one GPU"
 *   [DISAGG] "PD 分离与 KV 传输" (PD disaggregation and KV transfer)
 *   [L7]     "Lecture 7 · Prefill 与 Decode：分块 prefill、解耦与 NVIDIA Dynamo"
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer argument documented as "device" points to device memory
 *   owned by the caller.  The library keeps no pointer after a call returns,
 *   except the multiplexing jobs (see run_mux_round).
 * - Every call except run_mux_round only enqueues work on the given stream
 *   (NULL = the null stream) and returns at once.
 * - Return codes: PKV_OK (0) or a negative PKV_E* code.  Arguments are
 *   validated on the host before any HIP call; on failure nothing is
 *   enqueued.  pkv_last_error() describes the last failure of the calling
 *   thread.  No call throws across the ABI.
 * - Element types: PKV_BF16 (bfloat16, fp32 accumulation, bf16 output
 *   rounded to nearest even) or PKV_F32 (fp32 throughout).
 * - Supported shapes: head_dim 64 or 128; block_size 16, 32, 64 or 128;
 *   num_shards dividing num_kv_heads, at most PKV_MAX_SHARDS; num_q_heads a
 *   multiple of num_kv_heads with at most 16 q-heads per KV head.
 *
 * Pool layout (one layer of one instance)
 * ---------------------------------------
 * The pages view a layer's KV pool as [slot, kv_heads, head_dim] with
 * slot = block_id * block_size + offset ([DISAGG] "实现").  Here the heads
 * of a layer are cut into num_shards contiguous ranges of H/S heads (the
 * TP 4 / TP 8 split of [DISAGG] "布局转换"); shard s stores heads
 * [s*H/S, (s+1)*H/S) as
 *     k[s]: [num_blocks][H/S][block_size][head_dim]   (token rows)
 *     v[s]: [num_blocks][H/S][head_dim][block_size]   (dim-major in a block)
 * so one (block, head) of K or V is one contiguous block_size*head_dim run.
 * V is stored dim-major so that consecutive keys of one dim are adjacent:
 * the P*V product then reads whole 16-byte runs of keys.  All shards of an
 * instance share a request's block table.
 *
 * Out-of-range indices: every kernel checks each block id it reads from a
 * block table against [0, num_blocks) and each slot against the pool; a row
 * with a bad index is skipped (attention treats the key as absent) and, when
 * err_word is non-NULL, the kernel ORs a PKV_ERRBIT_* bit into it.  No bad
 * index is ever dereferenced.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_MAX_SHARDS 16
#define PKV_VERSION 1

enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2 /* kv_relayout_convert destinations only */ };

enum {
  PKV_OK = 0,
  PKV_EINVAL = -1,        /* bad argument, found on the host before any HIP call */
  PKV_EUNSUPPORTED = -2,  /* valid but unsupported shape or element type          */
  PKV_EHIP = -3,          /* a HIP runtime call failed; pkv_last_error names it    */
  PKV_ERANGE = -4         /* a size exceeds a documented limit                     */
};

enum { PKV_ERRBIT_BLOCK_ID = 1, PKV_ERRBIT_SLOT = 2, PKV_ERRBIT_TABLE = 4, PKV_ERRBIT_CONTEXT = 8 };

/* One layer of one instance's paged KV pool (see "Pool layout" above). */
typedef struct pkv_pool_layer {
  void* k[PKV_MAX_SHARDS];   /* device, shard s: [num_blocks][H/S][block_size][head_dim] */
  void* v[PKV_MAX_SHARDS];   /* device, shard s: [num_blocks][H/S][head_dim][block_size] */
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;      /* H, all shards together */
  int32_t num_shards;        /* S */
  int32_t head_dim;
  int32_t dtype;             /* PKV_F32 or PKV_BF16 */
  int32_t* err_word;         /* optional device int32, see "Out-of-range indices" */
} pkv_pool_layer;

/* Description of the last failure on the calling thread ("" if none). */
const char* pkv_last_error(void);

/* PKV_VERSION of the built library. */
int pkv_version(void);

/*
 * pkv_slot_mapping - slot of every token about to be written.
 * [DISAGG] "实现": token p of a request with block table bt lives at
 * slot = bt[p / bs] * bs + p % bs.
 *
 * Tokens are packed request by request: token i of request b (start_loc[b]
 * <= i < start_loc[b+1]) sits at position pos_start[b] + (i - start_loc[b]).
 *   block_tables  device int32 [batch][bt_stride]
 *   start_loc     device int32 [batch + 1], non-decreasing, start_loc[0] = 0,
 *                 start_loc[batch] = num_tokens
 *   pos_start     device int32 [batch]
 *   slots_out     device int32 [num_tokens]; a token whose block-table index
 *                 is past bt_stride or whose block id is out of range gets
 *                 slot -1 (and sets PKV_ERRBIT_TABLE / _BLOCK_ID in err_word).
 *   num_blocks    pool size used for the range check.
 * Decode uses start_loc = 0,1,..,B and pos_start = context_len - 1; a
 * prefill chunk of T tokens at S uses start_loc = {0, T}, pos_start = {S}.
 */
int pkv_slot_mapping(const int32_t* block_tables, int32_t bt_stride, const int32_t* start_loc,
                     const int32_t* pos_start, int32_t batch, int32_t num_tokens, int32_t block_size,
                     int32_t num_blocks, int32_t* slots_out, int32_t* err_word, hipStream_t stream);

/*
 * kv_write - scatter new K/V rows of one layer into the pool.
 * [DISAGG] "实现" (the per-layer write of the admit step): row i of k and v
 * goes to slots[i], every head to its shard.
 *   k, v    device [n_tokens][num_kv_heads][head_dim], element type of the pool
 *   slots   device int32 [n_tokens]; slot < 0 means "skip this row"
 */
int kv_write(const pkv_pool_layer* pool, const void* k, const void* v, const int32_t* slots,
             int32_t n_tokens, hipStream_t stream);

/*
 * kv_relayout - move one layer of one request from a source pool into a
 * destination pool with another block size and/or head-shard split.
 * [DISAGG] self-test answer 3 and "布局转换": gather through the source
 * block table, redistribute by the destination's head split, write at the
 * destination block table's positions.  Submitted once per layer so that a
 * layer can move as soon as it is computed ([DISAGG] "流程").
 *   src_bt  device int32, at least ceil(n_tokens / src->block_size) entries
 *   dst_bt  device int32, at least ceil(n_tokens / dst->block_size) entries
 * Requires equal num_kv_heads, head_dim and dtype.  Only the first n_tokens
 * slots of the destination are written; the destination may hold more
 * blocks (decode reserves room for the next token).  src and dst must not
 * overlap.
 */
int kv_relayout(const pkv_pool_layer* src, const int32_t* src_bt, const pkv_pool_layer* dst,
                const int32_t* dst_bt, int32_t n_tokens, hipStream_t stream);

/*
 * kv_relayout_convert - kv_relayout into a destination that also differs in
 * element type and/or physical layout.  [DISAGG] "布局转换" lists, besides
 * block size and head split, the attention backend's layout (K and V fused
 * or not, the order of the head and token dimensions) and the KV dtype (BF16
 * on one side, FP8 on the other), all best converted on the GPU around the
 * transfer.
 * Destination layouts (per shard s, local head lh, block b, offset o, dim d):
 *   PKV_LAYOUT_POOL        this library's pool: k[s][b][lh][o][d],
 *                          v[s][b][lh][d][o] (readable by the attention calls
 *                          when the dtype is PKV_BF16 or PKV_F32)
 *   PKV_LAYOUT_TOKEN_MAJOR k[s][b][o][lh][d] and v[s][b][o][lh][d] (slot-major
 *                          rows, the pages' [slot, kv_heads, head_dim] view)
 *   PKV_LAYOUT_KV_FUSED    k[s][b][0][o][lh][d] for K and k[s][b][1][o][lh][d]
 *                          for V in one tensor per shard (v[] unused)
 * Element types: the source's dtype, or PKV_FP8_E4M3 from a PKV_BF16 source:
 * OCP E4M3 ("fn": bias 7, no infinities, largest finite 448), stored value =
 * round-to-nearest-even of clamp(x * fp32(1 / scale), -448, 448), the
 * fp32 reciprocal and product being IEEE fp32 operations; the reader
 * multiplies by scale; a NaN input stays a NaN code (0x7F or 0xFF).  scale
 * must be finite and > 0 (ignored without a dtype change).  Tokens at or
 * past n_tokens are not written.  Everything else as kv_relayout (tables,
 * shards, the source's error word, no overlap).
 * Errors: PKV_EINVAL for NULL/misaligned (16 B) buffers, shape mismatch,
 * bad layout or scale; PKV_EUNSUPPORTED for block sizes, shard counts or
 * dtype pairs outside the lists above.
 */
enum { PKV_LAYOUT_POOL = 0, PKV_LAYOUT_TOKEN_MAJOR = 1, PKV_LAYOUT_KV_FUSED = 2 };
typedef struct pkv_kv_dest {
  void* k[PKV_MAX_SHARDS];
  void* v[PKV_MAX_SHARDS];
  int32_t num_blocks;
  int32_t block_size;        /* 16, 32, 64 or 128 */
  int32_t num_kv_heads;
  int32_t num_shards;
  int32_t head_dim;
  int32_t dtype;             /* the source's dtype, or PKV_FP8_E4M3 */
  int32_t layout;            /* PKV_LAYOUT_* */
  float scale;               /* PKV_FP8_E4M3 only */
} pkv_kv_dest;
int kv_relayout_convert(const pkv_pool_layer* src, const int32_t* src_bt, const pkv_kv_dest* dst,
                        const int32_t* dst_bt, int32_t n_tokens, hipStream_t stream);

/*
 * attn_prefill_chunk - causal GQA attention for one chunk of each request.
 * [L7] section 2.3: the queries of a chunk starting at S attend to every key
 * of the earlier chunks and, under a causal mask, to the keys of their own
 * chunk, so chunking is lossless.  Query i of the chunk (absolute position
 * S+i) sees keys [0, S+i]; q-head h reads KV head h / (Hq/Hkv).
 *   q, out        device [sum T][num_q_heads][head_dim], packed request by
 *                 request (start_loc)
 *   block_tables  device int32 [batch][bt_stride]
 *   start_loc     device int32 [batch + 1] offsets of each request's chunk
 *   chunk_start   device int32 [batch] S of each request
 *   max_chunk_len host upper bound of every T (sizes the grid)
 *   max_total_len host upper bound of every S+T: at least max_chunk_len, and
 *                 the table must address it (bt_stride * block_size >=
 *                 max_total_len), else PKV_EINVAL before any launch.  A chunk
 *                 reaching past it attends to keys [0, max_total_len) only
 *                 and sets PKV_ERRBIT_CONTEXT.
 * The chunk's own K/V must already be in the pool (kv_write); keys
 * [0, S+T) are read from the pool only.  scale <= 0 selects 1/sqrt(head_dim).
 */
int attn_prefill_chunk(const pkv_pool_layer* pool, const void* q, void* out, const int32_t* block_tables,
                       int32_t bt_stride, const int32_t* start_loc, const int32_t* chunk_start,
                       int32_t batch, int32_t max_chunk_len, int32_t max_total_len, int32_t num_q_heads,
                       float scale, hipStream_t stream);

/*
 * attn_decode - one query per request over its whole cached context.
 * [L7] section 1.1: each decode step adds one token per request and reads
 * all of its KV.  The query sits at position L-1 and sees keys [0, L) with
 * L = context_lens[b] (its own K/V already written at L-1).
 *   q, out          device [batch][num_q_heads][head_dim]
 *   block_tables    device int32 [batch][bt_stride]
 *   context_lens    device int32 [batch], each in [1, max_context_len]; a
 *                   longer context is cut to its first max_context_len keys
 *                   (every plan and dtype alike) and sets PKV_ERRBIT_CONTEXT
 *   max_context_len host upper bound of every L (sizes the grid); the table
 *                   must address it: bt_stride * block_size >= max_context_len
 *   workspace       device scratch of at least
 *                   pkv_attn_decode_workspace_size(...) bytes for the
 *                   split-KV partial results; caller-owned, may be NULL
 *                   when that size is 0.  Calls that share a workspace must
 *                   be ordered on one stream.
 * scale <= 0 selects 1/sqrt(head_dim).
 * The library picks the work split from the batch, KV-head count,
 * max_context_len and dtype.  With at least 512 (request, KV head) pairs, or
 * contexts short enough, every pair is one workgroup and no workspace is
 * used.  Otherwise fp32 cuts each pair into equal splits of keys, and bf16
 * uses a stream split: one round of workgroups (512, or the environment
 * variable PKV_DECODE_STREAM_WGS, read once) each takes an equal run of
 * 32-key tiles over the whole batch, so uneven contexts leave no idle tail.
 * PKV_DECODE_SPLIT_TOKENS (a multiple of 32, read once) forces equal splits
 * of that many keys, for tuning.  A pair handled by one workgroup is
 * finished by the attention kernel; the partial results of the others are
 * merged by a second kernel on the same stream.
 *
 * Workspace sizes.  pkv_attn_decode_workspace_size_for returns exactly what
 * attn_decode (and attn_decode_append, run_mux_round) need for this pool's
 * KV-head count, head dim and dtype (0 for arguments those calls reject).
 * pkv_attn_decode_workspace_size is told neither the KV-head count nor the
 * dtype, so it returns the largest need over every supported group size
 * (1, 2, 4, 8, 16 q-heads per KV head) and both dtypes: always enough,
 * often more than the call uses.
 */
size_t pkv_attn_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t max_context_len,
                                      int32_t head_dim);
size_t pkv_attn_decode_workspace_size_for(const pkv_pool_layer* pool, int32_t batch, int32_t num_q_heads,
                                          int32_t max_context_len);
int attn_decode(const pkv_pool_layer* pool, const void* q, void* out, const int32_t* block_tables,
                int32_t bt_stride, const int32_t* context_lens, int32_t batch, int32_t max_context_len,
                int32_t num_q_heads, float scale, void* workspace, size_t workspace_bytes,
                hipStream_t stream);

/*
 * attn_decode_noalloc - attn_decode for callers that cannot allocate memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels and results as attn_decode, with the
 * split-KV partial results in a fixed device array of the library instead
 * of a caller workspace.  It calls no allocating routine.
 * Arguments, layouts and errors as attn_decode, without the workspace.  The
 * array holds PKV_DECODE_NOALLOC_SCRATCH_BYTES (16 MiB); a call whose split
 * plan needs more (pkv_attn_decode_workspace_size_for) returns PKV_ERANGE
 * before any HIP call.  Each GPU holds its own copy of the array from the
 * first call on it until the process ends.  Every call on one GPU uses that
 * same array: calls that can overlap on one GPU (on other streams, or graph
 * replays beside other work) race and must not be issued; calls ordered on
 * one stream are safe (no state is kept from one call to the next).
 */
#define PKV_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int attn_decode_noalloc(const pkv_pool_layer* pool, const void* q, void* out, const int32_t* block_tables,
                        int32_t bt_stride, const int32_t* context_lens, int32_t batch, int32_t max_context_len,
                        int32_t num_q_heads, float scale, hipStream_t stream);

/*
 * attn_decode_append - one decode step's K/V append and attention, in one
 * launch for batches with a workgroup per (request, KV head) pair (with the
 * stream split used for fewer pairs, a small kernel writes the rows first).  [DISAGG] "实现" (a decode step writes the new token's K/V at the
 * request's next slot, then attends over all its cached keys) and [L7]
 * section 1.1.  For request b with context L = context_lens[b] (the new
 * token included): the rows k_new[b], v_new[b] ([B, Hkv, D], device,
 * 16-byte aligned) are written at position L-1, slot
 * block_tables[b][(L-1)/bs] * bs + (L-1) % bs, with the same result in the
 * pool as kv_write; and out[b] is attn_decode over keys [0, L), key L-1
 * taken from k_new/v_new (not read back from the pool).  Other arguments,
 * workspace size (pkv_attn_decode_workspace_size) and errors as
 * attn_decode.  A request whose context exceeds max_context_len, or whose
 * slot L-1 lies in a block id outside the pool, has nothing written and
 * sets the error word (PKV_ERRBIT_CONTEXT / PKV_ERRBIT_BLOCK_ID); its
 * output is then attn_decode's (the context cut to max_context_len; a key
 * in a bad block is absent).  The request's
 * slot L-1 must not be read by any other call on another stream meanwhile.
 */
int attn_decode_append(const pkv_pool_layer* pool, const void* q, const void* k_new, const void* v_new, void* out,
                       const int32_t* block_tables, int32_t bt_stride, const int32_t* context_lens, int32_t batch,
                       int32_t max_context_len, int32_t num_q_heads, float scale, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/*
 * Stall-free mixed batch ([L7] section 2.4): each step takes
 * every decoding request first, one token each, and fills what is left of a
 * per-step token budget with prefill chunks, so the step time is bounded and
 * decode never waits behind a prefill.
 *
 * pkv_stall_free_chunk - the chunk a prefill gets in a step:
 * min(prompt_remaining, max(0, token_budget - num_decode)); 0 means the
 * decode requests used the whole budget.  Returns -1 (EINVAL) for a negative
 * argument.
 */
int pkv_stall_free_chunk(int32_t token_budget, int32_t num_decode, int32_t prompt_remaining);
/*
 * pkv_stall_free_batch - the prefill chunks of one stall-free step for
 * several prompts ([L7] section 2.4, steps 2-4): the num_decode decoding
 * requests take one token each first (never dropped, even past the
 * budget); then each prompt, in the order given (the caller lists the
 * unfinished prefills before the newly admitted requests), takes
 * min(its remaining tokens, what is left of token_budget).
 *   prompt_remaining  host int32 [num_prompts], each >= 0
 *   chunks_out        host int32 [num_prompts]: the chunk of each prompt
 * Returns the prefill tokens of the step (sum of chunks_out), or PKV_EINVAL
 * for a negative argument or NULL array.
 */
int pkv_stall_free_batch(int32_t token_budget, int32_t num_decode, const int32_t* prompt_remaining,
                         int32_t num_prompts, int32_t* chunks_out);
/*
 * attn_mixed_batch - one layer of such a batch in a single launch: the
 * decode attention of num_decode requests (arguments as attn_decode) and
 * the prefill attention of num_prefill chunks (arguments as
 * attn_prefill_chunk), the two sharing the pool and num_q_heads.  Decode
 * first is the rule for what enters the batch; inside the launch the
 * prefill workgroups (the long ones) are dispatched first and the decode
 * workgroups fill the device around them, since the step ends with its
 * last workgroup.  The outputs equal those of attn_decode and
 * attn_prefill_chunk called one after the other (to rounding order).  Either part may be empty
 * (num_decode = 0, or num_prefill = 0 / max_chunk_len = 0).  The decode part
 * always uses equal splits of the context (the workspace needed is at most
 * pkv_attn_decode_workspace_size(num_decode, ...)); when it needs more than
 * one split, a merge kernel follows on the same stream.  bf16 runs one fused
 * kernel; fp32 runs the two kernels back to back.  The chunks' own K/V must
 * be written (kv_write) before the call.
 */
int attn_mixed_batch(const pkv_pool_layer* pool, const void* q_dec, void* out_dec, const int32_t* dec_block_tables,
                     int32_t dec_bt_stride, const int32_t* context_lens, int32_t num_decode, int32_t max_context_len,
                     const void* q_pf, void* out_pf, const int32_t* pf_block_tables, int32_t pf_bt_stride,
                     const int32_t* start_loc, const int32_t* chunk_start, int32_t num_prefill,
                     int32_t max_chunk_len, int32_t max_total_len, int32_t num_q_heads, float scale,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * PD multiplexing on one GPU ([MUX] "SGLang's PD multiplexing").
 *
 * The device's compute units are cut into split levels: prefill gets x CUs
 * and decode the rest, x on a grid of cu_granularity, prefill at least half,
 * decode at least min_decode_cus; sm_group_num - 2 levels are kept, evenly
 * spaced.  Group 0 runs everything on the whole device as prefill, the last
 * group as decode.  A split level is a pair of HIP streams created with
 * complementary CU masks (hipExtStreamCreateWithCUMask), the local analogue
 * of a green-context SM split.  The level follows the decode batch size:
 * clamp(decode_bs * levels / decode_bs_divisor, 1, levels) when both
 * phases are present.  Prefill advances token_budget / prompt_tokens layers
 * per round (at least one).
 * ------------------------------------------------------------------------- */
typedef struct pkv_mux pkv_mux;

/* The policy alone, as pure host functions (no device, no streams): the
 * split levels of `total_units` units on a grid of `granularity` (also the
 * minimum part), decode keeping at least `min_decode` units; then the group
 * index for a decode batch, and the layers per round of a prompt.  The
 * pages' SM tables follow from the same rule with (total, minimum part,
 * granularity) = (132, 8, 8), (108, 4, 2), (78, 8, 8) and min_decode 16;
 * pkv_mux_policy_groups_grid takes the minimum part separately for them. */
int pkv_mux_policy_groups_grid(int total_units, int min_part, int granularity, int min_decode, int group_num,
                               int32_t* prefill_units, int32_t* decode_units, int32_t cap, int32_t* n);
int pkv_mux_policy_choose(int num_groups, int decode_bs, int has_prefill, int decode_bs_divisor);
int pkv_mux_policy_layers_per_round(int prefill_tokens, int num_layers, int token_budget);
/* The CU masks of a split, as pkv_mux_create builds them ("Green contexts:
 * carving out SMs for a stream" in [MUX]: a stream bound to a subset of the
 * compute units).  MI355X sends mask bit i to CU i / 8 of XCD i % 8, so
 * decode takes the lowest decode_cus / 8 CUs of every XCD and prefill the
 * rest: both queues keep CUs on every XCD.  decode_cus must be a multiple
 * of 8 with 0 < decode_cus < total_cus; writes ceil(total_cus / 32) words
 * each.  PKV_EINVAL / PKV_EUNSUPPORTED on a bad argument. */
int pkv_mux_policy_cu_masks(int total_cus, int decode_cus, uint32_t* prefill_words, uint32_t* decode_words,
                            int32_t cap_words);
/* 1 if a CU mask (bit i = CU i / 8 of XCD i % 8) keeps at least one CU on
 * every XCD, else 0 (such a mask can never run the workgroups dispatched to
 * the XCD it leaves empty: pkv_mux_create and run_mux_round refuse it);
 * PKV_EINVAL on a bad argument. */
int pkv_mux_policy_mask_ok(const uint32_t* words, int32_t nwords, int total_cus);

/* Builds the CU-masked stream pairs of every level on `device`.  The total
 * CU count is the device's; cu_granularity must divide it. */
int pkv_mux_create(int device, int cu_granularity, int min_decode_cus, int sm_group_num,
                   int decode_bs_divisor, int token_budget, pkv_mux** out);
void pkv_mux_destroy(pkv_mux* mux);
/* (prefill CUs, decode CUs) of each group; *n = group count (<= cap written). */
int pkv_mux_groups(const pkv_mux* mux, int32_t* prefill_cus, int32_t* decode_cus, int32_t cap, int32_t* n);
/* Group index the policy picks. */
int pkv_mux_choose(const pkv_mux* mux, int decode_bs, int has_prefill);
/* Layers per round for a prompt of prefill_tokens tokens. */
int pkv_mux_layers_per_round(const pkv_mux* mux, int prefill_tokens, int num_layers);
/* Fixes the level used while a prefill runs (1 .. group count - 2), in
 * place of the batch-size rule; -1 restores the rule.  For level sweeps. */
int pkv_mux_set_level_override(pkv_mux* mux, int level);
/* Manual divisions ([MUX] "SGLang's PD multiplexing", level choice and its
 * exercise): thresholds[i-1] is the decode batch size from which split
 * level i is used (n = group count - 2 values, non-decreasing, >= 1); below
 * the first threshold level 1.  It replaces the decode_bs_divisor rule while
 * set; n = 0 restores the rule.  Decode only and prefill only still use the
 * whole device.  pkv_mux_policy_choose_manual is the same rule without a
 * mux (num_groups - 2 thresholds).  -1 (EINVAL) on a bad argument. */
int pkv_mux_set_manual_divisions(pkv_mux* mux, const int32_t* thresholds, int32_t n);
/* Per-level decode graphs ([MUX] "SGLang's PD multiplexing": a CUDA-graph
 * state for each level): with enable != 0, run_mux_round captures the
 * decode step (every layer's kv_write and attn_decode) as one HIP graph on
 * the level's decode stream the first time it runs there, and replays it
 * while the decode step's arguments (every pointer and size of
 * pkv_decode_step and its pools) stay the same; a change recaptures.
 * Results are those of the plain launches.  Off by default; the graphs are
 * released by pkv_mux_destroy. */
int pkv_mux_set_decode_graphs(pkv_mux* mux, int enable);
/* Decode step in append form: with enable != 0, each layer of the decode
 * step is one attn_decode_append launch (the new rows go to position L-1
 * of each request through its block table; pkv_decode_step.slots is not
 * used) instead of kv_write + attn_decode.  Off by default.  Captured
 * decode graphs are captured again.  -1 (EINVAL) on a NULL mux. */
int pkv_mux_set_decode_append(pkv_mux* mux, int enable);
int pkv_mux_policy_choose_manual(int num_groups, int decode_bs, int has_prefill, const int32_t* thresholds);
/* Stream of a group: which = 0 prefill, 1 decode (a hipStream_t). */
void* pkv_mux_stream(const pkv_mux* mux, int level, int which);
/* The 32-bit words of a group's CU mask (which = 0 prefill, 1 decode). */
int pkv_mux_cu_mask(const pkv_mux* mux, int level, int which, uint32_t* words, int32_t cap, int32_t* n);

/* One decode step of a batch over all layers: per layer, write the new
 * token's K/V at its slot, then decode attention. Host arrays of per-layer
 * device pointers. */
typedef struct pkv_decode_step {
  int32_t num_layers;
  const pkv_pool_layer* pools;     /* host [num_layers] */
  const void* const* q;            /* host [num_layers] of device [B][Hq][D] */
  const void* const* k_new;        /* host [num_layers] of device [B][Hkv][D] */
  const void* const* v_new;
  void* const* out;                /* host [num_layers] of device [B][Hq][D] */
  const int32_t* slots;            /* device [B] slot of each request's new token */
  const int32_t* block_tables;     /* device [B][bt_stride] */
  int32_t bt_stride;
  const int32_t* context_lens;     /* device [B] */
  int32_t batch;
  int32_t max_context_len;
  int32_t num_q_heads;
  float scale;
  void* workspace;                 /* device, pkv_attn_decode_workspace_size bytes */
  size_t workspace_bytes;
} pkv_decode_step;

/* A whole-prompt prefill cut by layer ([MUX]: prefill runs layers
 * [start, end) per round).  next_layer is the cursor the library advances. */
typedef struct pkv_prefill_job {
  int32_t num_layers;
  const pkv_pool_layer* pools;     /* host [num_layers] */
  const void* const* q;            /* host [num_layers] of device [N][Hq][D] */
  const void* const* k;            /* host [num_layers] of device [N][Hkv][D] */
  const void* const* v;
  void* const* out;                /* host [num_layers] of device [N][Hq][D] */
  const int32_t* slots;            /* device [N] */
  const int32_t* block_table;      /* device [1][bt_stride] */
  int32_t bt_stride;
  const int32_t* start_loc;        /* device [2] = {0, N} */
  const int32_t* chunk_start;      /* device [1] = {0} */
  int32_t num_tokens;              /* N */
  int32_t num_q_heads;
  float scale;
  int32_t next_layer;              /* in/out: first layer not yet submitted */
  int32_t submitted_all;           /* out: 1 once every layer is enqueued */
} pkv_prefill_job;

/*
 * run_mux_round - one round of the multiplexing loop ([MUX] "SGLang's PD
 * multiplexing", the main loop).  Enqueues the decode step `d` on the
 * decode stream of the current level, then the next layers of `p` on the
 * prefill stream, records the prefill-done event after the last layer, and
 * blocks on the decode stream only.  The level is re-chosen (after syncing
 * both streams of the old level) only when a prefill starts or finishes.
 * Either d or p may be NULL.  The job and every buffer it names must stay
 * alive until *prefill_done_out is 1 or pkv_mux_wait_prefill returns.
 *   level_out          group index used this round
 *   prefill_done_out   1 once the last prefill layer has finished on the GPU
 */
int run_mux_round(pkv_mux* mux, const pkv_decode_step* d, pkv_prefill_job* p, int32_t* level_out,
                  int32_t* prefill_done_out);
/* Blocks until every submitted prefill layer has finished. */
int pkv_mux_wait_prefill(pkv_mux* mux);

/* The host validation run_mux_round applies to a decode step / prefill job,
 * alone (no device work, no mux): every layer's pool valid and equal in
 * shape to layer 0's (dtype, KV heads, head dim, block size, shards,
 * blocks), every per-layer tensor non-NULL and 16-byte aligned, q-heads a
 * supported multiple of the KV heads, scale finite and >= 0, the block
 * table wide enough for max_context_len (decode) or the prompt (prefill),
 * and the decode workspace at least the plan's size.  PKV_OK or the code
 * run_mux_round would return. */
int pkv_mux_check_decode_step(const pkv_decode_step* d);
int pkv_mux_check_prefill_job(const pkv_prefill_job* p);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
