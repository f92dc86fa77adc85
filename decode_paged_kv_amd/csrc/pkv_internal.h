// Internal declarations shared by the HIP kernels and the C-ABI glue of
// libpkv.  Nothing here is part of the public ABI (include/pkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/pkv.h"

namespace pkv {

// Pool of one layer as passed to kernels (by value, in the kernarg segment).
struct PoolDev {
  char* k[PKV_MAX_SHARDS];
  char* v[PKV_MAX_SHARDS];
  int num_blocks;
  int block_size;
  int bs_shift;          // log2(block_size); block sizes are powers of two
  int heads_per_shard;
  int num_kv_heads;
  int head_dim;
  int32_t* err;          // optional error word (nullptr = none)
};

// bfloat16 is carried as raw 16-bit patterns in device buffers.
typedef uint16_t bf16_t;

#ifdef __HIPCC__
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float x) {
  __bf16 b = static_cast<__bf16>(x);
  return __builtin_bit_cast(bf16_t, b);
}
// Two floats to a bf16 pair (lo in bits 0-15), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
}
// c + a.lo*b.lo + a.hi*b.hi over bf16 pairs, fp32 accumulate (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a), __builtin_bit_cast(bf16x2_v, b), c, false);
}
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u32x4_t global_u32x4_t;
// 16-byte non-temporal store (the data is not read back soon).  The cast to
// the global address space keeps it a global_store rather than a flat one.
__device__ __forceinline__ void store_nt16(void* p, const uint4& v) {
  u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, (global_u32x4_t*)p);
}
// 16-byte non-temporal load: streamed data that this kernel reads once.
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4_t w = __builtin_nontemporal_load((const global_u32x4_t*)p);
  return make_uint4(w.x, w.y, w.z, w.w);
}
// Raw buffer view of one contiguous range whose base and size are
// wave-uniform: the descriptor sits in scalar registers and a lane adds only
// a 32-bit offset, so a load costs no vector address arithmetic.  Bytes past
// `bytes` read as zero (bytes = 0: every load reads zero, nothing is touched).
// Descriptor word 3 = untyped 32-bit elements (the gfx9 raw-buffer setting).
typedef __amdgpu_buffer_rsrc_t buffer_rsrc_t;
__device__ __forceinline__ buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
// cache policy of a buffer load: kCached for data other workgroups re-read
// through L2, kStream (the nt bit) for data read once
enum { kCached = 0, kStream = 2 };
template <int POLICY = kCached>
__device__ __forceinline__ uint4 buffer_load16(buffer_rsrc_t r, int voffset, int soffset) {
  const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(r, voffset, soffset, POLICY);
  return make_uint4(w.x, w.y, w.z, w.w);
}
template <int POLICY = kCached>
__device__ __forceinline__ uint2 buffer_load8(buffer_rsrc_t r, int voffset, int soffset) {
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(r, voffset, soffset, POLICY);
  return make_uint2(w.x, w.y);
}
__device__ __forceinline__ void flag_error(int32_t* err, int bit) {
  if (err) atomicOr(err, bit);
}
// Base offset (in elements) of the (block, local head) tile of a shard:
// K and V tiles both hold block_size * head_dim elements.
__device__ __forceinline__ size_t tile_elems(const PoolDev& p, int blk, int local_head) {
  return ((size_t)blk * p.heads_per_shard + local_head) * ((size_t)p.block_size * p.head_dim);
}
#endif

// ---- launchers (each validates nothing: the ABI layer has done it) ----
hipError_t launch_slot_mapping(const int32_t* bt, int bt_stride, const int32_t* start_loc, const int32_t* pos_start,
                               int batch, int num_tokens, int block_size, int num_blocks, int32_t* slots,
                               int32_t* err, hipStream_t s);
hipError_t launch_kv_write(const PoolDev& pool, int dtype, const void* k, const void* v, const int32_t* slots,
                           int n_tokens, hipStream_t s);
hipError_t launch_kv_relayout(const PoolDev& src, const int32_t* src_bt, const PoolDev& dst, const int32_t* dst_bt,
                              int dtype, int n_tokens, hipStream_t s);
hipError_t launch_kv_relayout_convert(const PoolDev& src, const int32_t* src_bt, const pkv_kv_dest& dst,
                                      int heads_per_shard, const int32_t* dst_bt, int src_dtype, int n_tokens,
                                      int32_t* err, hipStream_t s);

struct DecodePlan {
  int max_len;        // max_context_len: longer contexts are cut to it and flagged
  int split_tokens;   // keys per split (multiple of 32); split plan only
  int num_splits;     // splits per (request, kv head) at max_context_len; split plan only
  int stream_wgs;     // > 0: stream split over this many workgroups instead
  bool line_k;        // bf16, one split per pair: the whole-line K kernel
                      // (for a launch on part of the CUs); false from
                      // plan_decode
  size_t workspace;   // bytes of partial results needed (0: none)
};
// stream_ok = false: never the stream split (equal splits instead)
DecodePlan plan_decode(int batch, int num_q_heads, int num_kv_heads, int max_context_len, int head_dim, int dtype,
                       bool stream_ok = true);
// the merge kernel of an equal-splits plan (no-op for other plans)
hipError_t launch_decode_split_merge(const PoolDev& pool, int dtype, void* out, const int32_t* ctx, int bt_stride,
                                     int batch, int num_q_heads, const DecodePlan& plan, void* workspace,
                                     hipStream_t s);
// k_new / v_new non-null: append mode (each request's new K/V row written
// at position L-1 and used for that key; see attn_decode_append)
hipError_t launch_attn_decode(const PoolDev& pool, int dtype, const void* q, void* out, const int32_t* bt,
                              int bt_stride, const int32_t* ctx, int batch, int num_q_heads, float scale,
                              const DecodePlan& plan, void* workspace, hipStream_t s, const void* k_new = nullptr,
                              const void* v_new = nullptr);
hipError_t launch_attn_prefill(const PoolDev& pool, int dtype, const void* q, void* out, const int32_t* bt,
                               int bt_stride, const int32_t* start_loc, const int32_t* chunk_start, int batch,
                               int max_chunk_len, int max_total_len, int num_q_heads, float scale, hipStream_t s);
// decode (plan made with stream_ok = false) and prefill chunks of one layer
// in one launch (bf16), decode workgroups first; fp32 runs the two kernels
struct MixedDecode {
  const void* q;
  void* out;
  const int32_t* bt;
  int bt_stride;
  const int32_t* ctx;
  int batch;
  DecodePlan plan;
  void* workspace;
};
struct MixedPrefill {
  const void* q;
  void* out;
  const int32_t* bt;
  int bt_stride;
  const int32_t* start_loc;
  const int32_t* chunk_start;
  int batch;
  int max_chunk_len;
  int max_total_len;
};
hipError_t launch_attn_mixed(const PoolDev& pool, int dtype, const MixedDecode& d, const MixedPrefill& p,
                             int num_q_heads, float scale, hipStream_t s);

}  // namespace pkv
