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
  // the destination and source block ids are read together (the source
  // ids do not wait for the destination id's check)
  const int dblk = dst_bt[j];
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
  if (dblk < 0 || dblk >= dst.num_blocks) {
    if (threadIdx.x == 0) flag_error(dst.err, PKV_ERRBIT_BLOCK_ID);
    return;
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

// ------------------------------------------------------ relayout + convert ----
// One workgroup per (destination block j of the request, head), as
// kv_relayout, for a destination that may differ in element type (bf16 ->
// OCP E4M3 with a per-tensor scale) and layout (pool, token-major, K/V
// fused).  Every global load is a 16-byte run of the source: K runs are
// VEC dims of one token row, V runs are VEC tokens of one dim row (V is
// dim-major in the source pool).  K runs map to token rows on every
// destination, and so do V runs on the pool layout (dim rows there too).
// For the token-major layouts, V is turned round in LDS: the dim-row runs
// of up to 32 tokens are written into a token-major LDS tile, then read
// back as VEC-dim runs of one token and stored, so both the loads and the
// stores stay 16-byte runs (8-byte for E4M3).  Each thread issues its loads
// of a round before converting and storing.
struct ConvDest {
  char* k[PKV_MAX_SHARDS];
  char* v[PKV_MAX_SHARDS];
  int num_blocks, block_size, heads_per_shard, head_dim, layout, esize;
  float inv_scale;
  int32_t* err;
};

// x * inv clamped to the largest finite E4M3 magnitude; NaN stays NaN (tested
// on the bits: the library is built without NaN semantics for comparisons)
__device__ __forceinline__ float fp8_sat(float x, float inv) {
  const float f = x * inv;
  const bool nan = (__float_as_uint(f) & 0x7fffffffu) > 0x7f800000u;
  return nan ? f : fminf(fmaxf(f, -448.f), 448.f);
}

__device__ __forceinline__ uint8_t fp8_byte(float x, float inv) {
  return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(fp8_sat(x, inv), 0.f, 0, false) & 0xff);
}

// VEC source values -> destination bytes at dst (E4M3 when FP8); streamed stores
template <typename T, bool FP8>
__device__ __forceinline__ void store_run(char* dst, const T (&x)[16 / sizeof(T)], float inv) {
  constexpr int VEC = 16 / sizeof(T);
  if constexpr (FP8) {
    static_assert(VEC == 8, "E4M3 from bf16 only");
    uint32_t w[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float f[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) f[j] = fp8_sat(bf16_to_f32(x[4 * i + j]), inv);
      const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      w[i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
    }
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(1))) u32x2_t global_u32x2_t;
    const u32x2_t v = {w[0], w[1]};
    __builtin_nontemporal_store(v, (global_u32x2_t*)dst);
  } else {
    uint4 v;
    __builtin_memcpy(&v, x, 16);
    store_nt16(dst, v);
  }
}

// one element (ragged tails)
template <typename T, bool FP8>
__device__ __forceinline__ void store_one(char* dst, T x, float inv) {
  if constexpr (FP8) *reinterpret_cast<uint8_t*>(dst) = fp8_byte(bf16_to_f32(x), inv);
  else *reinterpret_cast<T*>(dst) = x;
}

constexpr int kConvTc = 32;         // tokens per chunk (and rows of the LDS transpose tile)

template <typename T, bool FP8, int LAYOUT>
__global__ void __launch_bounds__(kThreads)
kv_relayout_convert_kernel(PoolDev src, const int32_t* __restrict__ src_bt, ConvDest dst,
                           const int32_t* __restrict__ dst_bt, int n_tokens) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int ES = FP8 ? 1 : sizeof(T);           // destination element bytes
  constexpr int LPAD = 8 / sizeof(T);              // 8-byte row pad of the LDS tile
  constexpr bool kPoolV = LAYOUT == PKV_LAYOUT_POOL;
  // 16-byte runs per thread per chunk, K and V each, at the largest head dim
  constexpr int kConvNpt = kConvTc * 128 * (int)sizeof(T) / 16 / kThreads;
  __shared__ int sblk[128 / 16];
  __shared__ __align__(16) T vt[kPoolV ? 1 : kConvTc * (128 + LPAD)];
  const int j = blockIdx.x, h = blockIdx.y;
  const int D = dst.head_dim;
  const int bsd = dst.block_size, bss = src.block_size;
  const int p0 = j * bsd;
  const int valid = min(bsd, n_tokens - p0);
  // the destination and source block ids are read together (the source
  // ids do not wait for the destination id's check)
  const int dblk = dst_bt[j];
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
  if (dblk < 0 || dblk >= dst.num_blocks) {
    if (threadIdx.x == 0) flag_error(dst.err, PKV_ERRBIT_BLOCK_ID);
    return;
  }
  __syncthreads();
  const int hsd = dst.heads_per_shard;
  const int dsh = h / hsd, dlh = h - dsh * hsd;
  const int ssh = h / src.heads_per_shard, slh = h - ssh * src.heads_per_shard;
  const T* sk = reinterpret_cast<const T*>(src.k[ssh]);
  const T* sv = reinterpret_cast<const T*>(src.v[ssh]);
  const size_t stile = (size_t)bss * D;
  const int off0 = p0 & (bss - 1);
  const float inv = dst.inv_scale;
  // destination byte offset of element (token o, dim d) of K (kv = 0) or V (kv = 1)
  auto dst_off = [&](int kv, int o, int d) -> size_t {
    if constexpr (LAYOUT == PKV_LAYOUT_POOL) {
      const size_t tile = ((size_t)dblk * hsd + dlh) * ((size_t)bsd * D);
      return (tile + (kv ? (size_t)d * bsd + o : (size_t)o * D + d)) * ES;
    } else {
      const size_t row = LAYOUT == PKV_LAYOUT_KV_FUSED ? ((size_t)dblk * 2 + kv) * bsd + o : (size_t)dblk * bsd + o;
      return ((row * hsd + dlh) * D + d) * ES;
    }
  };
  // source element offsets of (span token r, dim d): K rows, V dim rows
  auto src_k = [&](int b, int r, int d) {
    return ((size_t)b * src.heads_per_shard + slh) * stile + (size_t)(r & (bss - 1)) * D + d;
  };
  auto src_v = [&](int b, int r, int d) {
    return ((size_t)b * src.heads_per_shard + slh) * stile + (size_t)d * bss + (r & (bss - 1));
  };
  char* dk = dst.k[dsh];
  char* dv = LAYOUT == PKV_LAYOUT_KV_FUSED ? dst.k[dsh] : dst.v[dsh];
  const int rpt_shift = __builtin_ctz(D / VEC);    // runs per token row (K)
  const int tc = min(bsd, kConvTc);                // tokens per chunk
  const int vpk_shift = __builtin_ctz(tc / VEC);   // runs per dim row of a chunk (V)
  const int ldsr = D + LPAD;
  // Chunks of tc tokens.  Every load of a chunk (K rows, V dim rows, ragged
  // tail elements) is issued and consumed before its first store, and the
  // stores come last: a wait for a load issued after a store would also wait
  // for the store.
  for (int t0 = 0; t0 < valid; t0 += tc) {
    const int nt = min(tc, valid - t0);
    const int nk = nt << rpt_shift, nvr = D << vpk_shift;
    uint4 kw[kConvNpt], vw[kConvNpt];
    int kb[kConvNpt], vn[kConvNpt];                // K: source block (-1: none); V: elements present
#pragma unroll
    for (int u = 0; u < kConvNpt; ++u) {
      const int e = threadIdx.x + u * kThreads;
      {
        const int o = e >> rpt_shift, d = (e & ((1 << rpt_shift) - 1)) * VEC;
        const int b = e < nk ? sblk[(off0 + t0 + o) >> src.bs_shift] : -1;
        kb[u] = b;
        kw[u] = b >= 0 ? load_nt16(sk + src_k(b, off0 + t0 + o, d)) : make_uint4(0, 0, 0, 0);
      }
      {
        const int d = e >> vpk_shift, o = (e & ((1 << vpk_shift) - 1)) * VEC;
        const int b = (e < nvr && o < nt) ? sblk[(off0 + t0 + o) >> src.bs_shift] : -1;
        vn[u] = b >= 0 ? min(VEC, nt - o) : 0;
        vw[u] = vn[u] == VEC ? load_nt16(sv + src_v(b, off0 + t0 + o, d)) : make_uint4(0, 0, 0, 0);
        if (vn[u] > 0 && vn[u] < VEC) {            // ragged tail of the request: element loads
          const T* sp = sv + src_v(b, off0 + t0 + o, d);
          T x[VEC];
#pragma unroll
          for (int i = 0; i < VEC; ++i) x[i] = i < vn[u] ? sp[i] : T(0);
          __builtin_memcpy(&vw[u], x, 16);
        }
      }
    }
    if constexpr (!kPoolV) {
      // V dim-row runs -> the LDS tile vt[token][dim] -> token-row runs
#pragma unroll
      for (int u = 0; u < kConvNpt; ++u) {
        if (vn[u] == 0) continue;
        const int e = threadIdx.x + u * kThreads;
        const int d = e >> vpk_shift, o = (e & ((1 << vpk_shift) - 1)) * VEC;
        T x[VEC];
        __builtin_memcpy(x, &vw[u], 16);
#pragma unroll
        for (int i = 0; i < VEC; ++i) vt[(o + i) * ldsr + d] = x[i];   // rows past nt are never read
      }
      __syncthreads();
      for (int e = threadIdx.x; e < nk; e += kThreads) {
        const int o = e >> rpt_shift, d = (e & ((1 << rpt_shift) - 1)) * VEC;
        if (sblk[(off0 + t0 + o) >> src.bs_shift] < 0) continue;
        T x[VEC];
        const uint2* lp = reinterpret_cast<const uint2*>(&vt[o * ldsr + d]);
        const uint2 a = lp[0], c = lp[1];
        __builtin_memcpy(x, &a, 8);
        __builtin_memcpy(reinterpret_cast<char*>(x) + 8, &c, 8);
        store_run<T, FP8>(dv + dst_off(1, t0 + o, d), x, inv);
      }
    } else {
      // V dim-row runs -> the pool layout's dim rows
#pragma unroll
      for (int u = 0; u < kConvNpt; ++u) {
        if (vn[u] == 0) continue;
        const int e = threadIdx.x + u * kThreads;
        const int d = e >> vpk_shift, o = (e & ((1 << vpk_shift) - 1)) * VEC;
        T x[VEC];
        __builtin_memcpy(x, &vw[u], 16);
        if (vn[u] == VEC) {
          store_run<T, FP8>(dv + dst_off(1, t0 + o, d), x, inv);
        } else {
#pragma unroll
          for (int i = 0; i < VEC; ++i)
            if (i < vn[u]) store_one<T, FP8>(dv + dst_off(1, t0 + o + i, d), x[i], inv);
        }
      }
    }
    // K: token rows -> token rows
#pragma unroll
    for (int u = 0; u < kConvNpt; ++u) {
      if (kb[u] < 0) continue;
      const int e = threadIdx.x + u * kThreads;
      const int o = e >> rpt_shift, d = (e & ((1 << rpt_shift) - 1)) * VEC;
      T x[VEC];
      __builtin_memcpy(x, &kw[u], 16);
      store_run<T, FP8>(dk + dst_off(0, t0 + o, d), x, inv);
    }
    if (!kPoolV && t0 + tc < valid) __syncthreads();   // the tile is rewritten by the next chunk
  }
}

template <typename T, bool FP8>
void launch_convert_layout(int layout, dim3 grid, hipStream_t s, const PoolDev& src, const int32_t* src_bt,
                           const ConvDest& cd, const int32_t* dst_bt, int n_tokens) {
  if (layout == PKV_LAYOUT_POOL)
    hipLaunchKernelGGL((kv_relayout_convert_kernel<T, FP8, PKV_LAYOUT_POOL>), grid, dim3(kThreads), 0, s, src,
                       src_bt, cd, dst_bt, n_tokens);
  else if (layout == PKV_LAYOUT_TOKEN_MAJOR)
    hipLaunchKernelGGL((kv_relayout_convert_kernel<T, FP8, PKV_LAYOUT_TOKEN_MAJOR>), grid, dim3(kThreads), 0, s, src,
                       src_bt, cd, dst_bt, n_tokens);
  else
    hipLaunchKernelGGL((kv_relayout_convert_kernel<T, FP8, PKV_LAYOUT_KV_FUSED>), grid, dim3(kThreads), 0, s, src,
                       src_bt, cd, dst_bt, n_tokens);
}

}  // namespace

hipError_t launch_kv_relayout_convert(const PoolDev& src, const int32_t* src_bt, const pkv_kv_dest& dst,
                                      int heads_per_shard, const int32_t* dst_bt, int src_dtype, int n_tokens,
                                      int32_t* err, hipStream_t s) {
  if (n_tokens == 0) return hipSuccess;
  ConvDest cd{};
  for (int i = 0; i < PKV_MAX_SHARDS; ++i) {
    cd.k[i] = static_cast<char*>(dst.k[i]);
    cd.v[i] = static_cast<char*>(dst.v[i]);
  }
  cd.num_blocks = dst.num_blocks;
  cd.block_size = dst.block_size;
  cd.heads_per_shard = heads_per_shard;
  cd.head_dim = dst.head_dim;
  cd.layout = dst.layout;
  cd.esize = dst.dtype == PKV_FP8_E4M3 ? 1 : (src_dtype == PKV_BF16 ? 2 : 4);
  cd.inv_scale = dst.dtype == PKV_FP8_E4M3 ? 1.0f / dst.scale : 1.0f;
  cd.err = err;
  const dim3 grid((n_tokens + dst.block_size - 1) / dst.block_size, dst.num_kv_heads);
  if (dst.dtype == PKV_FP8_E4M3)
    launch_convert_layout<bf16_t, true>(dst.layout, grid, s, src, src_bt, cd, dst_bt, n_tokens);
  else if (src_dtype == PKV_BF16)
    launch_convert_layout<bf16_t, false>(dst.layout, grid, s, src, src_bt, cd, dst_bt, n_tokens);
  else
    launch_convert_layout<float, false>(dst.layout, grid, s, src, src_bt, cd, dst_bt, n_tokens);
  return hipGetLastError();
}

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
