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
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kXcds = 8;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Row of the 32-key half tile that lane row m of the S^T MFMA's A operand
// holds: chosen so that accumulator registers 8s..8s+7 of a lane in half
// h = lane/32 are keys 16s + 8h + 0..7.
__device__ __forceinline__ int key_perm(int m) {
  return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

template <int D>
struct PrefillCfg {
  static constexpr int BM = 128, BN = 64, THREADS = 256;
  static constexpr int KS = D / 16;     // MFMA k-steps of q.k
  static constexpr int DT = D / 32;     // 32-dim output tiles
  static constexpr int KROW = D + 8;    // LDS K row stride (elements)
  static constexpr int VROW = BN + 8;   // LDS V^T row stride (elements)
  static constexpr int GROUPS = BN / 16;            // 16-key groups per tile (each inside one block)
  static constexpr int KLANES = D / 8;              // lanes per K row in a group load
  static constexpr int KACTIVE = 16 * KLANES;       // threads that load K rows of a group (256 for D=128)
  static constexpr int SK = BN * KROW;              // one K buffer (elements)
  static constexpr int SV = D * VROW;               // one V buffer
};

// Running max update rule: the max used for exp2 moves only when a tile's
// max exceeds it by more than this (log2 units), so p <= 2^8 and the O
// accumulators are rescaled rarely.
constexpr float kRescaleSlack = 8.0f;

template <int D>
__global__ void __launch_bounds__(256, 2)
attn_prefill_bf16_kernel(PoolDev pool, const bf16_t* __restrict__ q, bf16_t* __restrict__ out,
                         const int32_t* __restrict__ bt, int bt_stride, const int32_t* __restrict__ start_loc,
                         const int32_t* __restrict__ chunk_start, int batch, int ntiles, int num_q_heads,
                         int group, float scale_log2, int total_items) {
  using C = PrefillCfg<D>;
  // double-buffered K and V^T tiles
  __shared__ __attribute__((aligned(16))) bf16_t sk[2 * C::SK];
  __shared__ __attribute__((aligned(16))) bf16_t sv[2 * C::SV];

  // ---- work item (XCD-contiguous runs) ----
  const int per_xcd = gridDim.x / kXcds;
  const int item = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (item >= total_items) return;
  const int per_kvh = ntiles * group * batch;
  const int kvh = item / per_kvh;
  int rem = item - kvh * per_kvh;
  const int qt = ntiles - 1 - rem / (group * batch);
  rem %= group * batch;
  const int g = rem / batch;
  const int b = rem - g * batch;
  const int h = kvh * group + g;

  const int q0 = start_loc[b];
  const int T = start_loc[b + 1] - q0;
  if (qt * C::BM >= T) return;
  const int S = chunk_start[b];
  const int kv_len = min(S + T, bt_stride << pool.bs_shift);
  if (S + T > (bt_stride << pool.bs_shift) && threadIdx.x == 0) flag_error(pool.err, PKV_ERRBIT_TABLE);
  const int kend = min(kv_len, S + min(T, (qt + 1) * C::BM));   // one past the last query's position

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);    // wave-uniform (lets branches on it stay scalar)
  const int half = lane >> 5, l32 = lane & 31;
  const int hl = pool.heads_per_shard;
  const int sh = kvh / hl, lh = kvh - sh * hl;
  const bf16_t* kpool = reinterpret_cast<const bf16_t*>(pool.k[sh]);
  const bf16_t* vpool = reinterpret_cast<const bf16_t*>(pool.v[sh]);
  const int bs = pool.block_size;
  const size_t tile_stride = (size_t)bs * D;                     // elements per (block, head) tile
  const size_t head_off = (size_t)lh * tile_stride;
  const size_t block_stride = (size_t)hl * tile_stride;
  const int32_t* table = bt + (size_t)b * bt_stride;

  // ---- this lane's query row and its Q fragments (B operand of S^T) ----
  const int qrel = qt * C::BM + wave * 32 + l32;
  const int qpos = S + qrel;
  uint4 qf[C::KS];
  {
    const bool ok = qrel < T;
    const bf16_t* qrow = q + ((size_t)(q0 + (ok ? qrel : 0)) * num_q_heads + h) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) qf[s] = ok ? *reinterpret_cast<const uint4*>(qrow + 16 * s) : make_uint4(0, 0, 0, 0);
  }
  const int wave_first_q = S + qt * C::BM + wave * 32;

  // ---- tile loader.  Group r of a tile is keys 16r..16r+15, which lie in one
  // block: its block id is uniform, so each group is read through a buffer
  // descriptor on that block's (block, head) tile and a lane adds only its
  // fixed offset.  K: thread t loads row t / KLANES of the group, dims
  // (t % KLANES) * 8 (threads >= KACTIVE idle for D = 64).  V: thread t loads
  // dim t >> 1, keys 8 * (t & 1) of the dim-major tile.  A group with a bad
  // block id (or wholly past the request) gets a zero-size descriptor, reads
  // zeros, and its bit in the returned mask marks its keys absent. ----
  const int k_row = tid / C::KLANES, k_col = (tid % C::KLANES) * 8;
  const int k_row_perm = key_perm(k_row);     // LDS row of this key (key_perm is its own inverse)
  const int v_dim = tid >> 1, v_key = (tid & 1) * 8;
  const bool k_act = C::KACTIVE >= C::THREADS || tid < C::KACTIVE;
  const bool v_act = 2 * D >= C::THREADS || v_dim < D;
  const int k_voff = (k_row * D + k_col) * 2, v_voff = (v_dim * bs + v_key) * 2;   // bytes
  const int tile_bytes = bs * D * 2;
  uint4 rk[C::GROUPS], rv[C::GROUPS];
  auto load_tile = [&](int kt) -> uint32_t {
    const int kbase = kt * C::BN;
    int blk[C::GROUPS];
#pragma unroll
    for (int r = 0; r < C::GROUPS; ++r) {
      const int key16 = kbase + 16 * r;
      blk[r] = key16 < kv_len ? __builtin_amdgcn_readfirstlane(table[key16 >> pool.bs_shift]) : -1;
    }
    uint32_t absent = 0;
#pragma unroll
    for (int r = 0; r < C::GROUPS; ++r) {
      const int key16 = kbase + 16 * r;
      const bool ok = blk[r] >= 0 && blk[r] < pool.num_blocks;      // uniform
      if (!ok) {
        absent |= 1u << r;
        if (key16 < kv_len && tid == 0) flag_error(pool.err, PKV_ERRBIT_BLOCK_ID);
      }
      const size_t tbase = ok ? (size_t)blk[r] * block_stride + head_off : 0;
      const int off = key16 & (bs - 1);
      const buffer_rsrc_t rsk = buffer_rsrc(kpool + tbase, ok ? tile_bytes : 0);
      const buffer_rsrc_t rsv = buffer_rsrc(vpool + tbase, ok ? tile_bytes : 0);
      if (k_act) rk[r] = buffer_load16(rsk, k_voff, off * D * 2);
      if (v_act) rv[r] = buffer_load16(rsv, v_voff, off * 2);
    }
    // the request's last tile: keys past kv_len hold arbitrary bits; their
    // scores are masked by causality, their V entries must be zero (p = 0
    // times a NaN pattern would still poison the sum)
    if (kbase + C::BN > kv_len && v_act) {
#pragma unroll
      for (int r = 0; r < C::GROUPS; ++r) {
        const int nvalid = kv_len - (kbase + 16 * r) - v_key;
        uint32_t* w = reinterpret_cast<uint32_t*>(&rv[r]);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e >= nvalid) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
      }
    }
    return absent;
  };
  auto store_tile = [&](int buf) {
    bf16_t* kb = sk + buf * C::SK;
    bf16_t* vb = sv + buf * C::SV;
#pragma unroll
    for (int r = 0; r < C::GROUPS; ++r) {
      if (k_act) *reinterpret_cast<uint4*>(&kb[(16 * r + k_row_perm) * C::KROW + k_col]) = rk[r];
      if (v_act) *reinterpret_cast<uint4*>(&vb[v_dim * C::VROW + 16 * r + v_key]) = rv[r];
    }
  };

  f32x16_t o[C::DT];
#pragma unroll
  for (int t = 0; t < C::DT; ++t) o[t] = f32x16_t{};
  // running max (log2 units): finite start, so a tile whose keys are all
  // masked or absent gives p = exp2(-inf) = 0 rather than exp2(-inf + inf)
  float m = -1e30f, lsum = 0.f;

  const int nkt = (kend + C::BN - 1) / C::BN;
  uint32_t absent = load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    uint32_t absent_next = 0;
    if (kt + 1 < nkt) absent_next = load_tile(kt + 1);   // in flight during this tile's math
    const bf16_t* kb = sk + buf * C::SK;
    const bf16_t* vb = sv + buf * C::SV;
    const int kbase = kt * C::BN;
    // ---- S^T = K Q^T over two 32-key halves ----
    // all K fragments are read before the first MFMA so the LDS latency is
    // paid once per tile, not once per MFMA
    f32x16_t st[2];
    uint4 kf[2][C::KS];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const bf16_t* krow = &kb[(32 * i + l32) * C::KROW + 8 * half];
#pragma unroll
      for (int s = 0; s < C::KS; ++s) kf[i][s] = *reinterpret_cast<const uint4*>(krow + 16 * s);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      st[i] = f32x16_t{};
#pragma unroll
      for (int s = 0; s < C::KS; ++s) st[i] = mfma32(kf[i][s], qf[s], st[i]);
    }
    // schedule: 8 reads ahead, then one read behind each MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int j = 0; j < 2 * C::KS - 8; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    // ---- causal mask (only where the tile reaches past this wave's first query) ----
    if (kbase + C::BN - 1 > wave_first_q) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kbase + 32 * i + 16 * (r >> 3) + 8 * half + (r & 7);
          if (key > qpos) st[i][r] = -INFINITY;
        }
    }
    // ---- keys of groups with a bad block id are absent ----
    if (absent) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if ((absent >> (2 * i + (r >> 3))) & 1) st[i][r] = -INFINITY;
    }
    // ---- online softmax for query l32 (keys split over lanes l and l^32) ----
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(st[i][r], st[i][r + 1]));
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2;
    // move the running max only when this tile exceeds it by the slack
    const bool grow = mx > m + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {         // wave-uniform branch
      const float mnew = grow ? mx : m;
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);     // 0 on the first tile
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int t = 0; t < C::DT; ++t) o[t] *= alpha;
    }
    // p in bf16 (the MFMA operand); the row sum adds those same rounded
    // values, two per v_dot2 against (1, 1)
    constexpr uint32_t kOnes = 0x3F803F80u;
    float psum[2] = {0.f, 0.f};
    uint4 pf[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(st[i][8 * sp + e], scale_log2, -m));
        pf[i][sp] = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                               pack_bf16x2(p[6], p[7]));
        psum[sp] = dot2_bf16(pf[i][sp].x, kOnes, psum[sp]);
        psum[sp] = dot2_bf16(pf[i][sp].y, kOnes, psum[sp]);
        psum[sp] = dot2_bf16(pf[i][sp].z, kOnes, psum[sp]);
        psum[sp] = dot2_bf16(pf[i][sp].w, kOnes, psum[sp]);
      }
    lsum += psum[0] + psum[1];
    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
#pragma unroll
        for (int t = 0; t < C::DT; ++t) {
          const uint4 va = *reinterpret_cast<const uint4*>(&vb[(32 * t + l32) * C::VROW + 32 * i + 16 * sp + 8 * half]);
          o[t] = mfma32(va, pf[i][sp], o[t]);
        }
      }
    if (kt + 1 < nkt) store_tile(buf ^ 1);           // the other buffer was last read before the previous barrier
    absent = absent_next;
    __syncthreads();
  }

  // ---- normalise and store: lane holds dims 32t + 8a + 4*half + 0..3 of its query ----
  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (qrel < T) {
    const float inv = 1.f / ltot;
    bf16_t* orow = out + ((size_t)(q0 + qrel) * num_q_heads + h) * D;
#pragma unroll
    for (int t = 0; t < C::DT; ++t)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const uint2 w = make_uint2(pack_bf16x2(o[t][4 * a] * inv, o[t][4 * a + 1] * inv),
                                   pack_bf16x2(o[t][4 * a + 2] * inv, o[t][4 * a + 3] * inv));
        *reinterpret_cast<uint2*>(orow + 32 * t + 8 * a + 4 * half) = w;
      }
  }
}

// fp32: one wave per (query row, q-head); lane owns head-dim columns.
template <int D>
__global__ void __launch_bounds__(256)
attn_prefill_f32_kernel(PoolDev pool, const float* __restrict__ q, float* __restrict__ out,
                        const int32_t* __restrict__ bt, int bt_stride, const int32_t* __restrict__ start_loc,
                        const int32_t* __restrict__ chunk_start, int max_chunk_len, int num_q_heads, int group,
                        float scale_log2) {
  constexpr int DPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);     // query row within the chunk
  const int h = blockIdx.y, b = blockIdx.z;
  const int q0 = start_loc[b];
  const int T = start_loc[b + 1] - q0;
  if (row >= T || row >= max_chunk_len) return;
  const int S = chunk_start[b];
  const int pos = S + row;
  if (pos >= (bt_stride << pool.bs_shift)) {
    if (lane == 0) flag_error(pool.err, PKV_ERRBIT_TABLE);
    return;
  }
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
  for (int key = 0; key <= pos; ++key) {
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
                               int max_chunk_len, int num_q_heads, float scale, hipStream_t s) {
  if (batch == 0 || max_chunk_len == 0) return hipSuccess;
  const int group = num_q_heads / pool.num_kv_heads;
  const float sl2 = scale * kLog2e;
  if (dtype == PKV_BF16) {
    constexpr int BM = 128;
    const int ntiles = (max_chunk_len + BM - 1) / BM;
    const int items = pool.num_kv_heads * ntiles * group * batch;
    const int grid = (items + kXcds - 1) / kXcds * kXcds;
    if (pool.head_dim == 128)
      hipLaunchKernelGGL(attn_prefill_bf16_kernel<128>, dim3(grid), dim3(256), 0, s, pool,
                         static_cast<const bf16_t*>(q), static_cast<bf16_t*>(out), bt, bt_stride, start_loc,
                         chunk_start, batch, ntiles, num_q_heads, group, sl2, items);
    else
      hipLaunchKernelGGL(attn_prefill_bf16_kernel<64>, dim3(grid), dim3(256), 0, s, pool,
                         static_cast<const bf16_t*>(q), static_cast<bf16_t*>(out), bt, bt_stride, start_loc,
                         chunk_start, batch, ntiles, num_q_heads, group, sl2, items);
    return hipGetLastError();
  }
  const dim3 grid((max_chunk_len + 3) / 4, num_q_heads, batch);
  if (pool.head_dim == 128)
    hipLaunchKernelGGL(attn_prefill_f32_kernel<128>, grid, dim3(256), 0, s, pool, static_cast<const float*>(q),
                       static_cast<float*>(out), bt, bt_stride, start_loc, chunk_start, max_chunk_len, num_q_heads,
                       group, sl2);
  else
    hipLaunchKernelGGL(attn_prefill_f32_kernel<64>, grid, dim3(256), 0, s, pool, static_cast<const float*>(q),
                       static_cast<float*>(out), bt, bt_stride, start_loc, chunk_start, max_chunk_len, num_q_heads,
                       group, sl2);
  return hipGetLastError();
}

}  // namespace pkv
