// bf16 paged GQA decode attention for one workgroup, the whole-line form,
// used where the decode runs on part of the device's CUs (a CU-masked
// stream beside a prefill).  One workgroup per (KV head, request), all of
// the request's keys, as decode_bf16.h does for such batches, whose work
// decomposition, softmax and merge this form shares.  What differs is how a
// tile's K and V reach the matrix cores.
//
// decode_bf16.h loads K straight in the S^T operand layout: one instruction
// reads 64 bytes of each of 16 key rows, so every 128-byte line takes two
// instructions; and V 8 bytes per lane.  On half of the CUs each CU needs
// twice the bandwidth and such requests limit it: a loads-only probe reads
// about 4.1 TB/s with that pattern, 4.8 with K in whole lines and 5.0 with V
// at 16 bytes per lane as well; on the whole device HBM is the limit and
// the direct form is faster (it needs no LDS round trip).  Here K is loaded
// in whole key rows, each instruction 1 KB of whole 128-byte lines, and
// turned into the operand layout through a 32-key LDS tile the wave owns
// (written, then read back).  A row's 16-byte chunk c is stored at position
// c ^ swz(row), so the 16 rows one operand read touches fall in distinct
// banks.  The rows each S^T MFMA takes are chosen so that a lane's
// accumulators hold 8 consecutive keys of the tile, the layout in which a
// 16x16x32 P V MFMA takes P; its V operand is then 8 consecutive keys of one
// dim row, one 16-byte load per lane (an instruction reads 512 contiguous
// bytes from each of the tile's two blocks).  Both carry the non-temporal
// hint.
//
// A tile's registers are refilled with the wave's next tile as soon as they
// are consumed: K right after it is written to LDS, V right after P V, so
// two tiles per wave are in flight.  The 4 waves merge (m, l, acc) through
// LDS at the end, in passes of at most 8 KB (the K tiles take 8 KB per
// wave at head dim 128).
#pragma once

#include "decode_bf16.h"

namespace pkv {
namespace decode_line {

using decode_impl::bf16x8_t;
using decode_impl::col_max;
using decode_impl::col_sum;
using decode_impl::f32x4_t;
using decode_impl::kDecodeSlack;
using decode_impl::kThreads;
using decode_impl::kWaves;

__device__ __forceinline__ f32x4_t mfma_qk(const u32x4_t& a, const u32x4_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_pv(const u32x4_t& a, const u32x4_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// The loads of a tile's operands (q, K, V), the LDS transposition of K and
// the waits that guard them are written out: the waits the compiler derives
// for registers loaded one loop iteration ahead are stricter than the issue
// order needs and would leave one tile in flight per wave instead of two.
// Each wait names the registers it makes valid, so no use of a loaded value
// can be scheduled before it.
// A wave's loads into registers complete in issue order, so a wait for at
// most N loads in flight makes valid every load issued before the last N.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
__device__ __forceinline__ void lds_write16(char* p, const u32x4_t& v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ u32x4_t lds_read16(const char* p) {
  u32x4_t v;
  const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(a) : "memory");
  return v;
}
// the eight (four) reads of one tile's K operands have returned
__device__ __forceinline__ void wait_lds8(u32x4_t (&k)[8]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(k[0]), "+v"(k[1]), "+v"(k[2]), "+v"(k[3]), "+v"(k[4]), "+v"(k[5]), "+v"(k[6]), "+v"(k[7])
               :
               : "memory");
}
__device__ __forceinline__ void wait_lds4(u32x4_t (&k)[4]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(k[0]), "+v"(k[1]), "+v"(k[2]), "+v"(k[3]) : : "memory");
}
// A buffer descriptor built from values that are the same in every lane
// (a tile's block id, its pool and head), said so to the compiler so the
// descriptor lives in scalar registers, as the load instructions need.
__device__ __forceinline__ buffer_rsrc_t buffer_rsrc_uniform(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return buffer_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), __builtin_amdgcn_readfirstlane(bytes));
}
// 16 bytes per lane of a buffer, non-temporal; valid after a wait naming it
__device__ __forceinline__ void vload16_nt(u32x4_t& v, buffer_rsrc_t r, int voffset, int soffset) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen nt" : "+v"(v) : "v"(voffset), "s"(r), "s"(soffset) : "memory");
}
// 16 bytes per lane from a global address; valid after a wait naming it
__device__ __forceinline__ void gload16(u32x4_t& v, const void* p) {
  asm volatile("global_load_dwordx4 %0, %1, off" : "+v"(v) : "v"(p) : "memory");
}
// the same, non-temporal
__device__ __forceinline__ void gload16_nt(u32x4_t& v, const void* p) {
  asm volatile("global_load_dwordx4 %0, %1, off nt" : "+v"(v) : "v"(p) : "memory");
}
// waits that make a tile's V registers (DT) or q's fragments valid
template <int N>
__device__ __forceinline__ void wait_vm_v(u32x4_t (&v)[8]) {
  asm volatile("s_waitcnt vmcnt(%8)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
               : "n"(N)
               : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm_v(u32x4_t (&v)[4]) {
  asm volatile("s_waitcnt vmcnt(%4)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]) : "n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm_k(u32x4_t (&k)[8]) {
  asm volatile("s_waitcnt vmcnt(%8)"
               : "+v"(k[0]), "+v"(k[1]), "+v"(k[2]), "+v"(k[3]), "+v"(k[4]), "+v"(k[5]), "+v"(k[6]), "+v"(k[7])
               : "n"(N)
               : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm_k(u32x4_t (&k)[4]) {
  asm volatile("s_waitcnt vmcnt(%4)" : "+v"(k[0]), "+v"(k[1]), "+v"(k[2]), "+v"(k[3]) : "n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm_q(u32x4_t (&q)[4]) {
  asm volatile("s_waitcnt vmcnt(%4)" : "+v"(q[0]), "+v"(q[1]), "+v"(q[2]), "+v"(q[3]) : "n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm_q(u32x4_t (&q)[2]) {
  asm volatile("s_waitcnt vmcnt(%2)" : "+v"(q[0]), "+v"(q[1]) : "n"(N) : "memory");
}

// One 32-key tile's K rows (as loaded: whole rows, 1 KB per instruction),
// its V operands and its two block ids (-1: absent).
template <int D>
struct LineTile {
  u32x4_t k[32 * 2 * D / 1024];   // instruction i, lane t: row RPI i + t / NCH, chunk (t % NCH) ^ swz(row)
  u32x4_t v[D / 16];              // A of O^T: dim 16m + l%16, keys 8(l/16) .. +7 of the tile
  int blk[2];
};

// The K tile in LDS: row q of a tile is key q (2D bytes), its 16-byte chunk c
// at position c ^ swz(q), swz(q) = (cr(q) >> SWS) & (NCH - 1) with
// cr(q) = (q & 3) | ((q >> 3) << 2).  The S^T MFMA of key set h reads rows
// 8(r / 4) + 4h + r % 4 for r = 0..15, whose cr values are the 16 distinct
// r: with 256-byte rows (D = 128) each row is a whole bank window, with
// 128-byte rows (D = 64) two rows share one, and either way the 16 rows of
// an operand read hit 16 distinct 16-byte bank groups.
template <int D>
struct LineKCfg {
  static constexpr int NCH = D / 8;                 // 16-byte chunks per row
  static constexpr int ROWB = 2 * D;                // bytes per row
  static constexpr int TILE = 32 * ROWB;            // one 32-key tile
  static constexpr int RPI = 1024 / ROWB;           // rows per 1 KB load instruction
  static constexpr int NLD = 32 / RPI;              // K load instructions per tile
  static constexpr int SWS = NCH == 16 ? 0 : 1;
  static constexpr int REGION = kWaves * TILE;      // the tile of every wave
  static __device__ __forceinline__ int swz(int q) { return (((q & 3) | ((q >> 3) << 2)) >> SWS) & (NCH - 1); }
};
static_assert(LineKCfg<128>::RPI * LineKCfg<128>::NLD == 32 && LineKCfg<64>::RPI * LineKCfg<64>::NLD == 32,
              "K tile loads");

// The 4-wave merge stages at most 8 KB of accumulators at a time: DC dims of
// every q-head per pass.
template <int D, int G>
struct LineMerge {
  static constexpr int DC = (512 / G) < D ? 512 / G : D;
  static constexpr int PASSES = D / DC;
  static_assert(DC % 16 == 0 && D % DC == 0, "merge passes");
};

template <int D, int G>
struct LineSmem {
  float acc[kWaves][G][LineMerge<D, G>::DC];
  float m[kWaves][G];
  float l[kWaves][G];
  float snew[G];            // score of the appended key, per q-head (log2 units)
};

// One workgroup's work: every key of (request b, KV head kvh), one split
// per pair, so the workgroup writes the output rows itself.  kregion:
// LineKCfg<D>::REGION bytes of LDS (1 KB aligned), the K tile of every wave.
template <int D, int G, bool APPEND>
__device__ __forceinline__ void decode_line_block(PoolDev pool, const bf16_t* __restrict__ q,
                                                  bf16_t* __restrict__ out, const int32_t* __restrict__ bt,
                                                  int bt_stride, const int32_t* __restrict__ ctx, int num_q_heads,
                                                  float scale_log2, int max_len, const bf16_t* __restrict__ k_new,
                                                  const bf16_t* __restrict__ v_new, int kvh, int b,
                                                  char* const kregion, LineSmem<D, G>& sm) {
  static_assert(G >= 1 && G <= 16, "the q-heads of a KV head are the 16 MFMA columns");
  constexpr int KC = D / 32, DT = D / 16, TK = 32;
  using KCF = LineKCfg<D>;
  using MG = LineMerge<D, G>;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, j4 = lane >> 4;
  // keys a request may have: max_context_len, which the host has checked
  // against the table's capacity; a longer context is cut to it and flagged
  const int cap = max_len;
  const int hl = pool.heads_per_shard;
  const int bs = pool.block_size;
  const size_t block_stride = (size_t)hl * bs * D;
  const int tile_bytes = bs * D * 2;

  // The workgroup's keys [start, end) of request b and KV head kvh.  With
  // `last` (append mode) the request's new key L-1 follows them: its K/V
  // come from k_new / v_new, are added to the softmax in the merge, and are
  // written to the pool there; the tiles stop at L-1.
  struct Seg {
    int b, kvh, start, end;
    bool last;
  };
  // its KV head's pools, its table, its end (wave-uniform, in scalar
  // registers)
  const bf16_t* kpool = nullptr;
  const bf16_t* vpool = nullptr;
  size_t head_off = 0;                                          // elements
  const int32_t* table = bt;
  int end = 0;
  // q as the B operand of S^T: head l16 (zero columns past G), dims 32c + 8 j4
  u32x4_t qf[KC];
  auto bind = [&](const Seg& sg) {
    const int sh = sg.kvh / hl, lh = sg.kvh - sh * hl;
    kpool = reinterpret_cast<const bf16_t*>(pool.k[sh]);
    vpool = reinterpret_cast<const bf16_t*>(pool.v[sh]);
    head_off = (size_t)lh * bs * D;
    table = bt + (size_t)sg.b * bt_stride;
    end = sg.end;
    // every lane loads (a lane past G a valid row, zeroed once it lands)
    const bf16_t* qrow = q + ((size_t)sg.b * num_q_heads + (size_t)sg.kvh * G + (l16 < G ? l16 : 0)) * D + 8 * j4;
#pragma unroll
    for (int c = 0; c < KC; ++c) gload16(qf[c], qrow + 32 * c);
  };

  // V of lane l: dim l16 of a 16-dim slab, keys 8 j4 .. +7 of the tile: the
  // 8-key run 8 (j4 % 2) of key half j4 / 2
  const int v_lane = l16 * bs + 8 * (j4 & 1);                   // elements from the half's first key
  // this wave's K tile in LDS
  char* const ktile = kregion + wave * KCF::TILE;
  // K loads: instruction i reads rows RPI i .. +RPI-1 (all in key half
  // RPI i / 16); lane t reads the chunk (t % NCH) ^ swz(row) of row
  // RPI i + t / NCH, which it then writes to position t % NCH of that row in
  // LDS, i.e. to byte 1024 i + 16 t of the tile
  int kdma_voff[KCF::NLD];
#pragma unroll
  for (int i = 0; i < KCF::NLD; ++i) {
    const int row = KCF::RPI * i + lane / KCF::NCH;
    const int c = (lane % KCF::NCH) ^ KCF::swz(row);
    kdma_voff[i] = ((row & 15) * D + 8 * c) * 2;
  }
  // S^T MFMA h takes the keys 8(r / 4) + 4h + r % 4 as its rows r = 0..15,
  // so that its accumulator rows 4 j4 .. +3 are keys 8 j4 + 4h .. +3 and a
  // lane ends up with keys 8 j4 .. +7 of the tile for its head, the layout
  // in which P V takes P.  K operand read of lane l for set h: that row,
  // chunk 4c + j4 at position (4c + j4) ^ swz(row) = byte offset kx[h] ^ 64c
  int kx[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 8 * (l16 >> 2) + 4 * h + (l16 & 3);
    const int ksw = KCF::swz(row);
    kx[h] = row * KCF::ROWB + 16 * (j4 ^ (ksw & 3)) + 64 * (ksw >> 2);
  }
  // block ids of the tile at k0 (-1: past the context or out of range)
  auto fetch_ids = [&](int k0, int (&ids)[2]) {
    bool bad = false;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int key16 = k0 + 16 * h;
      const int blk = key16 < end ? table[key16 >> pool.bs_shift] : -1;
      const bool ok = blk >= 0 && blk < pool.num_blocks;
      bad |= key16 < end && !ok;
      // the id is wave-uniform; saying so keeps the descriptors built from
      // it in scalar registers
      ids[h] = __builtin_amdgcn_readfirstlane(ok ? blk : -1);
    }
    if (bad && lane == 0) flag_error(pool.err, PKV_ERRBIT_BLOCK_ID);
  };
  // K rows of the tile at k0 (an absent block's rows read zeros)
  auto issue_k = [&](int k0, LineTile<D>& r) {
#pragma unroll
    for (int i = 0; i < KCF::NLD; ++i) {
      const int h = (KCF::RPI * i) >> 4;
      const bool ok = r.blk[h] >= 0;
      const buffer_rsrc_t rs = buffer_rsrc_uniform(kpool + (ok ? (size_t)r.blk[h] * block_stride + head_off : 0),
                                                   ok ? tile_bytes : 0);
      const int soff = __builtin_amdgcn_readfirstlane(((k0 + 16 * h) & (bs - 1)) * D * 2);
      vload16_nt(r.k[i], rs, kdma_voff[i], soff);
    }
  };
  // V of the tile at k0: one 16-byte load per lane and 16-dim slab, lanes
  // j4 < 2 from key half 0's block, the others from half 1's (an absent
  // block's lanes read block 0 of the pool, in bounds, and are zeroed before
  // use)
  auto issue_v = [&](int k0, LineTile<D>& r) {
    const int h = j4 >> 1;
    const int blk = h ? r.blk[1] : r.blk[0];
    const bf16_t* vp = vpool + head_off + v_lane +
                       (blk >= 0 ? (size_t)blk * block_stride + ((k0 + 16 * h) & (bs - 1)) : 0);
#pragma unroll
    for (int mm = 0; mm < DT; ++mm) gload16_nt(r.v[mm], vp + (size_t)mm * 16 * bs);
  };

  f32x4_t o[DT];
  // running max of head l16 (log2 units; finite start, so a tile whose keys
  // are all absent gives p = exp2(-inf) = 0) and this lane's share of the sum
  float m = -1e30f, lsum = 0.f;
  constexpr uint32_t kOnes = 0x3F803F80u;       // bf16 (1, 1)

  // one tile: S^T, softmax, P V; the registers are refilled with the tile
  // at k0_next (< 0: none) as they are consumed, whose block ids were read
  // one tile earlier into ids_next; then the ids of the tile at k0_next2
  int ids_next[2] = {-1, -1};
  // Every tile step issues the loads of its register set's next tile, an
  // absent one (past the segment) through a descriptor with no records that
  // reads zeros and touches no memory, and the prologue loads both sets.  So
  // every path issues the same sequence of loads and each wait names a fixed
  // count: after a tile's K loads come its V loads (DT) and the other set's
  // next tile (NLD + DT); after its V loads, that other tile and this set's
  // next K loads (NLD).  Loads into registers complete in issue order.  (A
  // wait inside a branch would let the compiler copy the named registers
  // before it; loads whose destination is not kept live would let it reuse
  // the register while the load is in flight.)
  auto process = [&](int k0, LineTile<D>& r, int k0_next, int k0_next2) {
    wait_vm_k<2 * DT + KCF::NLD>(r.k);
    // K rows into the LDS tile, then back in the operand layout (one wave's
    // LDS operations complete in order)
#pragma unroll
    for (int i = 0; i < KCF::NLD; ++i) lds_write16(ktile + i * 1024 + 16 * lane, r.k[i]);
    u32x4_t kf[2 * KC];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < KC; ++c) kf[h * KC + c] = lds_read16(ktile + (kx[h] ^ (64 * c)));
    if constexpr (KC == 4)
      wait_lds8(kf);
    else
      wait_lds4(kf);
    f32x4_t st[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      st[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) st[h] = mfma_qk(kf[h * KC + c], qf[c], st[h]);
    }
    // this lane's keys 8 j4 .. +7 lie in key half j4 / 2
    const bool okh = (j4 < 2 ? r.blk[0] : r.blk[1]) >= 0;
    const bool has_next = k0_next >= 0;
    __builtin_amdgcn_sched_barrier(0);
    r.blk[0] = has_next ? ids_next[0] : -1;
    r.blk[1] = has_next ? ids_next[1] : -1;
    issue_k(has_next ? k0_next : 0, r);
    if (has_next && k0_next2 >= 0) fetch_ids(k0_next2, ids_next);
    __builtin_amdgcn_sched_barrier(0);
    float x[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = k0 + 8 * j4 + 4 * h + rr;
        const bool valid = key < end && okh;
        x[h][rr] = valid ? st[h][rr] : -INFINITY;
        mx = fmaxf(mx, x[h][rr]);
      }
    mx = col_max(mx) * scale_log2;
    const bool grow = mx > m + kDecodeSlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {          // wave-uniform branch
      const float mnew = grow ? mx : m;
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int mm = 0; mm < DT; ++mm) o[mm] *= alpha;
    }
    // P of keys 8 j4 .. +7 (set 0's four, then set 1's), the B operand of P V
    u32x4_t pb;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float p[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) p[rr] = __builtin_amdgcn_exp2f(fmaf(x[h][rr], scale_log2, -m));
      pb[2 * h] = pack_bf16x2(p[0], p[1]);
      pb[2 * h + 1] = pack_bf16x2(p[2], p[3]);
      lsum = dot2_bf16(pb[2 * h], kOnes, lsum);       // the sum of the same bf16 p the MFMA uses
      lsum = dot2_bf16(pb[2 * h + 1], kOnes, lsum);
    }
    // this tile's V
    wait_vm_v<2 * KCF::NLD + DT>(r.v);
    // V entries of keys past the context (the request's last tile) and of an
    // absent block hold arbitrary bits and must be zero (p = 0 times a NaN
    // pattern is NaN).  Each lane masks its 8 keys (all kept before the last
    // tile): no branch, so the compiler needs no copies of the V registers.
    {
      const int nvalid = okh ? end - (k0 + 8 * j4) : 0;
      u32x4_t mk;
#pragma unroll
      for (int i = 0; i < 4; ++i) mk[i] = nvalid >= 2 * i + 2 ? 0xFFFFFFFFu : nvalid == 2 * i + 1 ? 0x0000FFFFu : 0u;
#pragma unroll
      for (int mm = 0; mm < DT; ++mm) r.v[mm] &= mk;
    }
#pragma unroll
    for (int mm = 0; mm < DT; ++mm) o[mm] = mfma_pv(r.v[mm], pb, o[mm]);
    __builtin_amdgcn_sched_barrier(0);
    issue_v(has_next ? k0_next : 0, r);
    __builtin_amdgcn_sched_barrier(0);
  };

  // two tiles in flight per wave: ra holds tiles wave + 8i, rb tiles
  // wave + 8i + 4
  LineTile<D> ra, rb;
  constexpr int W = kWaves;
  // q, the block ids and the loads of the first two tiles
  auto prologue = [&](const Seg& sg) {
    bind(sg);
    const int ntiles = (sg.end - sg.start + TK - 1) / TK;
    // both register sets, a tile past the segment as an absent one (its keys
    // lie past `end`, so fetch_ids gives -1)
    __builtin_amdgcn_sched_barrier(0);
    fetch_ids(sg.start + wave * TK, ra.blk);
    issue_k(sg.start + wave * TK, ra);
    issue_v(sg.start + wave * TK, ra);
    __builtin_amdgcn_sched_barrier(0);
    fetch_ids(sg.start + (wave + W) * TK, rb.blk);
    issue_k(sg.start + (wave + W) * TK, rb);
    issue_v(sg.start + (wave + W) * TK, rb);
    __builtin_amdgcn_sched_barrier(0);
    if (wave + 2 * W < ntiles) fetch_ids(sg.start + (wave + 2 * W) * TK, ids_next);
  };
  // the tiles (the prologue has run)
  auto body = [&](const Seg& sg) {
    const int start = sg.start;
    const int ntiles = (sg.end - start + TK - 1) / TK;
    // q: its loads are followed by the prologue's two tiles
    wait_vm_q<2 * (KCF::NLD + DT)>(qf);
    if (l16 >= G) {
#pragma unroll
      for (int c = 0; c < KC; ++c) qf[c] = u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int mm = 0; mm < DT; ++mm) o[mm] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m = -1e30f;
    lsum = 0.f;
    auto at = [&](int t) { return t < ntiles ? start + t * TK : -1; };
    // the loop's back edge follows a set-1 tile only, so a set-0 tile is
    // always preceded by a set-1 step (or the prologue)
    int t = wave;
    if (t < ntiles) {
      while (true) {
        process(start + t * TK, ra, at(t + 2 * W), at(t + 3 * W));
        if (t + W >= ntiles) break;
        process(start + (t + W) * TK, rb, at(t + 3 * W), at(t + 4 * W));
        t += 2 * W;
        if (t >= ntiles) break;
      }
    }
    // every load of both sets has landed before their registers may be
    // reused (the last ones read zeros)
    wait_vm_k<0>(ra.k);
    wait_vm_k<0>(rb.k);
    wait_vm_v<0>(ra.v);
    wait_vm_v<0>(rb.v);
  };
  // The appended key (append mode): its row is written to the pool at
  // position L-1 (the tiles never read that slot) and its score for each
  // q-head computed into LDS (wave w takes heads w, w+4, ...; a lane 1 or 2
  // dims); a block id outside the pool makes it absent, as for any key.  Run
  // by every wave right after its tiles; the merge's first barrier publishes
  // the scores.
  auto append_key = [&](const Seg& sg) -> bool {
    bool add_new = false;
    if (APPEND && sg.last) {
      const int L = sg.end + 1;
      const bf16_t* kn = k_new + ((size_t)sg.b * (num_q_heads / G) + sg.kvh) * D;
      const bf16_t* vn = v_new + ((size_t)sg.b * (num_q_heads / G) + sg.kvh) * D;
      const int32_t* tb = bt + (size_t)sg.b * bt_stride;
      const int blk = tb[(L - 1) >> pool.bs_shift];
      add_new = blk >= 0 && blk < pool.num_blocks;
      if (add_new) {
        for (int g = wave; g < G; g += kWaves) {
          const bf16_t* qr = q + ((size_t)sg.b * num_q_heads + (size_t)sg.kvh * G + g) * D;
          float part = 0.f;
          for (int d = lane; d < D; d += 64) part = fmaf(bf16_to_f32(qr[d]), bf16_to_f32(kn[d]), part);
#pragma unroll
          for (int o2 = 32; o2 >= 1; o2 >>= 1) part += __shfl_xor(part, o2);
          if (lane == 0) sm.snew[g] = part * scale_log2;
        }
        const int sh = sg.kvh / hl, lh = sg.kvh - sh * hl;
        const size_t tile = ((size_t)blk * hl + lh) * ((size_t)bs * D);
        const int off = (L - 1) & (bs - 1);
        bf16_t* kp = const_cast<bf16_t*>(reinterpret_cast<const bf16_t*>(pool.k[sh])) + tile + (size_t)off * D;
        bf16_t* vp = const_cast<bf16_t*>(reinterpret_cast<const bf16_t*>(pool.v[sh])) + tile + off;
        for (int d = threadIdx.x; d < D; d += kThreads) {
          kp[d] = kn[d];
          vp[(size_t)d * bs] = vn[d];
        }
      } else if (threadIdx.x == 0) {
        flag_error(pool.err, PKV_ERRBIT_BLOCK_ID);
      }
    }
    return add_new;
  };
  // the 4 waves' (m, l, acc), combined and written, DC dims of
  // every q-head per pass
  auto merge = [&](const Seg& sg, bool add_new) {
    lsum = col_sum(lsum);
    if (l16 < G && j4 == 0) {
      sm.m[wave][l16] = m;
      sm.l[wave][l16] = lsum;
    }
#pragma unroll
    for (int pass = 0; pass < MG::PASSES; ++pass) {
      if (l16 < G) {
#pragma unroll
        for (int mm = 0; mm < DT; ++mm)
          if (mm / (MG::DC / 16) == pass)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sm.acc[wave][l16][16 * mm - pass * MG::DC + 4 * j4 + rr] = o[mm][rr];
      }
      __syncthreads();
      for (int i = threadIdx.x; i < G * MG::DC; i += kThreads) {
        const int g = i / MG::DC, dd = i - g * MG::DC, d = pass * MG::DC + dd;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm.m[w][g]);
        float l = 0.f, acc = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float f = __builtin_amdgcn_exp2f(sm.m[w][g] - mx);
          l += sm.l[w][g] * f;
          acc += sm.acc[w][g][dd] * f;
        }
        if (add_new) {
          const float sn = sm.snew[g];
          const float mf = fmaxf(mx, sn);
          const float fo = __builtin_amdgcn_exp2f(mx - mf), fn = __builtin_amdgcn_exp2f(sn - mf);
          const bf16_t* vn = v_new + ((size_t)sg.b * (num_q_heads / G) + sg.kvh) * D;
          l = l * fo + fn;
          acc = acc * fo + fn * bf16_to_f32(vn[d]);
          mx = mf;
        }
        const int h = sg.kvh * G + g;
        out[((size_t)sg.b * num_q_heads + h) * D + d] = f32_to_bf16(acc / l);
      }
      __syncthreads();                            // the merge buffers are free again
    }
  };

  int L = ctx[b];
  if (L > cap) {                              // past max_context_len: cut, flagged
    if (threadIdx.x == 0 && kvh == 0) flag_error(pool.err, PKV_ERRBIT_CONTEXT);
    L = cap;
  }
  if (L <= 0) return;
  const bool last = APPEND && ctx[b] <= cap;
  const Seg sg{b, kvh, 0, last ? L - 1 : L, last};
  prologue(sg);
  body(sg);
  const bool add_new = append_key(sg);
  merge(sg, add_new);
}

}  // namespace decode_line
}  // namespace pkv
