// Calibration of the device's dense bf16 matrix-core rate and its shader
// clock while the matrix cores are busy (measurement infrastructure of the
// benchmark; not part of the attention library).
//
// Every wave runs `iters` rounds of four independent accumulation chains of
// v_mfma_f32_32x32x16_bf16 (32*32*16*2 flop each) and reads the shader clock
// counter (s_memtime, one tick per shader clock) and the constant 100 MHz
// reference counter (s_memrealtime) before and after; their ratio is the
// clock the waves ran at.  Stores are vector stores (each lane writes its own
// word).
//
// Two operand regimes: constant operands (every MFMA of a wave multiplies
// the same A and B), and eight different pairs of pseudo-random bf16
// operands that consecutive MFMAs cycle through, as the operands of an
// attention kernel change from one MFMA to the next.  The part's clock under
// a saturated matrix-core load depends on how much the operand bits switch.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

namespace {

// a value in [-2, 2) from a 32-bit integer hash of (wave, lane, k, e)
__device__ __forceinline__ float hash_unit(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return (float)(x >> 8) * (4.0f / 16777216.0f) - 2.0f;
}

template <bool RANDOM>
__global__ void __launch_bounds__(256, 2)
mfma_chain_kernel(int iters, float* __restrict__ sink, unsigned long long* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  constexpr int NP = RANDOM ? 8 : 1;            // operand pairs cycled through
  bf16x8_t a[NP], b[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (RANDOM) {
        const uint32_t key = (((uint32_t)wave * 64u + lane) * 8u + k) * 8u + e;
        a[k][e] = (__bf16)hash_unit(2u * key);
        b[k][e] = (__bf16)hash_unit(2u * key + 1u);
      } else {
        a[k][e] = (__bf16)(0.001f * (float)((lane + e) & 7));
        b[k][e] = (__bf16)(0.002f * (float)((lane * 3 + e) & 7));
      }
    }
  // distinct starting values keep the four chains distinct computations
  f32x16_t c0, c1, c2, c3;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    c0[r] = 0.f;
    c1[r] = 1.f;
    c2[r] = 2.f;
    c3[r] = (float)lane;
  }
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  // iters is a multiple of NP (the host checks it); round i uses pairs
  // i, i+1, i+2, i+3 (mod NP) for its four chains
  for (int i = 0; i < iters; i += NP) {
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[k], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(k + 1) % NP], b[(k + 1) % NP], c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(k + 2) % NP], b[(k + 2) % NP], c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(k + 3) % NP], b[(k + 3) % NP], c3, 0, 0, 0);
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float acc = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc += c0[r] + c1[r] + c2[r] + c3[r];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
  // lanes 0 and 1 of each wave write its shader-clock and reference-clock spans
  if (lane < 2) clocks[(size_t)wave * 2 + lane] = lane == 0 ? t1 - t0 : r1 - r0;
}

}  // namespace

extern "C" {

// Launches `blocks` workgroups of 256 threads (4 waves) on `stream`.
//   sink    device float [blocks * 256]
//   clocks  device uint64 [blocks * 4 * 2]: per wave, shader clocks then
//           100 MHz reference ticks over its MFMA loop
// Each wave performs iters * 4 * 32768 flop.  Returns 0 or the HIP error.
int pkv_calib_mfma(int iters, int blocks, float* sink, unsigned long long* clocks, hipStream_t stream) {
  if (iters <= 0 || blocks <= 0 || !sink || !clocks) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_chain_kernel<false>, dim3(blocks), dim3(256), 0, stream, iters, sink, clocks);
  return (int)hipGetLastError();
}

// The same with the eight pseudo-random operand pairs; iters must be a
// multiple of 8.
int pkv_calib_mfma_random(int iters, int blocks, float* sink, unsigned long long* clocks, hipStream_t stream) {
  if (iters <= 0 || iters % 8 != 0 || blocks <= 0 || !sink || !clocks) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_chain_kernel<true>, dim3(blocks), dim3(256), 0, stream, iters, sink, clocks);
  return (int)hipGetLastError();
}

}  // extern "C"
