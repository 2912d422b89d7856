// Measurement aid: the bf16 MFMA rate this device sustains right now with
// nothing but back-to-back v_mfma_f32_32x32x16_bf16 on register operands
// (four independent accumulator chains per wave, two waves per SIMD, every CU
// busy). Two operand kinds:
//  - constant: every product multiplies the same two fragments. Few operand
//    bits toggle, the chip draws little power and holds its top clock: the
//    rate at which the matrix cores issue.
//  - random: each wave cycles through 8 A and 8 B fragments of varied bf16
//    values, so every product sees new operands, as the attention kernel's
//    products do. The chip's power limit then lowers the clock: the practical
//    ceiling for MFMA work on real data on this device.

#include <hip/hip_runtime.h>

#include <cmath>
#include <string>

#include "tara.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kChains = 4;
constexpr int kThreads = 256;      // four waves, one per SIMD
constexpr int kBlocksPerCu = 2;    // two waves per SIMD, as the attention kernel runs
constexpr int kFrags = 8;          // operand fragments per side in the random kind

// Marsaglia's xorshift32 ("Xorshift RNGs", J. Stat. Software 8(14), 2003),
// shifts 13, 17, 5; the result mapped to [-2, 2)
__device__ __forceinline__ float xorshift_uniform(unsigned& s) {
  s ^= s << 13;
  s ^= s >> 17;
  s ^= s << 5;
  return (float)(s >> 8) * (4.0f / 16777216.0f) - 2.0f;
}

template <bool RANDOM>
__global__ __launch_bounds__(kThreads) void mfma_probe_kernel(int iters, float* sink) {
  bf16x8 a[kFrags], b[kFrags];
  // seed: the global thread id times Knuth's multiplicative constant, made odd (never 0)
  unsigned s = (blockIdx.x * kThreads + threadIdx.x) * 2654435761u | 1u;
#pragma unroll
  for (int f = 0; f < kFrags; ++f)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (RANDOM) {
        a[f][i] = (__bf16)xorshift_uniform(s);
        b[f][i] = (__bf16)xorshift_uniform(s);
      } else {
        a[f][i] = (__bf16)(1.0f + 0.001f * (threadIdx.x & 7));
        b[f][i] = (__bf16)(0.5f - 0.001f * i);
      }
    }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  // rounds of kChains products; the random kind pairs fragment (u + 2c) of A
  // with (3u + c) of B in round u of each group of kFrags rounds
  int it = 0;
  for (; it + kFrags <= iters; it += kFrags) {
#pragma unroll
    for (int u = 0; u < kFrags; ++u)
#pragma unroll
      for (int c = 0; c < kChains; ++c) {
        const int fa = RANDOM ? (u + 2 * c) % kFrags : 0, fb = RANDOM ? (3 * u + c) % kFrags : 0;
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fa], b[fb], acc[c], 0, 0, 0);
      }
  }
  for (; it < iters; ++it)
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[c], acc[c], 0, 0, 0);
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[c][r];
  // never true for these operands; keeps the products live
  if (sink && sum == -1.0f) sink[blockIdx.x] = sum;
}

}  // namespace

extern "C" int tara_probe_mfma_bf16(int iterations, int operands, float* tflops, tara_stream_t stream_) {
  if (!tflops) return TARA_ERR_NULL_POINTER;
  if (iterations < 1 || iterations > (1 << 24)) return TARA_ERR_BAD_PARAM;
  if (operands != TARA_PROBE_CONSTANT && operands != TARA_PROBE_RANDOM) return TARA_ERR_BAD_PARAM;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return TARA_ERR_HIP;
  const int blocks = cus * kBlocksPerCu;
  auto launch = [&]() {
    if (operands == TARA_PROBE_RANDOM)
      hipLaunchKernelGGL(mfma_probe_kernel<true>, dim3(blocks), dim3(kThreads), 0, stream, iterations, nullptr);
    else
      hipLaunchKernelGGL(mfma_probe_kernel<false>, dim3(blocks), dim3(kThreads), 0, stream, iterations, nullptr);
  };
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int status = TARA_OK;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) status = TARA_ERR_HIP;
  if (status == TARA_OK) {
    // one untimed launch brings the clock to where this load settles; the second is timed
    launch();
    (void)hipEventRecord(e0, stream);
    launch();
    (void)hipEventRecord(e1, stream);
    float ms = 0.0f;
    if (hipGetLastError() != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
        hipEventElapsedTime(&ms, e0, e1) != hipSuccess || !(ms > 0.0f)) {
      status = TARA_ERR_HIP;
    } else {
      const double flop = (double)blocks * (kThreads / 64) * kChains * (double)iterations * 32.0 * 32.0 * 16.0 * 2.0;
      *tflops = (float)(flop / (ms * 1e-3) / 1e12);
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  return status;
}
