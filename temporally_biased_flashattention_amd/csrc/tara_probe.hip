// Measurement aid: the bf16 MFMA rate this device sustains right now with
// nothing but back-to-back v_mfma_f32_32x32x16_bf16 on register operands
// (four independent accumulator chains per wave, two waves per SIMD, every CU
// busy). It is the practical ceiling the attention kernel's MFMA work runs
// against on the same clock, next to the nominal 2.5 PFLOP/s.

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

__global__ __launch_bounds__(kThreads) void mfma_probe_kernel(int iters, float* sink) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1.0f + 0.001f * (threadIdx.x & 7));
    b[i] = (__bf16)(0.5f - 0.001f * i);
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  // never true for these operands; keeps the products live
  if (sink && s == -1.0f) sink[blockIdx.x] = s;
}

}  // namespace

extern "C" int tara_probe_mfma_bf16(int iterations, float* tflops, tara_stream_t stream_) {
  if (!tflops) return TARA_ERR_NULL_POINTER;
  if (iterations < 1 || iterations > (1 << 24)) return TARA_ERR_BAD_PARAM;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return TARA_ERR_HIP;
  const int blocks = cus * kBlocksPerCu;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int status = TARA_OK;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) status = TARA_ERR_HIP;
  if (status == TARA_OK) {
    // one untimed launch brings the clock up; the second is timed
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(kThreads), 0, stream, iterations, nullptr);
    (void)hipEventRecord(e0, stream);
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(kThreads), 0, stream, iterations, nullptr);
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
