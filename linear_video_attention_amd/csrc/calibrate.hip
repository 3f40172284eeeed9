// On-box reference rates for the rooflines: a tight bf16 MFMA loop and a large device-to-device
// copy, each timed with HIP events on the null stream.  Measurement helpers only; no stage of the
// layer uses them.
#include <hip/hip_runtime.h>

#include "vdn_internal.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kBlocksPerCU = 8;
constexpr int kThreads = 256;
constexpr int kChains = 4;          // independent accumulators per wave

// Every wave issues kChains independent v_mfma_f32_32x32x16_bf16 per iteration.
__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(float* out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(threadIdx.x * 0.001f);
    b[j] = (__bf16)(j * 0.01f);
  }
  f32x16 c[kChains] = {};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int k = 0; k < kChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k) s += c[k][k];
  if (s == 12345.0f) out[threadIdx.x] = s;          // keeps the loop; never true for these inputs
}

}  // namespace

extern "C" vdn_status vdn_measure_mfma_bf16_tflops(int iters, double* tflops) {
  if (!tflops || iters <= 0) return VDN_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return VDN_ERR_HIP;
  float* out = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  vdn_status st = VDN_ERR_HIP;
  float ms = 0.f;
  const int blocks = cus * kBlocksPerCU;
  if (hipMalloc(&out, kThreads * sizeof(float)) == hipSuccess && hipEventCreate(&e0) == hipSuccess &&
      hipEventCreate(&e1) == hipSuccess) {
    mfma_loop_kernel<<<blocks, kThreads>>>(out, 64);                       // warm-up
    if (hipEventRecord(e0) == hipSuccess) {
      mfma_loop_kernel<<<blocks, kThreads>>>(out, iters);
      if (hipEventRecord(e1) == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
          hipEventElapsedTime(&ms, e0, e1) == hipSuccess && ms > 0.f) {
        const double flops = (double)blocks * (kThreads / 64) * iters * kChains * (2.0 * 32 * 32 * 16);
        *tflops = flops / (ms * 1e-3) / 1e12;
        st = VDN_OK;
      }
    }
  }
  (void)hipGetLastError();
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (out) (void)hipFree(out);
  return st;
}

extern "C" vdn_status vdn_measure_copy_gbs(size_t bytes, double* gbs) {
  if (!gbs || bytes < 16) return VDN_ERR_INVALID_ARG;
  void *src = nullptr, *dst = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  vdn_status st = VDN_ERR_HIP;
  float ms = 0.f;
  if (hipMalloc(&src, bytes) != hipSuccess || hipMalloc(&dst, bytes) != hipSuccess) {
    st = VDN_ERR_OUT_OF_MEMORY;
  } else if (hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess &&
             hipMemsetAsync(src, 1, bytes, nullptr) == hipSuccess &&
             hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, nullptr) == hipSuccess &&   // warm-up
             hipEventRecord(e0) == hipSuccess &&
             hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, nullptr) == hipSuccess &&
             hipEventRecord(e1) == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
             hipEventElapsedTime(&ms, e0, e1) == hipSuccess && ms > 0.f) {
    *gbs = 2.0 * (double)bytes / (ms * 1e-3) / 1e9;                       // read + write
    st = VDN_OK;
  }
  (void)hipGetLastError();
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (src) (void)hipFree(src);
  if (dst) (void)hipFree(dst);
  return st;
}
