// Device-side helpers shared by the VDN kernels: element loads/stores for the two input types.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace vdn {

// bf16 is carried as its raw 16-bit pattern in memory.
using bf16_t = uint16_t;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(((uint32_t)x) << 16); }

__device__ __forceinline__ void store_elt(float* p, float x) { *p = x; }
__device__ __forceinline__ void store_elt(bf16_t* p, float x) {
  __bf16 b = (__bf16)x;                    // round to nearest even
  *p = __builtin_bit_cast(bf16_t, b);
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

// Sigmoid from the hardware exp2 and reciprocal (v_exp_f32, v_rcp_f32: about 1 ulp each) instead of
// the IEEE-exact division sequence; large |x| saturate to 0 or 1.
__device__ __forceinline__ float fast_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

}  // namespace vdn
