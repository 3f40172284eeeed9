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

// Workgroup barrier that orders LDS only.  __syncthreads() also fences global memory, which on
// this target waits for every outstanding vector-memory operation of the wave (vmcnt(0)): the
// global loads, stores and LDS DMA copies issued for later tiles or steps, so a multi-stage tile
// pipeline drains at every barrier (an LDS-only fence does the same, since LDS DMA is counted by
// vmcnt).  Here the wave waits only for its own LDS operations (lgkmcnt(0)) before s_barrier,
// and the memory clobber keeps the compiler from moving memory accesses across it.  A tile copied
// by LDS DMA must be waited for with an explicit vmcnt by every wave that issued part of it
// before the barrier, and nothing written to global memory by another wave is visible after it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace vdn
