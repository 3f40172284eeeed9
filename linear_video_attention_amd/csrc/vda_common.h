// Device helpers shared by the VDA kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace vdn {

// Gauss-Jordan in-place inverse of the D x D matrix held as R x R register blocks by a 16 x 16
// thread grid (thread (ty, tx) owns rows ty*R.., cols tx*R..).  rowbuf/colbuf: [2][D] shared.
// No pivoting: the callers invert I + A with A symmetric positive semi-definite, whose pivots are
// all >= 1.  The pivot loop is split into (block, unrolled offset) so that every register index
// is a compile-time constant.
template <int D>
__device__ __forceinline__ void gauss_jordan_inverse(float (&a)[D / 16][D / 16], float* rowbuf, float* colbuf,
                                                     int ty, int tx) {
  constexpr int R = D / 16;
  for (int pb = 0; pb < 16; ++pb) {
#pragma unroll
    for (int pr = 0; pr < R; ++pr) {
      const int p = pb * R + pr;
      float* rb = rowbuf + (p & 1) * D;
      float* cb = colbuf + (p & 1) * D;
      if (ty == pb) {
#pragma unroll
        for (int jj = 0; jj < R; ++jj) rb[tx * R + jj] = a[pr][jj];
      }
      if (tx == pb) {
#pragma unroll
        for (int ii = 0; ii < R; ++ii) cb[ty * R + ii] = a[ii][pr];
      }
      __syncthreads();
      const float inv = 1.0f / rb[p];
      float rj[R], fi[R];
#pragma unroll
      for (int jj = 0; jj < R; ++jj) rj[jj] = (tx == pb && jj == pr) ? inv : rb[tx * R + jj] * inv;
#pragma unroll
      for (int ii = 0; ii < R; ++ii) fi[ii] = cb[ty * R + ii];
#pragma unroll
      for (int ii = 0; ii < R; ++ii) {
        const bool prow = (ty == pb && ii == pr);
#pragma unroll
        for (int jj = 0; jj < R; ++jj) {
          const bool pcol = (tx == pb && jj == pr);
          a[ii][jj] = prow ? rj[jj] : ((pcol ? 0.f : a[ii][jj]) - fi[ii] * rj[jj]);
        }
      }
    }
  }
}

}  // namespace vdn
