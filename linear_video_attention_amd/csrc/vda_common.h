// Device helpers shared by the VDA kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace vdn {

// Gauss-Jordan in-place inverse of the D x D matrix held as R x R register blocks by a 16 x 16
// thread grid (thread (ty, tx) owns rows ty*R.., cols tx*R..).  rowbuf/colbuf: [2][D] shared.
// No pivoting: the callers invert I + A with A symmetric positive semi-definite, whose pivots are
// all >= 1.  Pivot p maps a to
//   a_ij - a_ip a_pj / a_pp (i, j != p),  a_pj / a_pp (row p),  -a_ip / a_pp (column p),  1 / a_pp;
// every element takes the rank-one update a_ij - f_i r_j with r_j = a_pj / a_pp, and the owners of
// row and column p then overwrite those with their own values (the same arithmetic as a
// per-element select, at one FMA per element).  The pivot loop is split into (block, unrolled
// offset) so that every register index is a compile-time constant.
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
      for (int jj = 0; jj < R; ++jj) rj[jj] = rb[tx * R + jj] * inv;
#pragma unroll
      for (int ii = 0; ii < R; ++ii) fi[ii] = cb[ty * R + ii];
#pragma unroll
      for (int ii = 0; ii < R; ++ii)
#pragma unroll
        for (int jj = 0; jj < R; ++jj) a[ii][jj] -= fi[ii] * rj[jj];
      const bool own_row = ty == pb, own_col = tx == pb;
#pragma unroll
      for (int jj = 0; jj < R; ++jj) a[pr][jj] = own_row ? rj[jj] : a[pr][jj];
#pragma unroll
      for (int ii = 0; ii < R; ++ii) a[ii][pr] = own_col ? -fi[ii] * inv : a[ii][pr];
      a[pr][pr] = (own_row && own_col) ? inv : a[pr][pr];
    }
  }
}

}  // namespace vdn
