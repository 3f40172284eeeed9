// Device helpers shared by the VDA kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace vdn {

// Gauss-Jordan in-place inverse of the D x D matrix held as R x R register blocks by a 16 x 16
// thread grid (thread (ty, tx) owns rows ty*R.., cols tx*R..).  rowbuf/colbuf: [2][D] shared.
// No pivoting: the callers invert I + A with A symmetric positive semi-definite, whose pivots are
// all >= 1.  Pivot p maps a to
//   a_ij - a_ip a_pj / a_pp (i, j != p),  a_pj / a_pp (row p),  -a_ip / a_pp (column p),  1 / a_pp;
// every element takes the rank-one update a_ij - g_i a_pj with g_i = a_ip / a_pp, and the owners
// of column p then store -g_i, the owners of row p a_pj / a_pp, the owner of a_pp 1 / a_pp.  The
// kernel is bound by vector-ALU issue (366 eliminations at 768p, two per CU on part of the chip),
// so the per-pivot work is kept to the FMAs of the update plus one multiply per owned row (g_i):
// the row fix-up runs as a branch taken by the one wave that holds row p, 1 / a_pp is a
// reciprocal refined by one Newton step, and the column fix-up is a sign-flipped copy of g.
// The pivot loop is split into (block, unrolled offset) so that every register index is a
// compile-time constant.
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
      const float piv = rb[p];
      float inv = __builtin_amdgcn_rcpf(piv);
      inv = __builtin_fmaf(__builtin_fmaf(-piv, inv, 1.0f), inv, inv);
      float rj[R], gi[R];
#pragma unroll
      for (int jj = 0; jj < R; ++jj) rj[jj] = rb[tx * R + jj];
#pragma unroll
      for (int ii = 0; ii < R; ++ii) gi[ii] = cb[ty * R + ii] * inv;
#pragma unroll
      for (int ii = 0; ii < R; ++ii)
#pragma unroll
        for (int jj = 0; jj < R; ++jj) a[ii][jj] = __builtin_fmaf(-gi[ii], rj[jj], a[ii][jj]);
      if (ty == pb) {                      // the one wave holding row p
#pragma unroll
        for (int jj = 0; jj < R; ++jj) a[pr][jj] = rj[jj] * inv;
      }
      const bool own_col = tx == pb;
#pragma unroll
      for (int ii = 0; ii < R; ++ii) a[ii][pr] = own_col ? -gi[ii] : a[ii][pr];
      a[pr][pr] = (ty == pb && own_col) ? inv : a[pr][pr];
    }
  }
}

}  // namespace vdn
