// Backward pass (reverse mode) of the VDN layer: generic fp32 kernels for every d in {16..128}.
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models": the forward computes, per head,
//   out  = (g_s * o_s) Wp0 + (g_l * r) Wp1,   g = sigmoid(q Wg),  r = RMSNorm(o_l)
//          (section "Gating the Softmax and Linear Branch Outputs"),
//   o_s  = softmax over the query frame's key set (section "Local Softmax and Long-Range Linear
//          Memory"),
//   o_l  = (S_fwd + S_rev) q with every frame step S <- (S Diag(alpha_f) + B_f) M_f,
//          M_f = (I + A_f)^-1 (section "Video Delta Attention: A Frame-Wise Solution").
// The backward runs the transposes of those steps, in this order (each a kernel below):
//   1. merge_bwd        per 64-row block of one frame and head: gates, RMSNorm and projections
//                       transposed -> do_s, do_l, the gate/readout part of dq, the row-wise inputs
//                       of the weight gradients, and D = rowsum(do_s * o_s)
//   2. xty_reduce       X^T Y over row segments: the weight gradients (all rows of all heads) and,
//                       per chunk and head, the readout adjoint sum_i do_l_i q_i^T
//   3. frame_states     per (chunk, head, direction): the state entering every scanned frame
//   4. scan_bwd         per (head, direction), frames in reverse scan order: adjoint of each frame
//                       step -> dB_f and the adjoint after the write, and the text state's adjoint
//      frame_dm         per (scanned frame, head, direction): dM_f and dalpha_f from that adjoint
//   5. frame_mats       per (frame or text, head): dA = -M^T dM M^T; writes dA + dA^T and dB
//      token_grads      per (64 tokens, frame or text, head): dk = beta (dA + dA^T) k + beta dB^T v,
//                       dv = beta dB k, dbeta = k^T dA k + v^T dB k (text at beta/2), as row-block products
//   6. softmax_dq       per query: P from the saved normaliser, dS = P (dP - D), dq += tau dS K
//   7. softmax_dkv      per key: over every query row that sees it, dV += P^T do_s, dK += tau dS^T q
// All gradients are accumulated in fp32 into the caller's fp32 buffers.
#include <type_traits>

#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

constexpr int kThreads = 256;

// ---- D x D products on 16 x 16 threads, each thread an R x R block (R = D / 16) ----
// c[ii][jj] = sum_k a(ty R + ii, k) b(k, tx R + jj); a and b read LDS or global memory.
template <int D, class FA, class FB>
__device__ __forceinline__ void mm_block(FA a, FB b, float (&c)[D / 16][D / 16], int ty, int tx) {
  constexpr int R = D / 16;
#pragma unroll
  for (int ii = 0; ii < R; ++ii)
#pragma unroll
    for (int jj = 0; jj < R; ++jj) c[ii][jj] = 0.f;
  for (int kk = 0; kk < D; ++kk) {
    float av[R], bv[R];
#pragma unroll
    for (int ii = 0; ii < R; ++ii) av[ii] = a(ty * R + ii, kk);
#pragma unroll
    for (int jj = 0; jj < R; ++jj) bv[jj] = b(kk, tx * R + jj);
#pragma unroll
    for (int ii = 0; ii < R; ++ii)
#pragma unroll
      for (int jj = 0; jj < R; ++jj) c[ii][jj] = fmaf(av[ii], bv[jj], c[ii][jj]);
  }
}

// The same product with the right-hand operand b read from global memory (g, d x d row-major)
// through LDS, 16 rows of k at a time (coalesced loads instead of per-thread strided reads):
// b(k, j) = g[k d + j], or g[j d + k] when BT.  Every thread of the block must call it; wst holds
// 16 x D floats.
template <int D, bool BT, class FA>
__device__ __forceinline__ void mm_gstage(FA a, const float* __restrict__ g, float (*wst)[D], float (&c)[D / 16][D / 16],
                                          int ty, int tx) {
  constexpr int R = D / 16;
  const int tid = ty * 16 + tx;
#pragma unroll
  for (int ii = 0; ii < R; ++ii)
#pragma unroll
    for (int jj = 0; jj < R; ++jj) c[ii][jj] = 0.f;
  for (int k0 = 0; k0 < D; k0 += 16) {
    __syncthreads();
    for (int e = tid; e < 16 * D; e += kThreads) {
      if (BT) {
        const int kk = e % 16, j = e / 16;
        wst[kk][j] = g[(int64_t)j * D + k0 + kk];
      } else {
        const int kk = e / D, j = e % D;
        wst[kk][j] = g[(int64_t)(k0 + kk) * D + j];
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < 16; ++kk) {
      float av[R], bv[R];
#pragma unroll
      for (int ii = 0; ii < R; ++ii) av[ii] = a(ty * R + ii, k0 + kk);
#pragma unroll
      for (int jj = 0; jj < R; ++jj) bv[jj] = wst[kk][tx * R + jj];
#pragma unroll
      for (int ii = 0; ii < R; ++ii)
#pragma unroll
        for (int jj = 0; jj < R; ++jj) c[ii][jj] = fmaf(av[ii], bv[jj], c[ii][jj]);
    }
  }
}

// c = A b with the left-hand operand from global memory stored transposed: a(i, k) = g[k d + i]
// (rows of k staged through LDS as above).
template <int D, class FB>
__device__ __forceinline__ void mm_gstage_at(const float* __restrict__ g, FB b, float (*wst)[D],
                                             float (&c)[D / 16][D / 16], int ty, int tx) {
  constexpr int R = D / 16;
  const int tid = ty * 16 + tx;
#pragma unroll
  for (int ii = 0; ii < R; ++ii)
#pragma unroll
    for (int jj = 0; jj < R; ++jj) c[ii][jj] = 0.f;
  for (int k0 = 0; k0 < D; k0 += 16) {
    __syncthreads();
    for (int e = tid; e < 16 * D; e += kThreads) wst[e / D][e % D] = g[(int64_t)(k0 + e / D) * D + e % D];
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < 16; ++kk) {
      float av[R], bv[R];
#pragma unroll
      for (int ii = 0; ii < R; ++ii) av[ii] = wst[kk][ty * R + ii];
#pragma unroll
      for (int jj = 0; jj < R; ++jj) bv[jj] = b(k0 + kk, tx * R + jj);
#pragma unroll
      for (int ii = 0; ii < R; ++ii)
#pragma unroll
        for (int jj = 0; jj < R; ++jj) c[ii][jj] = fmaf(av[ii], bv[jj], c[ii][jj]);
    }
  }
}

// ---- 1. merge backward ----
// Rows are (token, head) pairs of one frame and head, kRows per block; threads 16 (row groups of
// kRows/16) x 16 (column groups of D/16).
#ifndef VDN_BWD_ROWS
#define VDN_BWD_ROWS 64
#endif
constexpr int kRows = VDN_BWD_ROWS;   // rows per block of the merge and token-gradient products (32: within 1 %)

constexpr int kWChunk = 16;            // rows of the right-hand matrix staged in LDS at a time

template <int D>
struct MergeSmem {
  float q[kRows][D + 1], dout[kRows][D + 1], t1[kRows][D + 1], t2[kRows][D + 1];
  float w[kWChunk][D];
};

// out[r][j] = sum_k x[r][k] w(k, j) for the thread's rows and columns; w is staged through LDS in
// chunks of kWChunk rows (every thread of the block must call it)
template <int D, class FW>
__device__ __forceinline__ void rows_mm(const float (*x)[D + 1], FW w, float (*wst)[D], float (&out)[kRows / 16][D / 16],
                                        int ty, int tx) {
  constexpr int RR = kRows / 16, RC = D / 16;
  const int tid = ty * 16 + tx;
#pragma unroll
  for (int i = 0; i < RR; ++i)
#pragma unroll
    for (int j = 0; j < RC; ++j) out[i][j] = 0.f;
  for (int k0 = 0; k0 < D; k0 += kWChunk) {
    __syncthreads();                                  // the previous chunk has been consumed
    for (int e = tid; e < kWChunk * D; e += kThreads) wst[e / D][e % D] = w(k0 + e / D, e % D);
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < kWChunk; ++kk) {
      float xv[RR], wv[RC];
#pragma unroll
      for (int i = 0; i < RR; ++i) xv[i] = x[ty * RR + i][k0 + kk];
#pragma unroll
      for (int j = 0; j < RC; ++j) wv[j] = wst[kk][tx * RC + j];
#pragma unroll
      for (int i = 0; i < RR; ++i)
#pragma unroll
        for (int j = 0; j < RC; ++j) out[i][j] = fmaf(xv[i], wv[j], out[i][j]);
    }
  }
}

template <typename Tin, int D>
__global__ __launch_bounds__(kThreads) void merge_bwd_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ o_s, const float* __restrict__ states,
    const Tin* __restrict__ gate_w, const Tin* __restrict__ proj_w, const Tin* __restrict__ dout,
    float* __restrict__ dq, float* __restrict__ do_s, float* __restrict__ do_l, float* __restrict__ x_s,
    float* __restrict__ x_l, float* __restrict__ dz_s, float* __restrict__ dz_l, float* __restrict__ dsum,
    int T, int N, int C, int Nc, int H, int anchors) {
  constexpr int RR = kRows / 16, RC = D / 16;
  constexpr int64_t DD = (int64_t)D * D;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  auto& S = *reinterpret_cast<MergeSmem<D>*>(smem_raw);
  const int t = blockIdx.y, h = blockIdx.z;
  const int n0 = blockIdx.x * kRows;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const bool bnd = anchors && (t == 0 || t == T - 1);
  const int slot = bnd ? Nc : t / C;
  const float* sf = states + ((int64_t)slot * H + h) * DD;                  // forward state
  const float* sr = states + ((int64_t)(Nc + 1 + slot) * H + h) * DD;      // reverse state
  auto row_ptr = [&](int r) { return ((int64_t)t * N + n0 + r) * H + h; };  // (token, head) index
  for (int e = tid; e < kRows * D; e += kThreads) {
    const int r = e / D, c = e % D;
    const bool ok = n0 + r < N;
    S.q[r][c] = ok ? to_f32(q[row_ptr(r) * D + c]) : 0.f;
    S.dout[r][c] = ok ? to_f32(dout[row_ptr(r) * D + c]) : 0.f;
  }
  __syncthreads();
  auto wmat = [&](const Tin* w) { return [w](int k, int j) { return to_f32(w[(int64_t)k * D + j]); }; };
  auto wmat_t = [&](const Tin* w) { return [w](int k, int j) { return to_f32(w[(int64_t)j * D + k]); }; };
  // o_l = S q  (row form: q S^T),  S = S_fwd + S_rev
  float ol[RR][RC], zs[RR][RC], zl[RR][RC], dxs[RR][RC], dxl[RR][RC];
  rows_mm<D>(S.q, [&](int k, int j) { return sf[(int64_t)j * D + k] + sr[(int64_t)j * D + k]; }, S.w, ol, ty, tx);
  rows_mm<D>(S.q, wmat(gate_w), S.w, zs, ty, tx);
  rows_mm<D>(S.q, wmat(gate_w + DD), S.w, zl, ty, tx);
  rows_mm<D>(S.dout, wmat_t(proj_w), S.w, dxs, ty, tx);
  rows_mm<D>(S.dout, wmat_t(proj_w + DD), S.w, dxl, ty, tx);
  // per-row RMS of o_l (row sums across the 16 column-group threads of the row group)
  float* red = &S.t1[0][0];                     // scratch [kRows][16]
  float* red2 = &S.t2[0][0];
#pragma unroll
  for (int i = 0; i < RR; ++i) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < RC; ++j) ss += ol[i][j] * ol[i][j];
    red[(ty * RR + i) * 16 + tx] = ss;
  }
  __syncthreads();
  float rho[RR];
#pragma unroll
  for (int i = 0; i < RR; ++i) {
    float ss = 0.f;
    for (int c = 0; c < 16; ++c) ss += red[(ty * RR + i) * 16 + c];
    rho[i] = sqrtf(ss / D + 1e-6f);
  }
  // gates, do_s, dz_s, dr, dz_l; rowsum(r * dr) and rowsum(do_s * o_s)
  float rdr[RR], dsm[RR];
  float dr[RR][RC], rr_[RR][RC];
#pragma unroll
  for (int i = 0; i < RR; ++i) {
    rdr[i] = 0.f;
    dsm[i] = 0.f;
    const int r = ty * RR + i;
    const bool ok = n0 + r < N;
#pragma unroll
    for (int j = 0; j < RC; ++j) {
      const int c = tx * RC + j;
      const float gs = sigmoidf_(zs[i][j]), gl = sigmoidf_(zl[i][j]);
      const float os = ok ? to_f32(o_s[row_ptr(r) * D + c]) : 0.f;
      const float rv = ol[i][j] / rho[i];
      const float dos = dxs[i][j] * gs;
      rr_[i][j] = rv;
      dr[i][j] = dxl[i][j] * gl;
      rdr[i] += rv * dr[i][j];
      dsm[i] += dos * os;
      zs[i][j] = dxs[i][j] * os * gs * (1.f - gs);          // dz_s
      zl[i][j] = dxl[i][j] * rv * gl * (1.f - gl);          // dz_l
      if (ok) {
        do_s[row_ptr(r) * D + c] = dos;
        x_s[row_ptr(r) * D + c] = gs * os;
        x_l[row_ptr(r) * D + c] = gl * rv;
        dz_s[row_ptr(r) * D + c] = zs[i][j];
        dz_l[row_ptr(r) * D + c] = zl[i][j];
      }
    }
  }
  __syncthreads();                               // red reused
#pragma unroll
  for (int i = 0; i < RR; ++i) {
    red[(ty * RR + i) * 16 + tx] = rdr[i];
    red2[(ty * RR + i) * 16 + tx] = dsm[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < RR; ++i) {
    float a = 0.f, b = 0.f;
    for (int c = 0; c < 16; ++c) {
      a += red[(ty * RR + i) * 16 + c];
      b += red2[(ty * RR + i) * 16 + c];
    }
    rdr[i] = a / D;
    dsm[i] = b;
  }
  if (tx == 0) {
#pragma unroll
    for (int i = 0; i < RR; ++i)
      if (n0 + ty * RR + i < N) dsum[row_ptr(ty * RR + i)] = dsm[i];
  }
  __syncthreads();
  // do_l = (dr - r mean(r dr)) / rho, kept in t1 for the readout transpose; dz_s, dz_l in q/dout
  // slots are not needed any more except q for nothing: stage dz_s -> t2, dz_l -> dout
#pragma unroll
  for (int i = 0; i < RR; ++i) {
    const int r = ty * RR + i;
    const bool ok = n0 + r < N;
#pragma unroll
    for (int j = 0; j < RC; ++j) {
      const int c = tx * RC + j;
      const float dl = (dr[i][j] - rr_[i][j] * rdr[i]) / rho[i];
      S.t1[r][c] = dl;
      S.t2[r][c] = zs[i][j];
      if (ok) do_l[row_ptr(r) * D + c] = dl;
    }
  }
  __syncthreads();
  // dz_l replaces dout in LDS (every thread has read dout already)
#pragma unroll
  for (int i = 0; i < RR; ++i)
#pragma unroll
    for (int j = 0; j < RC; ++j) S.dout[ty * RR + i][tx * RC + j] = zl[i][j];
  __syncthreads();
  // dq = dz_s Wg0^T + dz_l Wg1^T + do_l S
  float a1[RR][RC], a2[RR][RC], a3[RR][RC];
  rows_mm<D>(S.t2, wmat_t(gate_w), S.w, a1, ty, tx);
  rows_mm<D>(S.dout, wmat_t(gate_w + DD), S.w, a2, ty, tx);
  rows_mm<D>(S.t1, [&](int k, int j) { return sf[(int64_t)k * D + j] + sr[(int64_t)k * D + j]; }, S.w, a3, ty, tx);
#pragma unroll
  for (int i = 0; i < RR; ++i) {
    const int r = ty * RR + i;
    if (n0 + r >= N) continue;
#pragma unroll
    for (int j = 0; j < RC; ++j) dq[row_ptr(r) * D + tx * RC + j] = a1[i][j] + a2[i][j] + a3[i][j];
  }
}

// ---- 2. X^T Y over row segments ----
// Segment s covers rows [row0, row0 + nrows) of head `head` (head < 0: every head) of the
// [rows][H][D] arrays x, y; out[s] = sum_rows x^T y  (D x D).  Blocks: (segment, split); each
// block sums its share of the rows into partial[s][split] and the reduce kernel adds the splits.
template <int D, typename TX, typename TY>
__global__ __launch_bounds__(kThreads) void xty_partial_kernel(const TX* __restrict__ x, const TY* __restrict__ y,
                                                               const Segment* __restrict__ segs, int H, int splits,
                                                               float* __restrict__ partial) {
  constexpr int R = D / 16;
  constexpr int kTile = 32;
  __shared__ float xs[kTile][D + 1], ys[kTile][D + 1];
  const Segment sg = segs[blockIdx.x];
  const int split = blockIdx.y;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int heads = sg.head < 0 ? H : 1;
  const int64_t total = (int64_t)sg.nrows * heads;            // (row, head) pairs of the segment
  const int64_t per = (total + splits - 1) / splits;
  const int64_t p0 = split * per, p1 = min(total, p0 + per);
  float c[R][R];
#pragma unroll
  for (int ii = 0; ii < R; ++ii)
#pragma unroll
    for (int jj = 0; jj < R; ++jj) c[ii][jj] = 0.f;
  for (int64_t base = p0; base < p1; base += kTile) {
    for (int e = tid; e < kTile * D; e += kThreads) {
      const int r = e / D, col = e % D;
      const int64_t p = base + r;
      float xv = 0.f, yv = 0.f;
      if (p < p1) {
        const int64_t row = sg.row0 + p / heads;
        const int hh = sg.head < 0 ? (int)(p % heads) : sg.head;
        const int64_t off = (row * H + hh) * D + col;
        xv = to_f32(x[off]);
        yv = to_f32(y[off]);
      }
      xs[r][col] = xv;
      ys[r][col] = yv;
    }
    __syncthreads();
    for (int r = 0; r < kTile; ++r) {
      float av[R], bv[R];
#pragma unroll
      for (int ii = 0; ii < R; ++ii) av[ii] = xs[r][ty * R + ii];
#pragma unroll
      for (int jj = 0; jj < R; ++jj) bv[jj] = ys[r][tx * R + jj];
#pragma unroll
      for (int ii = 0; ii < R; ++ii)
#pragma unroll
        for (int jj = 0; jj < R; ++jj) c[ii][jj] = fmaf(av[ii], bv[jj], c[ii][jj]);
    }
    __syncthreads();
  }
  float* out = partial + ((int64_t)blockIdx.x * splits + split) * D * D;
#pragma unroll
  for (int ii = 0; ii < R; ++ii)
#pragma unroll
    for (int jj = 0; jj < R; ++jj) out[(int64_t)(ty * R + ii) * D + tx * R + jj] = c[ii][jj];
}

// grid (segments, D*D / 256): one thread per output element, summing the splits as eight
// interleaved partial sums (eight loads in flight), then those pairwise
template <int D>
__global__ __launch_bounds__(kThreads) void xty_reduce_kernel(const float* __restrict__ partial, int splits,
                                                              float* __restrict__ out, float scale) {
  const int s = blockIdx.x;
  const int e = blockIdx.y * kThreads + threadIdx.x;
  if (e >= D * D) return;
  const float* p = partial + (int64_t)s * splits * D * D + e;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int k = 0;
  for (; k + 8 <= splits; k += 8)
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] += p[(int64_t)(k + u) * D * D];
  for (; k < splits; ++k) acc[0] += p[(int64_t)k * D * D];
  const float sum = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  out[(int64_t)s * D * D + e] = sum * scale;
}

// ---- 3. states entering every scanned frame, per (chunk, head, direction) ----
// zin[dir][f][h] = state before frame f is written in direction dir.  The forward's chunk states
// give each chunk its entering state: S_fwd[j] has absorbed the chunks <= j - 2 and S_rev[j] the
// chunks >= j + 2 (slot Nc: S0), so chunk c starts from S_fwd[c + 1] (forward) or S_rev[c - 1]
// (reverse); the outermost chunk starts one chunk earlier and walks two.  Boundary frames (anchors
// on) are never written.
template <int D>
__global__ __launch_bounds__(kThreads) void frame_states_kernel(const float* __restrict__ states,
                                                                const float* __restrict__ minv,
                                                                const float* __restrict__ bw,
                                                                const float* __restrict__ alpha, int T, int C,
                                                                int anchors, int H, int Nc, float* __restrict__ zin) {
  constexpr int R = D / 16;
  constexpr int64_t DD = (int64_t)D * D;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  float(*z)[D + 1] = reinterpret_cast<float(*)[D + 1]>(smem_raw);                 // current state (rhs)
  float(*wst)[D] = reinterpret_cast<float(*)[D]>(z + D);                          // staged rows of M_f
  const int c = blockIdx.x, h = blockIdx.y, dir = blockIdx.z;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  // start slot and the frames to walk, [f_first, f_last] in walking order
  int slot, f_first, f_last;
  if (dir == 0) {
    slot = min(c + 1, Nc - 1);
    f_first = max(slot - 1, 0) * C;
    f_last = min((c + 1) * C, T) - 1;
  } else {
    slot = max(c - 1, 0);
    f_first = min((slot + 2) * C, T) - 1;
    f_last = c * C;
  }
  const float* s0 = states + ((int64_t)(dir * (Nc + 1) + slot) * H + h) * DD;
  for (int e = tid; e < D * D; e += kThreads) z[e / D][e % D] = s0[e];
  __syncthreads();
  const int step = dir == 0 ? 1 : -1;
  for (int f = f_first;; f += step) {
    const bool bnd = anchors && (f == 0 || f == T - 1);
    if (!bnd) {
      if (f / C == c) {
        float* zo = zin + (((int64_t)dir * T + f) * H + h) * DD;
        for (int e = tid; e < D * D; e += kThreads) zo[e] = z[e / D][e % D];
      }
      // rhs = Z Diag(alpha_f) + B_f, then Z <- rhs M_f
      const float* af = alpha ? alpha + ((int64_t)f * H + h) * D : nullptr;
      const float* bf = bw + ((int64_t)(1 + f) * H + h) * DD;
      const float* mf = minv + ((int64_t)(1 + f) * H + h) * DD;
      __syncthreads();
      for (int e = tid; e < D * D; e += kThreads) {
        const int r = e / D, cc = e % D;
        z[r][cc] = z[r][cc] * (af ? af[cc] : 1.f) + bf[e];
      }
      float cm[R][R];
      mm_gstage<D, false>([&](int i, int k) { return z[i][k]; }, mf, wst, cm, ty, tx);
      __syncthreads();
#pragma unroll
      for (int ii = 0; ii < R; ++ii)
#pragma unroll
        for (int jj = 0; jj < R; ++jj) z[ty * R + ii][tx * R + jj] = cm[ii][jj];
      __syncthreads();
    }
    if (f == f_last) break;
  }
}

// ---- 4. adjoint of the frame scans, per (head, direction) ----
// readout adjoints: dread[c] (c < Nc: chunk c's rows; c = Nc, Nc + 1: boundary frames 0 and T-1)
// enter the adjoint of the state of index mslot[dir][c] (frames written before that state is read).
template <int D>
__global__ __launch_bounds__(kThreads) void scan_bwd_kernel(
    const float* __restrict__ zin, const float* __restrict__ minv, const float* __restrict__ bw,
    const float* __restrict__ alpha, const float* __restrict__ dread, const int* __restrict__ mslot,
    const int* __restrict__ order, int nscan, int T, int H, int Nc, float* __restrict__ dmf,
    float* __restrict__ dbf, float* __restrict__ ds0) {
  constexpr int R = D / 16;
  constexpr int64_t DD = (int64_t)D * D;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  float(*adj)[D + 1] = reinterpret_cast<float(*)[D + 1]>(smem_raw);
  float(*rhs)[D + 1] = adj + D;
  float(*wst)[D] = reinterpret_cast<float(*)[D]>(rhs + D);                        // staged rows of M_f^T
  const int h = blockIdx.x, dir = blockIdx.y;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int* ms = mslot + dir * (Nc + 2);
  for (int e = tid; e < D * D; e += kThreads) adj[e / D][e % D] = 0.f;
  __syncthreads();
  auto add_reads = [&](int m) {
    for (int c = 0; c < Nc + 2; ++c)
      if (ms[c] == m) {
        const float* g = dread + ((int64_t)c * H + h) * DD;
        for (int e = tid; e < D * D; e += kThreads) adj[e / D][e % D] += g[e];
      }
    __syncthreads();
  };
  for (int m = nscan; m >= 1; --m) {
    add_reads(m);
    const int f = order[dir == 0 ? m - 1 : nscan - m];
    const float* af = alpha ? alpha + ((int64_t)f * H + h) * D : nullptr;
    const float* mf = minv + ((int64_t)(1 + f) * H + h) * DD;
    // dR = adj M^T (dB_f = dR); the adjoint after the write is kept for frame_dm (dM, dalpha)
    float dr[R][R];
    mm_gstage<D, true>([&](int i, int k) { return adj[i][k]; }, mf, wst, dr, ty, tx);
    float* dmo = dmf + (((int64_t)dir * T + f) * H + h) * DD;
    float* dbo = dbf + (((int64_t)dir * T + f) * H + h) * DD;
    for (int e = tid; e < D * D; e += kThreads) dmo[e] = adj[e / D][e % D];
#pragma unroll
    for (int ii = 0; ii < R; ++ii)
#pragma unroll
      for (int jj = 0; jj < R; ++jj) dbo[(int64_t)(ty * R + ii) * D + tx * R + jj] = dr[ii][jj];
    __syncthreads();                               // everyone is done with adj
    // adj <- dR Diag(alpha)
#pragma unroll
    for (int ii = 0; ii < R; ++ii)
#pragma unroll
      for (int jj = 0; jj < R; ++jj) {
        const int cc = tx * R + jj;
        adj[ty * R + ii][cc] = dr[ii][jj] * (af ? af[cc] : 1.f);
      }
    __syncthreads();
  }
  add_reads(0);
  float* o = ds0 + ((int64_t)dir * H + h) * DD;
  for (int e = tid; e < D * D; e += kThreads) o[e] = adj[e / D][e % D];
}

// ---- 4b. per (scanned frame, head, direction): dM = R^T adj and dalpha = diag(Z^T dR) ----
// R = Z Diag(alpha_f) + B_f with Z the state entering the frame; adj (the adjoint after the write,
// left in dmf by scan_bwd) is replaced by dM.
template <int D>
__global__ __launch_bounds__(kThreads) void frame_dm_kernel(const float* __restrict__ zin, const float* __restrict__ bw,
                                                            const float* __restrict__ alpha, int T, int H, int anchors,
                                                            float* __restrict__ dmf, const float* __restrict__ dbf,
                                                            float* __restrict__ dalf) {
  constexpr int R = D / 16;
  constexpr int64_t DD = (int64_t)D * D;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  float(*adj)[D + 1] = reinterpret_cast<float(*)[D + 1]>(smem_raw);
  float(*rhs)[D + 1] = adj + D;
  const int f = blockIdx.x, h = blockIdx.y, dir = blockIdx.z;
  if (anchors && (f == 0 || f == T - 1)) return;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const float* af = alpha ? alpha + ((int64_t)f * H + h) * D : nullptr;
  const int64_t slot = ((int64_t)dir * T + f) * H + h;
  const float* zf = zin + slot * DD;
  const float* bf = bw + ((int64_t)(1 + f) * H + h) * DD;
  float* dmo = dmf + slot * DD;
  for (int e = tid; e < D * D; e += kThreads) {
    const int r = e / D, cc = e % D;
    adj[r][cc] = dmo[e];
    rhs[r][cc] = zf[e] * (af ? af[cc] : 1.f) + bf[e];
  }
  __syncthreads();
  float dm[R][R];
  mm_block<D>([&](int i, int k) { return rhs[k][i]; }, [&](int k, int j) { return adj[k][j]; }, dm, ty, tx);
#pragma unroll
  for (int ii = 0; ii < R; ++ii)
#pragma unroll
    for (int jj = 0; jj < R; ++jj) dmo[(int64_t)(ty * R + ii) * D + tx * R + jj] = dm[ii][jj];
  if (dalf && tid < D) {
    const float* dr = dbf + slot * DD;
    float acc = 0.f;
    for (int r = 0; r < D; ++r) acc = fmaf(zf[(int64_t)r * D + tid], dr[(int64_t)r * D + tid], acc);
    dalf[slot * D + tid] = acc;
  }
}

// ---- 5a. per (frame or text, head): dA + dA^T and dB, with dA = -M^T dM M^T ----
template <int D>
__global__ __launch_bounds__(kThreads) void frame_mats_kernel(const float* __restrict__ minv, const float* __restrict__ bw,
                                                              const float* __restrict__ dmf,
                                                              const float* __restrict__ dbf,
                                                              const float* __restrict__ ds0, int T, int H, int n_text,
                                                              int anchors, float* __restrict__ gsym,
                                                              float* __restrict__ gdb) {
  constexpr int R = D / 16;
  constexpr int64_t DD = (int64_t)D * D;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  float(*ga)[D + 1] = reinterpret_cast<float(*)[D + 1]>(smem_raw);   // dM, then dA, then dA + dA^T
  float(*gb)[D + 1] = ga + D;                                         // dB
  float(*wst)[D] = reinterpret_cast<float(*)[D]>(gb + D);
  const int slot = blockIdx.x, h = blockIdx.y;
  if (slot > 0 && anchors && (slot - 1 == 0 || slot - 1 == T - 1)) return;
  if (slot == 0 && n_text == 0) return;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const float* m = minv + ((int64_t)slot * H + h) * DD;
  float c[R][R];
  auto put = [&](float (*dst)[D + 1], float sign) {
#pragma unroll
    for (int ii = 0; ii < R; ++ii)
#pragma unroll
      for (int jj = 0; jj < R; ++jj) dst[ty * R + ii][tx * R + jj] = sign * c[ii][jj];
  };
  // dM and dB of the slot: frames sum both directions; the text builds them from dS0 (both
  // directions): S0 = B0 M0, so dB0 = dS0 M0^T and dM0 = B0^T dS0
  if (slot > 0) {
    const int f = slot - 1;
    const float* m0 = dmf + ((int64_t)f * H + h) * DD;
    const float* m1 = dmf + (((int64_t)T + f) * H + h) * DD;
    const float* b0 = dbf + ((int64_t)f * H + h) * DD;
    const float* b1 = dbf + (((int64_t)T + f) * H + h) * DD;
    for (int e = tid; e < D * D; e += kThreads) {
      ga[e / D][e % D] = m0[e] + m1[e];
      gb[e / D][e % D] = b0[e] + b1[e];
    }
    __syncthreads();
  } else {
    const float* s0a = ds0 + (int64_t)h * DD;
    const float* s0b = ds0 + ((int64_t)H + h) * DD;
    for (int e = tid; e < D * D; e += kThreads) ga[e / D][e % D] = s0a[e] + s0b[e];
    __syncthreads();
    const float* b0 = bw + (int64_t)h * DD;
    float c2[R][R];
    mm_gstage<D, true>([&](int i, int kk) { return ga[i][kk]; }, m, wst, c, ty, tx);      // dS0 M0^T
    mm_gstage_at<D>(b0, [&](int kk, int j) { return ga[kk][j]; }, wst, c2, ty, tx);        // B0^T dS0
    __syncthreads();
    put(gb, 1.f);                                       // dB0
#pragma unroll
    for (int ii = 0; ii < R; ++ii)
#pragma unroll
      for (int jj = 0; jj < R; ++jj) c[ii][jj] = c2[ii][jj];
    put(ga, 1.f);                                       // dM0
    __syncthreads();
  }
  // dA = -M^T dM M^T, then ga <- dA + dA^T
  mm_gstage_at<D>(m, [&](int kk, int j) { return ga[kk][j]; }, wst, c, ty, tx);
  __syncthreads();
  put(ga, 1.f);
  mm_gstage<D, true>([&](int i, int kk) { return ga[i][kk]; }, m, wst, c, ty, tx);
  __syncthreads();
  put(ga, -1.f);
  __syncthreads();
#pragma unroll
  for (int ii = 0; ii < R; ++ii)
#pragma unroll
    for (int jj = 0; jj < R; ++jj) c[ii][jj] = ga[ty * R + ii][tx * R + jj] + ga[tx * R + jj][ty * R + ii];
  float* gs = gsym + ((int64_t)slot * H + h) * DD;
  float* gd = gdb + ((int64_t)slot * H + h) * DD;
#pragma unroll
  for (int ii = 0; ii < R; ++ii)
#pragma unroll
    for (int jj = 0; jj < R; ++jj) gs[(int64_t)(ty * R + ii) * D + tx * R + jj] = c[ii][jj];
  for (int e = tid; e < D * D; e += kThreads) gd[e] = gb[e / D][e % D];
}

// ---- 5b. token gradients, per (64 tokens, frame or text, head), as row-block products ----
// With G = dA + dA^T:  dk = w (K G + V dB),  dv = w K dB^T,  dbeta = w' (k^T G k / 2 + v^T dB k)
// (w = beta, or beta/2 for the text; w' = 1 or 1/2), each a 64 x d by d x d product.
template <int D>
struct TokSmem {
  float k[kRows][D + 1], v[kRows][D + 1];
  float w[kWChunk][D];
  float red[kRows][16];
};

template <typename Tin, int D>
__global__ __launch_bounds__(kThreads) void token_grads_kernel(
    const Tin* __restrict__ k, const Tin* __restrict__ v, const float* __restrict__ beta,
    const Tin* __restrict__ text_kv, const float* __restrict__ gsym, const float* __restrict__ gdb, int T, int N,
    int H, int n_text, int n_ctx, int anchors, float* __restrict__ dk, float* __restrict__ dv,
    float* __restrict__ dbeta, float* __restrict__ dtext_kv) {
  constexpr int RR = kRows / 16, RC = D / 16;
  constexpr int64_t DD = (int64_t)D * D;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  auto& S = *reinterpret_cast<TokSmem<D>*>(smem_raw);
  const int slot = blockIdx.y, h = blockIdx.z;
  if (slot > 0 && anchors && (slot - 1 == 0 || slot - 1 == T - 1)) return;
  const int U = slot == 0 ? n_text : N;
  const int u0 = blockIdx.x * kRows;
  if (u0 >= U) return;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const float wscale = slot == 0 ? 0.5f : 1.0f;
  const int64_t tok0 = slot == 0 ? 0 : (int64_t)(slot - 1) * N;
  const Tin* kb = slot == 0 ? text_kv : k;
  const Tin* vb = slot == 0 ? text_kv + (int64_t)n_ctx * H * D : v;     // V half of [2][n_ctx][H][d]
  float* dkb = slot == 0 ? dtext_kv : dk;
  float* dvb = slot == 0 ? dtext_kv + (int64_t)n_ctx * H * D : dv;
  const int64_t brow0 = slot == 0 ? 0 : n_text + tok0;
  auto row_off = [&](int r) { return ((tok0 + u0 + r) * H + h) * D; };
  for (int e = tid; e < kRows * D; e += kThreads) {
    const int r = e / D, cc = e % D;
    const bool ok = u0 + r < U;
    S.k[r][cc] = ok ? to_f32(kb[row_off(r) + cc]) : 0.f;
    S.v[r][cc] = ok ? to_f32(vb[row_off(r) + cc]) : 0.f;
  }
  __syncthreads();
  const float* gs = gsym + ((int64_t)slot * H + h) * DD;
  const float* gd = gdb + ((int64_t)slot * H + h) * DD;
  float g1[RR][RC], g2[RR][RC], gv[RR][RC];
  rows_mm<D>(S.k, [&](int kk, int j) { return gs[(int64_t)kk * D + j]; }, S.w, g1, ty, tx);   // K G
  rows_mm<D>(S.v, [&](int kk, int j) { return gd[(int64_t)kk * D + j]; }, S.w, g2, ty, tx);   // V dB
  rows_mm<D>(S.k, [&](int kk, int j) { return gd[(int64_t)j * D + kk]; }, S.w, gv, ty, tx);   // K dB^T
  float part[RR];
#pragma unroll
  for (int i = 0; i < RR; ++i) {
    const int r = ty * RR + i;
    const bool ok = u0 + r < U;
    const float wr = ok ? wscale * beta[(brow0 + u0 + r) * H + h] : 0.f;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < RC; ++j) {
      const int cc = tx * RC + j;
      acc += 0.5f * S.k[r][cc] * g1[i][j] + S.v[r][cc] * gv[i][j];
      if (ok) {
        dkb[row_off(r) + cc] += wr * (g1[i][j] + g2[i][j]);
        dvb[row_off(r) + cc] += wr * gv[i][j];
      }
    }
    part[i] = acc;
  }
#pragma unroll
  for (int i = 0; i < RR; ++i) S.red[ty * RR + i][tx] = part[i];
  __syncthreads();
  if (tid < kRows && u0 + tid < U) {
    float sum = 0.f;
#pragma unroll
    for (int cc = 0; cc < 16; ++cc) sum += S.red[tid][cc];
    dbeta[(brow0 + u0 + tid) * H + h] += wscale * sum;
  }
}

// ---- 6. softmax dq: one thread per query row.  Row group blockIdx.y holds nq rows (q, do_s, lse,
// dsum, dq indexed [groups][nq][H](...)) and uses key-range row t0 + blockIdx.y: the video frames
// (t0 = 0, nq = N) or the context rows (t0 = T, nq = n_ctx, one group).  Global keys: the n_ctx
// context tokens at key index j < ctx_pad. ----
template <typename Tin, int D>
__global__ __launch_bounds__(64) void softmax_dq_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v, const Tin* __restrict__ text_kv,
    const float* __restrict__ do_s, const float* __restrict__ lse, const float* __restrict__ dsum,
    const int* __restrict__ ranges, const int* __restrict__ nranges, int N, int t0, int H, int n_text, int text_pad,
    float tau, float* __restrict__ dq) {
  const int t = t0 + blockIdx.y, h = blockIdx.z;
  const int n = blockIdx.x * 64 + threadIdx.x;
  if (n >= N) return;
  const int64_t row = ((int64_t)blockIdx.y * N + n) * H + h;
  float qr[D], dor[D], acc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    qr[i] = to_f32(q[row * D + i]);
    dor[i] = do_s[row * D + i];
    acc[i] = 0.f;
  }
  const float l2 = lse[row], dd = dsum[row];
  const float c = tau * 1.4426950408889634f;
  const Tin* text_v = text_kv + (int64_t)n_text * H * D;
  const int nr = nranges[t];
  for (int r = 0; r < nr; ++r) {
    const int a = ranges[t * 2 * kMaxRanges + 2 * r], b = ranges[t * 2 * kMaxRanges + 2 * r + 1];
    for (int j = a; j < b; ++j) {
      const Tin *kp, *vp;
      if (j < text_pad) {
        kp = text_kv + ((int64_t)j * H + h) * D;
        vp = text_v + ((int64_t)j * H + h) * D;
      } else {
        kp = k + ((int64_t)(j - text_pad) * H + h) * D;
        vp = v + ((int64_t)(j - text_pad) * H + h) * D;
      }
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) {
        s = fmaf(qr[i], to_f32(kp[i]), s);
        dp = fmaf(dor[i], to_f32(vp[i]), dp);
      }
      const float p = exp2f(s * c - l2);
      const float ds = p * (dp - dd) * tau;
#pragma unroll
      for (int i = 0; i < D; ++i) acc[i] = fmaf(ds, to_f32(kp[i]), acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < D; ++i) dq[row * D + i] += acc[i];
}

// ---- 7. softmax dk, dv: one thread per key; the query frames that see a key frame come from a
// host table of frame ranges (qranges[kf] = list of [t0, t1) query-frame ranges) ----
template <typename Tin, int D>
__global__ __launch_bounds__(64) void softmax_dkv_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v, const Tin* __restrict__ text_kv,
    const float* __restrict__ do_s, const float* __restrict__ lse, const float* __restrict__ dsum,
    const int* __restrict__ qranges, const int* __restrict__ nqranges, int T, int N, int H, int n_text, float tau,
    const Tin* __restrict__ cq, const float* __restrict__ cdo, int n_cq, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ dtext_kv) {
  // key index j: 0 .. n_text-1 global (text, then audio) keys, then the video tokens; blockIdx.y =
  // key frame slot (0 = global keys, 1 + f = frame f).  Every key is also seen by the n_cq context
  // query rows cq (their do in cdo, lse and dsum after the T N video rows).
  const int slot = blockIdx.y, h = blockIdx.z;
  const int U = slot == 0 ? n_text : N;
  const int u = blockIdx.x * 64 + threadIdx.x;
  if (u >= U) return;
  const Tin* kp = slot == 0 ? text_kv + ((int64_t)u * H + h) * D : k + (((int64_t)(slot - 1) * N + u) * H + h) * D;
  const Tin* vp = slot == 0 ? text_kv + (((int64_t)n_text + u) * H + h) * D
                            : v + (((int64_t)(slot - 1) * N + u) * H + h) * D;
  float kr[D], vr[D], gk[D], gv[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    kr[i] = to_f32(kp[i]);
    vr[i] = to_f32(vp[i]);
    gk[i] = 0.f;
    gv[i] = 0.f;
  }
  const float c = tau * 1.4426950408889634f;
  const int* qr = qranges + slot * 2 * kMaxRanges;
  const int nr = nqranges[slot];
  for (int r = 0; r < nr; ++r) {
    const int t0 = qr[2 * r], t1 = qr[2 * r + 1];
    for (int64_t n = (int64_t)t0 * N; n < (int64_t)t1 * N; ++n) {
      const int64_t row = n * H + h;
      const Tin* qp = q + row * D;
      const float* dp_ = do_s + row * D;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) {
        s = fmaf(to_f32(qp[i]), kr[i], s);
        dp = fmaf(dp_[i], vr[i], dp);
      }
      const float p = exp2f(s * c - lse[row]);
      const float ds = p * (dp - dsum[row]) * tau;
#pragma unroll
      for (int i = 0; i < D; ++i) {
        gv[i] = fmaf(p, dp_[i], gv[i]);
        gk[i] = fmaf(ds, to_f32(qp[i]), gk[i]);
      }
    }
  }
  for (int n = 0; n < n_cq; ++n) {
    const int64_t crow = (int64_t)n * H + h;
    const int64_t row = (int64_t)T * N * H + crow;
    const Tin* qp = cq + crow * D;
    const float* dp_ = cdo + crow * D;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) {
      s = fmaf(to_f32(qp[i]), kr[i], s);
      dp = fmaf(dp_[i], vr[i], dp);
    }
    const float p = exp2f(s * c - lse[row]);
    const float ds = p * (dp - dsum[row]) * tau;
#pragma unroll
    for (int i = 0; i < D; ++i) {
      gv[i] = fmaf(p, dp_[i], gv[i]);
      gk[i] = fmaf(ds, to_f32(qp[i]), gk[i]);
    }
  }
  float* dkp = slot == 0 ? dtext_kv + ((int64_t)u * H + h) * D : dk + (((int64_t)(slot - 1) * N + u) * H + h) * D;
  float* dvp = slot == 0 ? dtext_kv + (((int64_t)n_text + u) * H + h) * D
                         : dv + (((int64_t)(slot - 1) * N + u) * H + h) * D;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    dkp[i] += gk[i];
    dvp[i] += gv[i];
  }
}

// Context query rows: do in fp32 and D = rowsum(do * o) of each row and head, stored after the T N
// video rows' values.  One 64-thread group per (row, head).
template <typename Tin, int D>
__global__ __launch_bounds__(64) void ctx_rows_dsum_kernel(const Tin* __restrict__ dctx, const Tin* __restrict__ octx,
                                                           float* __restrict__ do_ctx, float* __restrict__ dsum_ctx) {
  const int64_t row = blockIdx.x;             // (context row) * H + head
  float acc = 0.f;
  for (int i = threadIdx.x; i < D; i += 64) {
    const float g = to_f32(dctx[row * D + i]);
    do_ctx[row * D + i] = g;
    acc = fmaf(g, to_f32(octx[row * D + i]), acc);
  }
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (threadIdx.x == 0) dsum_ctx[row] = acc;
}

__global__ void sum2_kernel(const float* __restrict__ a, const float* __restrict__ b, float* __restrict__ out,
                            int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = a[i] + b[i];
}

__global__ void zero_kernel(float* __restrict__ x, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) x[i] = 0.f;
}

template <int D>
size_t merge_smem() { return sizeof(MergeSmem<D>); }

template <typename Tin, int D>
hipError_t run_t(const Shape& s, const Inputs& in, const Buffers& b, const BwdBuffers& w, const BwdOutputs& o,
                 bool mfma_softmax, hipStream_t st) {
  const int T = s.T, N = s.N, H = s.H, Nc = s.Nc;
  const int64_t DD = (int64_t)D * D;
  const float tau = 1.0f / sqrtf((float)D);
  // outputs that are accumulated start from zero
  auto zero = [&](float* x, int64_t n) {
    if (x && n > 0) zero_kernel<<<(int)((n + 255) / 256), 256, 0, st>>>(x, n);
  };
  zero(o.dk, (int64_t)T * N * H * D);
  zero(o.dv, (int64_t)T * N * H * D);
  zero(o.dbeta, ((int64_t)s.n_text + (int64_t)T * N) * H);
  zero(o.dtext_kv, (int64_t)2 * s.n_ctx * H * D);
  const int n_cq = w.dctx_out ? s.n_ctx : 0;       // context query rows in this backward
  if (n_cq > 0) {
    zero(o.dctx_q, (int64_t)n_cq * H * D);
    ctx_rows_dsum_kernel<Tin, D><<<dim3((unsigned)((int64_t)n_cq * H)), 64, 0, st>>>(
        (const Tin*)w.dctx_out, (const Tin*)w.octx, w.do_ctx, w.dsum + (int64_t)T * N * H);
  }
  if (o.dalpha) zero(w.dalf, (int64_t)2 * T * H * D);   // frames never written (boundary) keep zero
  // 1. merge backward (matrix cores for the plans whose softmax transpose runs on them)
  bool merged = false;
  if constexpr (std::is_same<Tin, bf16_t>::value && (D == 64 || D == 128)) {
    if (mfma_softmax) {
      const hipError_t e = launch_merge_bwd_mfma(s, in, b, w, o, st);
      if (e != hipSuccess) return e;
      merged = true;
    }
  }
  if (!merged) {
    const size_t sm = merge_smem<D>();
    (void)hipFuncSetAttribute((const void*)merge_bwd_kernel<Tin, D>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
    merge_bwd_kernel<Tin, D><<<dim3((N + kRows - 1) / kRows, T, H), kThreads, sm, st>>>(
        (const Tin*)in.q, (const Tin*)b.os, b.states, (const Tin*)in.gate_w, (const Tin*)in.proj_w,
        (const Tin*)w.dout, o.dq, w.do_s, w.do_l, w.x_s, w.x_l, w.dz_s, w.dz_l, w.dsum, T, N, s.C, Nc, H, s.anchors);
  }
  // 2. weight gradients (all rows, all heads) and per-chunk readout adjoints
  {
    auto xty = [&](auto x, auto y, const Segment* segs, int nseg, int splits, float* out) {
      using TX = std::remove_cv_t<std::remove_pointer_t<decltype(x)>>;
      using TY = std::remove_cv_t<std::remove_pointer_t<decltype(y)>>;
      bool on_mfma = false;   // matrix cores for the plans whose softmax transpose runs on them
      if constexpr (std::is_same<Tin, bf16_t>::value && (D == 64 || D == 128) &&
                    std::is_same<TX, float>::value != std::is_same<TY, float>::value) {
        if (mfma_softmax) {
          on_mfma = launch_xty_mfma(D, x, std::is_same<TX, float>::value, y, std::is_same<TY, float>::value, segs,
                                    nseg, splits, H, w.partial, st) == hipSuccess;   // else the generic kernel
        }
      }
      if (!on_mfma)
        xty_partial_kernel<D, TX, TY><<<dim3(nseg, splits), kThreads, 0, st>>>(x, y, segs, H, splits, w.partial);
      xty_reduce_kernel<D><<<dim3(nseg, (D * D + kThreads - 1) / kThreads), kThreads, 0, st>>>(w.partial, splits, out,
                                                                                               1.f);
    };
    const Tin* q = (const Tin*)in.q;
    const Tin* dout = (const Tin*)w.dout;
    // dWp = x^T dout, dWg = q^T dz over every row of every head
    xty(w.x_s, dout, w.seg_all, 1, w.splits_all, o.dproj_w);
    xty(w.x_l, dout, w.seg_all, 1, w.splits_all, o.dproj_w + DD);
    xty(q, (const float*)w.dz_s, w.seg_all, 1, w.splits_all, o.dgate_w);
    xty(q, (const float*)w.dz_l, w.seg_all, 1, w.splits_all, o.dgate_w + DD);
    // readout adjoints: per chunk (slot Nc: the boundary frames) and head, sum of do_l q^T
    xty((const float*)w.do_l, q, w.seg_read, (Nc + 2) * H, w.splits_read, w.dread);
  }
  // 3.-5. linear branch
  if (w.nscan > 0) {
    const size_t sm1 = (size_t)D * (D + 1) * 4 + (size_t)16 * D * 4;
    (void)hipFuncSetAttribute((const void*)frame_states_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm1);
    bool walked = false;   // matrix cores for the plans whose softmax transpose runs on them
    if constexpr (std::is_same<Tin, bf16_t>::value && (D == 64 || D == 128)) {
      if (mfma_softmax) {
        const hipError_t e = launch_frame_states_mfma(s, in, b, w, st);
        if (e != hipSuccess) return e;
        walked = true;
      }
    }
    if (!walked)
      frame_states_kernel<D><<<dim3(Nc, H, 2), kThreads, sm1, st>>>(b.states, b.minv, b.bw, in.alpha, T, s.C,
                                                                   s.anchors, H, Nc, w.zin);
  }
  {
    const size_t sm2 = (size_t)2 * D * (D + 1) * 4 + (size_t)16 * D * 4;
    (void)hipFuncSetAttribute((const void*)scan_bwd_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm2);
    bool chained = false;   // matrix cores for the plans whose softmax transpose runs on them
    if constexpr (std::is_same<Tin, bf16_t>::value && (D == 64 || D == 128)) {
      if (mfma_softmax) {
        const hipError_t e = launch_scan_bwd_mfma(s, in, b, w, st);
        if (e != hipSuccess) return e;
        chained = true;
      }
    }
    if (!chained)
      scan_bwd_kernel<D><<<dim3(H, 2), kThreads, sm2, st>>>(w.zin, b.minv, b.bw, in.alpha, w.dread, w.mslot, w.order,
                                                           w.nscan, T, H, Nc, w.dmf, w.dbf, w.ds0);
    if (w.nscan > 0) {
      const size_t smd = (size_t)2 * D * (D + 1) * 4;
      (void)hipFuncSetAttribute((const void*)frame_dm_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smd);
      frame_dm_kernel<D><<<dim3(T, H, 2), kThreads, smd, st>>>(w.zin, b.bw, in.alpha, T, H, s.anchors, w.dmf, w.dbf,
                                                               in.alpha ? w.dalf : nullptr);
    }
  }
  // 6.-7. softmax branch (dq adds to the merge part, dk/dv/dtext start from zero)
  if (mfma_softmax) {
    if constexpr (std::is_same<Tin, bf16_t>::value && (D == 64 || D == 128)) {
      const hipError_t e = launch_softmax_backward_mfma(s, in, b, w, o, st);
      if (e != hipSuccess) return e;
    }
  } else {
  softmax_dq_kernel<Tin, D><<<dim3((N + 63) / 64, T, H), 64, 0, st>>>(
      (const Tin*)in.q, (const Tin*)in.k, (const Tin*)in.v, (const Tin*)in.text_kv, w.do_s, w.lse, w.dsum, b.ranges,
      b.nranges, N, 0, H, s.n_ctx, s.ctx_pad, tau, o.dq);
  if (n_cq > 0) {
    const int64_t c0 = (int64_t)T * N * H;      // the context rows' lse and D follow the video rows'
    softmax_dq_kernel<Tin, D><<<dim3((n_cq + 63) / 64, 1, H), 64, 0, st>>>(
        (const Tin*)in.ctx_q, (const Tin*)in.k, (const Tin*)in.v, (const Tin*)in.text_kv, w.do_ctx, w.lse + c0,
        w.dsum + c0, b.ranges, b.nranges, n_cq, T, H, s.n_ctx, s.ctx_pad, tau, o.dctx_q);
  }
  softmax_dkv_kernel<Tin, D><<<dim3((max(N, s.n_ctx) + 63) / 64, T + 1, H), 64, 0, st>>>(
      (const Tin*)in.q, (const Tin*)in.k, (const Tin*)in.v, (const Tin*)in.text_kv, w.do_s, w.lse, w.dsum,
      w.qranges, w.nqranges, T, N, H, s.n_ctx, tau, (const Tin*)in.ctx_q, w.do_ctx, n_cq, o.dk, o.dv, o.dtext_kv);
  }
  {
    const size_t sm3 = (size_t)2 * D * (D + 1) * 4 + (size_t)16 * D * 4;
    (void)hipFuncSetAttribute((const void*)frame_mats_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm3);
    frame_mats_kernel<D><<<dim3(T + 1, H), kThreads, sm3, st>>>(b.minv, b.bw, w.dmf, w.dbf, w.ds0, T, H, s.n_text,
                                                               s.anchors, w.gsym, w.gdb);
    bool tok_done = false;   // matrix cores for the plans whose softmax transpose runs on them
    if constexpr (std::is_same<Tin, bf16_t>::value && (D == 64 || D == 128)) {
      if (mfma_softmax) {
        const hipError_t e = launch_token_grads_mfma(s, in, w, o, st);
        if (e != hipSuccess) return e;
        tok_done = true;
      }
    }
    if (!tok_done) {
      const size_t sm4 = sizeof(TokSmem<D>);
      (void)hipFuncSetAttribute((const void*)token_grads_kernel<Tin, D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)sm4);
      token_grads_kernel<Tin, D><<<dim3((max(N, s.n_text) + kRows - 1) / kRows, T + 1, H), kThreads, sm4, st>>>(
          (const Tin*)in.k, (const Tin*)in.v, in.beta, (const Tin*)in.text_kv, w.gsym, w.gdb, T, N, H, s.n_text,
          s.n_ctx, s.anchors, o.dk, o.dv, o.dbeta, o.dtext_kv);
    }
  }
  // dalpha: sum of both directions
  if (o.dalpha) {
    const int64_t n = (int64_t)T * H * D;
    sum2_kernel<<<(int)((n + 255) / 256), 256, 0, st>>>(w.dalf, w.dalf + n, o.dalpha, n);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const Shape& s, const Inputs& in, const Buffers& b, const BwdBuffers& w,
                           const BwdOutputs& o, bool mfma_softmax, hipStream_t st) {
  const bool bf = s.dtype == VDN_BF16;
  const bool mf = mfma_softmax && bf && (s.d == 64 || s.d == 128);
  switch (s.d) {
    case 16: return bf ? run_t<bf16_t, 16>(s, in, b, w, o, false, st) : run_t<float, 16>(s, in, b, w, o, false, st);
    case 32: return bf ? run_t<bf16_t, 32>(s, in, b, w, o, false, st) : run_t<float, 32>(s, in, b, w, o, false, st);
    case 64: return bf ? run_t<bf16_t, 64>(s, in, b, w, o, mf, st) : run_t<float, 64>(s, in, b, w, o, false, st);
    default: return bf ? run_t<bf16_t, 128>(s, in, b, w, o, mf, st) : run_t<float, 128>(s, in, b, w, o, false, st);
  }
}

}  // namespace vdn
