// Video Delta Attention (the linear branch): per-frame statistics, their inverse, and the two
// state scans.
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Video Delta
// Attention: A Frame-Wise Solution" (and "Faster Than It Plays ...", section "Two branches instead
// of one"): a frame's tokens jointly update the state as S <- (S + B)(I + A)^-1 with the weighted
// key Gram A = sum_u beta_u k_u k_u^T and write matrix B = sum_u beta_u v_u k_u^T.  Section "Local
// Softmax and Long-Range Linear Memory": the text is written once into both directions at half
// strength (beta/2 inside the joint solve, from the zero state); the forward state of a query
// frame has absorbed the non-boundary frames of chunks <= c-2 in increasing order, the reverse
// state those of chunks >= c+2 in decreasing order.
//
// Stage 1 (stats): one block per (frame or text, head) accumulates A and B in fp32, forms I + A
// and inverts it in place by Gauss-Jordan elimination without pivoting (I + A is symmetric
// positive definite with every pivot >= 1, so no pivot is small).  Writes M = (I + A)^-1 and B.
// Stage 2 (scan): the update acts on each row of S independently (row r of the new state only
// needs row r of the old state and of B), so one block owns 16 rows of S for one (head,
// direction) and walks the frames in order, x = s Diag(alpha_f) + B_f (the decay gate, when given,
// on the key channels of the inherited state), s = x M_f, storing the state at every chunk
// boundary.  Slot Nc of each direction holds S0, read by boundary query frames.
#include "dev_common.h"
#include "vda_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

constexpr int kTileU = 32;   // tokens staged per iteration

template <typename Tin, int D>
__global__ __launch_bounds__(256) void vda_stats_simt_kernel(
    const Tin* __restrict__ k, const Tin* __restrict__ v, const float* __restrict__ beta,
    const Tin* __restrict__ text_kv, float* __restrict__ minv, float* __restrict__ bw, int T, int N, int H,
    int n_text, int n_ctx, int anchors) {
  constexpr int R = D / 16;
  const int slot = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  if (slot > 0 && anchors && (slot - 1 == 0 || slot - 1 == T - 1)) return;   // boundary frames are never written

  __shared__ float ks[kTileU][D], vs[kTileU][D], ws[kTileU];
  __shared__ float rowbuf[2 * D], colbuf[2 * D];

  const int U = slot == 0 ? n_text : N;
  const int64_t tok0 = slot == 0 ? 0 : (int64_t)(slot - 1) * N;
  const Tin* kbase = slot == 0 ? text_kv : k;
  const Tin* vbase = slot == 0 ? text_kv + (int64_t)n_ctx * H * D : v;   // V half of [2][n_ctx][H][d]
  const float wscale = slot == 0 ? 0.5f : 1.0f;
  const int64_t brow0 = slot == 0 ? 0 : n_text + tok0;

  float a[R][R], bb[R][R];
#pragma unroll
  for (int ii = 0; ii < R; ++ii)
#pragma unroll
    for (int jj = 0; jj < R; ++jj) { a[ii][jj] = 0.f; bb[ii][jj] = 0.f; }

  for (int u0 = 0; u0 < U; u0 += kTileU) {
    for (int e = tid; e < kTileU * D; e += 256) {
      const int uu = e / D, i = e % D;
      const int u = u0 + uu;
      float kv = 0.f, vv = 0.f;
      if (u < U) {
        const int64_t off = ((tok0 + u) * H + h) * D + i;
        kv = to_f32(kbase[off]);
        vv = to_f32(vbase[off]);
      }
      ks[uu][i] = kv;
      vs[uu][i] = vv;
    }
    if (tid < kTileU) {
      const int u = u0 + tid;
      ws[tid] = u < U ? wscale * beta[(brow0 + u) * H + h] : 0.f;
    }
    __syncthreads();
    for (int uu = 0; uu < kTileU; ++uu) {
      const float w = ws[uu];
      float ki[R], vi[R], wkj[R];
#pragma unroll
      for (int ii = 0; ii < R; ++ii) { ki[ii] = ks[uu][ty * R + ii]; vi[ii] = vs[uu][ty * R + ii]; }
#pragma unroll
      for (int jj = 0; jj < R; ++jj) wkj[jj] = w * ks[uu][tx * R + jj];
#pragma unroll
      for (int ii = 0; ii < R; ++ii)
#pragma unroll
        for (int jj = 0; jj < R; ++jj) {
          a[ii][jj] += ki[ii] * wkj[jj];
          bb[ii][jj] += vi[ii] * wkj[jj];
        }
    }
    __syncthreads();
  }

  const int64_t mbase = ((int64_t)slot * H + h) * D * D;
#pragma unroll
  for (int ii = 0; ii < R; ++ii)
#pragma unroll
    for (int jj = 0; jj < R; ++jj) {
      const int i = ty * R + ii, j = tx * R + jj;
      bw[mbase + (int64_t)i * D + j] = bb[ii][jj];
      if (i == j) a[ii][jj] += 1.0f;
    }
  gauss_jordan_inverse<D>(a, rowbuf, colbuf, ty, tx);
#pragma unroll
  for (int ii = 0; ii < R; ++ii)
#pragma unroll
    for (int jj = 0; jj < R; ++jj) minv[mbase + (int64_t)(ty * R + ii) * D + tx * R + jj] = a[ii][jj];
}

// ---------------------------------------------------------------------------------------------
// Scan
// ---------------------------------------------------------------------------------------------

constexpr int kScanRows = 16;

// s <- (s Diag(alpha) + B) M for the block's rows; alpha == nullptr means no decay
template <int D>
__device__ __forceinline__ void scan_apply(float (&s)[D / 16], float (*x)[D], const float* __restrict__ bslot,
                                           const float* __restrict__ mslot, const float* __restrict__ aslot,
                                           int row0, int r, int jc) {
  constexpr int CPT = D / 16;
#pragma unroll
  for (int cc = 0; cc < CPT; ++cc) {
    const int col = jc * CPT + cc;
    x[r][col] = (aslot ? s[cc] * aslot[col] : s[cc]) + bslot[(int64_t)(row0 + r) * D + col];
  }
  __syncthreads();
  float o[CPT];
#pragma unroll
  for (int cc = 0; cc < CPT; ++cc) o[cc] = 0.f;
  for (int i = 0; i < D; ++i) {
    const float xi = x[r][i];
    const float* mrow = mslot + (int64_t)i * D + jc * CPT;
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) o[cc] += xi * mrow[cc];
  }
  __syncthreads();
#pragma unroll
  for (int cc = 0; cc < CPT; ++cc) s[cc] = o[cc];
}

template <int D>
__global__ __launch_bounds__(256) void vda_scan_simt_kernel(const float* __restrict__ minv,
                                                            const float* __restrict__ bw,
                                                            const float* __restrict__ alpha,
                                                            float* __restrict__ states, int T, int C, int Nc, int H,
                                                            int anchors) {
  constexpr int CPT = D / 16;
  constexpr int ROWS = D < kScanRows ? D : kScanRows;
  const int rblk = blockIdx.x, dir = blockIdx.y, h = blockIdx.z;
  const int row0 = rblk * ROWS;
  const int r = threadIdx.x / 16, jc = threadIdx.x % 16;
  const bool active = r < ROWS;
  __shared__ float x[kScanRows][D];
  const int64_t DD = (int64_t)D * D;
  float s[CPT];
#pragma unroll
  for (int cc = 0; cc < CPT; ++cc) s[cc] = 0.f;
  const int rr = active ? r : 0;

  auto apply = [&](int slot) {                       // slot 0: the text; slot 1 + f: frame f
    const float* bslot = bw + ((int64_t)slot * H + h) * DD;
    const float* mslot = minv + ((int64_t)slot * H + h) * DD;
    const float* aslot = (alpha && slot > 0) ? alpha + ((int64_t)(slot - 1) * H + h) * D : nullptr;
    scan_apply<D>(s, x, bslot, mslot, aslot, row0, rr, jc);
  };
  auto store = [&](int cslot) {
    if (!active) return;
    float* dst = states + (((int64_t)dir * (Nc + 1) + cslot) * H + h) * DD + (int64_t)(row0 + r) * D + jc * CPT;
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) dst[cc] = s[cc];
  };
  auto boundary = [&](int f) { return anchors && (f == 0 || f == T - 1); };

  apply(0);          // text, written from the zero state
  store(Nc);         // S0
  if (dir == 0) {
    for (int c = 0; c < Nc; ++c) {
      if (c >= 2) {
        const int f_end = min((c - 1) * C, T);
        for (int f = (c - 2) * C; f < f_end; ++f)
          if (!boundary(f)) apply(1 + f);
      }
      store(c);
    }
  } else {
    for (int c = Nc - 1; c >= 0; --c) {
      if (c + 2 <= Nc - 1) {
        const int f_hi = min((c + 3) * C, T) - 1;
        for (int f = f_hi; f >= (c + 2) * C; --f)
          if (!boundary(f)) apply(1 + f);
      }
      store(c);
    }
  }
}

template <typename Tin, int D>
void stats_t(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  dim3 grid(s.T + 1, s.H);
  vda_stats_simt_kernel<Tin, D><<<grid, 256, 0, st>>>((const Tin*)in.k, (const Tin*)in.v, in.beta,
                                                      (const Tin*)in.text_kv, b.minv, b.bw, s.T, s.N, s.H,
                                                      s.n_text, s.n_ctx, s.anchors);
}

template <typename Tin>
void stats_d(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  switch (s.d) {
    case 16: stats_t<Tin, 16>(s, in, b, st); break;
    case 32: stats_t<Tin, 32>(s, in, b, st); break;
    case 64: stats_t<Tin, 64>(s, in, b, st); break;
    default: stats_t<Tin, 128>(s, in, b, st); break;
  }
}

template <int D>
void scan_t(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  constexpr int ROWS = D < kScanRows ? D : kScanRows;
  dim3 grid(D / ROWS, 2, s.H);
  vda_scan_simt_kernel<D><<<grid, 256, 0, st>>>(b.minv, b.bw, in.alpha, b.states, s.T, s.C, s.Nc, s.H, s.anchors);
}

}  // namespace

hipError_t launch_vda_stats(const Shape& s, const Inputs& in, const Buffers& b, bool mfma, hipStream_t st) {
  if (mfma) return launch_vda_stats_mfma(s, in, b, st);
  if (s.dtype == VDN_BF16) stats_d<bf16_t>(s, in, b, st);
  else stats_d<float>(s, in, b, st);
  return hipGetLastError();
}

hipError_t launch_vda_scan(const Shape& s, const Inputs& in, const Buffers& b, bool mfma, hipStream_t st) {
  if (mfma) return launch_vda_scan_mfma(s, in, b, st);
  switch (s.d) {
    case 16: scan_t<16>(s, in, b, st); break;
    case 32: scan_t<32>(s, in, b, st); break;
    case 64: scan_t<64>(s, in, b, st); break;
    default: scan_t<128>(s, in, b, st); break;
  }
  return hipGetLastError();
}

}  // namespace vdn
