// MFMA state scans of Video Delta Attention (bf16 plans, d in {64, 128}).
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Video Delta
// Attention: A Frame-Wise Solution": each frame updates the state as S <- (S + B_f) M_f with
// M_f = (I + A_f)^-1, i.e. S <- S M_f + C_f with C_f = B_f M_f.  Section "Local Softmax and
// Long-Range Linear Memory": both directions start from the text state S0 = C_0 (the text written
// from the zero state); the forward state of a query frame in chunk c has absorbed, in increasing
// order, the non-boundary frames of chunks <= c-2, the reverse state, in decreasing order, those
// of chunks >= c+2.
//
// Two kernels:
//   * vda_cmul_kernel: C_f = B_f M_f for every frame (and the text), all frames in parallel;
//   * vda_scan_kernel: row r of the new state depends only on row r of the old state (and of C_f),
//     so the rows split into independent chains.  One workgroup owns 32 rows of one (head,
//     direction) and walks the frames; its 8 waves each produce 16 output columns.  The state lives
//     in LDS (fp32, double buffered: one barrier per frame); the wave's slice of M_f (read by rows
//     through M^T = M) and its tile of C_f are prefetched two frames ahead in registers.  The
//     workgroups of one (head, direction) are placed on one XCD so the frame's M_f is fetched into
//     that XCD's L2 once for all of them.
// Products run on v_mfma_f32_16x16x32_bf16 with both operands split into bf16 high and low parts,
// x M ~ xh Mh + xh Ml + xl Mh (relative error ~2^-16).
#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kRows = 32;          // state rows per workgroup (two 16-row MFMA tiles)

__device__ __forceinline__ void split8(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = e < 4 ? a[e] : b[e - 4];
    const __bf16 xh = (__bf16)x;
    hi[e] = xh;
    lo[e] = (__bf16)(x - (float)xh);
  }
}

// Operands of one step for one wave: its 16 columns of the right-hand matrix (by rows, k =
// ks*32 + lg*8 .. +8) and its 2 x 4 outputs of the additive term.
template <int D>
struct StepOps {
  f32x4 m[D / 32][2];
  f32x4 c[2];
};

template <int D>
__device__ __forceinline__ void load_mat(StepOps<D>& op, const float* __restrict__ mat, int col, int lg) {
  constexpr int KS = D / 32;
  const float* mr = mat + (int64_t)col * D + lg * 8;      // row `col` of the symmetric matrix
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    op.m[ks][0] = *reinterpret_cast<const f32x4*>(mr + ks * 32);
    op.m[ks][1] = *reinterpret_cast<const f32x4*>(mr + ks * 32 + 4);
  }
}

// additive term at (row0 + 16 rt + 4 lg + i, col), i = 0..3
template <int D>
__device__ __forceinline__ void load_add(StepOps<D>& op, const float* __restrict__ add, int row0, int col, int lg) {
  const float* a = add + (int64_t)(row0 + 4 * lg) * D + col;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) op.c[rt][i] = a[(16 * rt + i) * D];
}

// out[rt][i] = sum_k x[16 rt + 4 lg + i][k] * mat[k][col]  (+ additive term), x in LDS (fp32)
template <int D>
__device__ __forceinline__ void step_product(const float* __restrict__ x_lds, int ldx, const StepOps<D>& op,
                                             int l16, int lg, f32x4 (&acc)[2]) {
  constexpr int KS = D / 32;
  bf16x8 mh[KS], ml[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) split8(op.m[ks][0], op.m[ks][1], mh[ks], ml[ks]);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    acc[rt] = op.c[rt];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float* xr = x_lds + (16 * rt + l16) * ldx + ks * 32 + lg * 8;
      bf16x8 xh, xl;
      split8(*reinterpret_cast<const f32x4*>(xr), *reinterpret_cast<const f32x4*>(xr + 4), xh, xl);
      acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, mh[ks], acc[rt], 0, 0, 0);
      acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, ml[ks], acc[rt], 0, 0, 0);
      acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl, mh[ks], acc[rt], 0, 0, 0);
    }
  }
}

// C_f = B_f M_f for every slot (text = 0, frame f = 1 + f); boundary frames are skipped.
template <int D>
__global__ __launch_bounds__(D * 4) void vda_cmul_kernel(const float* __restrict__ minv, const float* __restrict__ bw,
                                                         float* __restrict__ cw, int T, int H, int anchors) {
  constexpr int LDX = D + 4;
  __shared__ __attribute__((aligned(16))) float x_lds[kRows][LDX];
  const int row0 = blockIdx.x * kRows, slot = blockIdx.y, h = blockIdx.z;
  if (slot > 0 && anchors && (slot - 1 == 0 || slot - 1 == T - 1)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  const int col = wave * 16 + l16;
  const int64_t base = ((int64_t)slot * H + h) * D * D;
  for (int e = tid; e < kRows * D / 4; e += blockDim.x) {
    const int r = e / (D / 4), c4 = e % (D / 4);
    *reinterpret_cast<f32x4*>(&x_lds[r][c4 * 4]) = *reinterpret_cast<const f32x4*>(bw + base + (int64_t)(row0 + r) * D + c4 * 4);
  }
  StepOps<D> op;
  load_mat<D>(op, minv + base, col, lg);
  op.c[0] = op.c[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  f32x4 acc[2];
  step_product<D>(&x_lds[0][0], LDX, op, l16, lg, acc);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) cw[base + (int64_t)(row0 + 16 * rt + 4 * lg + i) * D + col] = acc[rt][i];
}

template <int D>
__global__ __launch_bounds__(D * 4) void vda_scan_kernel(const float* __restrict__ minv, const float* __restrict__ cw,
                                                         float* __restrict__ states, int T, int C, int Nc, int H,
                                                         int anchors, int n_chains, int per_xcd) {
  constexpr int LDX = D + 4;
  constexpr int RB = D / kRows;                       // row blocks per (head, direction)
  __shared__ __attribute__((aligned(16))) float s_lds[2][kRows][LDX];
  // workgroup -> (head, direction, row block), the row blocks of one chain on one XCD
  const int w = blockIdx.x;
  const int L = (w & 7) * per_xcd + (w >> 3);
  if (L >= n_chains * RB) return;
  const int chain = L / RB, rb = L % RB;
  const int h = chain >> 1, dir = chain & 1;
  const int row0 = rb * kRows;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  const int col = wave * 16 + l16;
  const int64_t DD = (int64_t)D * D;
  auto mat_of = [&](int slot) { return minv + ((int64_t)slot * H + h) * DD; };
  auto add_of = [&](int slot) { return cw + ((int64_t)slot * H + h) * DD; };
  auto boundary = [&](int f) { return anchors && (f == 0 || f == T - 1); };
  auto next_frame = [&](int f) {                       // next frame this direction writes, or -1
    const int step = dir == 0 ? 1 : -1;
    for (f += step; f >= 0 && f < T; f += step)
      if (!boundary(f)) return f;
    return -1;
  };

  // S0 = C_0 (rows of this block) -> LDS buffer 0 and state slot Nc
  f32x4 acc[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rt + 4 * lg + i;
      acc[rt][i] = add_of(0)[(int64_t)(row0 + r) * D + col];
      s_lds[0][r][col] = acc[rt][i];
    }
  auto store = [&](int cslot) {
    float* dst = states + (((int64_t)dir * (Nc + 1) + cslot) * H + h) * DD + (int64_t)row0 * D + col;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(int64_t)(16 * rt + 4 * lg + i) * D] = acc[rt][i];
  };
  store(Nc);

  // Frames are applied in scan order with the operands of the next two frames in flight.  A chunk
  // slot is stored as soon as the next frame to apply is not part of its state: forward chunk c
  // holds the scanned frames of chunks <= c-2 (frames < (c-1) C), reverse chunk c those of chunks
  // >= c+2 (frames >= (c+2) C).
  int next_c = dir == 0 ? 0 : Nc - 1;
  auto store_before = [&](int f) {                     // f = next frame to apply, -1 at the end
    if (dir == 0) {
      while (next_c < Nc && (f < 0 || (next_c - 1) * C <= f)) store(next_c++);
    } else {
      while (next_c >= 0 && (f < 0 || f < (next_c + 2) * C)) store(next_c--);
    }
  };
  int buf = 0;
  auto apply = [&](const StepOps<D>& op) {
    __syncthreads();                                   // state in s_lds[buf] complete
    step_product<D>(&s_lds[buf][0][0], LDX, op, l16, lg, acc);
    buf ^= 1;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_lds[buf][16 * rt + 4 * lg + i][col] = acc[rt][i];
  };
  auto load = [&](StepOps<D>& op, int f) {              // past the last frame: a harmless reload
    const int slot = f >= 0 ? 1 + f : 0;
    load_mat<D>(op, mat_of(slot), col, lg);
    load_add<D>(op, add_of(slot), row0, col, lg);
  };
  int f0 = next_frame(dir == 0 ? -1 : T);
  int f1 = f0 >= 0 ? next_frame(f0) : -1;
  StepOps<D> opa, opb;                                 // operands of f0 and f1
  load(opa, f0);
  load(opb, f1);
  while (f0 >= 0) {
    store_before(f0);
    const int f2 = f1 >= 0 ? next_frame(f1) : -1;
    apply(opa);
    load(opa, f2);
    if (f1 < 0) break;
    store_before(f1);
    const int f3 = f2 >= 0 ? next_frame(f2) : -1;
    apply(opb);
    load(opb, f3);
    f0 = f2;
    f1 = f3;
  }
  store_before(-1);
}

template <int D>
void launch_t(const Shape& s, const Buffers& b, hipStream_t st) {
  vda_cmul_kernel<D><<<dim3(D / kRows, s.T + 1, s.H), D * 4, 0, st>>>(b.minv, b.bw, b.cw, s.T, s.H, s.anchors);
  // the row blocks of one (head, direction) stay on one XCD: per_xcd is a multiple of D / kRows
  const int n_chains = 2 * s.H;
  const int per_xcd = (n_chains + 7) / 8 * (D / kRows);
  vda_scan_kernel<D><<<8 * per_xcd, D * 4, 0, st>>>(b.minv, b.cw, b.states, s.T, s.C, s.Nc, s.H, s.anchors, n_chains,
                                                    per_xcd);
}

}  // namespace

hipError_t launch_vda_scan_mfma(const Shape& s, const Buffers& b, hipStream_t st) {
  if (s.d == 128) launch_t<128>(s, b, st);
  else launch_t<64>(s, b, st);
  return hipGetLastError();
}

}  // namespace vdn
