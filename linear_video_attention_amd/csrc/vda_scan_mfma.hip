// Chunk maps and chunk-level state scans of Video Delta Attention (bf16 plans, d in {64, 128}).
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Video Delta
// Attention: A Frame-Wise Solution": each frame updates the state as
// S <- (S Diag(alpha_f) + B_f) M_f = S G_f + C_f with G_f = Diag(alpha_f) M_f (the decay gate on
// the inherited state; alpha = 1 without it), M_f = (I + A_f)^-1 symmetric, C_f = B_f M_f.
// Section "Local Softmax and Long-Range Linear Memory": both directions start from the text state
// S0 = C_0; the forward state of a query frame in chunk c has absorbed, in increasing order, the
// non-boundary frames of chunks <= c-2, the reverse state, in decreasing order, those of chunks
// >= c+2.  Only whole chunks ever enter a state, so the frames of a chunk compose into one affine
// map S -> S P + Q:
//   forward  (increasing frames f1 < ... < fm):  P> = G_f1 ... G_fm,  Q> = (..(C_f1 G_f2 + C_f2) ..) + C_fm
//   reverse  (decreasing frames):                P< = G_fm ... G_f1,  Q< likewise from C_fm down
// (without decay P< = P>^T, the M_f being symmetric, so P< needs no chain of its own), and the
// states follow from a scan over chunks:
//   S>_0 = S>_1 = S0,  S>_c = S>_{c-1} P>_{c-2} + Q>_{c-2};   S<_{Nc-1} = S<_{Nc-2} = S0,
//   S<_c = S<_{c+1} P<_{c+2} + Q<_{c+2}.
//
// Two kernels, both built on the same row-chain step: row r of X M + Q depends only on row r of X,
// so a workgroup owns 16 RT rows and walks its steps; each of its D/16 waves produces 16 output
// columns with v_mfma_f32_16x16x32_bf16, both operands as bf16 high and low parts,
// x M ~ xh Mh + xh Ml + xl Mh (relative error ~2^-16).  The right-hand matrix arrives split (two
// bf16 planes holding its transpose row by row, so a lane's k-run is contiguous); the running rows
// are kept in LDS as their two bf16 planes (double buffered: one barrier per step) and the fp32
// accumulator is what gets stored.
//   * vda_compose_kernel: every (chunk, head, map part) in parallel: P>, Q>, Q< (fp32), and P<
//     with a decay gate; the maps are written as the planes of their transposes (the scan's
//     operand layout), P> also as its own planes (= P<^T) without decay.  At most C-1 steps each.
//   * vda_chunk_scan_kernel: one workgroup per (head, direction, 16 rows) walks the Nc-2 chunk
//     steps with the operands of the next two steps in flight, storing one state slot per step.
//     Slot Nc of each direction receives S0 (read by boundary query frames).
#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ __forceinline__ bool is_bnd(int f, int T, int anchors) { return anchors && (f == 0 || f == T - 1); }

// One step's operands for one wave: its 16 columns of the right-hand matrix (planes hi and lo,
// k = ks*32 + lg*8 .. +8) and its RT x 4 elements of the additive term (rows 16 rt + 4 lg + i).
template <int D, int RT>
struct StepOps {
  bf16x8 mh[D / 32], ml[D / 32];
  f32x4 c[RT];
};

// Rows [row0, row0 + 16 RT) in LDS as two bf16 planes, double buffered.
template <int D, int RT>
struct RowPlanes {
  static constexpr int LDX = D + 8;                   // bf16 row stride
  bf16_t hi[2][16 * RT][LDX];
  bf16_t lo[2][16 * RT][LDX];
};

// mt: the transpose of the right-hand matrix as two bf16 planes [2][D][D], row n = column n.
template <int D, int RT>
__device__ __forceinline__ void load_mat(StepOps<D, RT>& op, const bf16_t* __restrict__ mt, int col, int lg) {
  const bf16_t* p = mt + (int64_t)col * D + lg * 8;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    op.mh[ks] = *reinterpret_cast<const bf16x8*>(p + ks * 32);
    op.ml[ks] = *reinterpret_cast<const bf16x8*>(p + (int64_t)D * D + ks * 32);
  }
}

template <int D, int RT>
__device__ __forceinline__ void load_add(StepOps<D, RT>& op, const float* __restrict__ add, int row0, int col, int lg) {
  const float* a = add + (int64_t)(row0 + 4 * lg) * D + col;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) op.c[rt][i] = a[(16 * rt + i) * D];
}

template <int D, int RT>
__device__ __forceinline__ void put_rows(RowPlanes<D, RT>& s, int buf, const f32x4 (&acc)[RT], int col, int lg) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 xh = (__bf16)acc[rt][i];
      s.hi[buf][16 * rt + 4 * lg + i][col] = __builtin_bit_cast(bf16_t, xh);
      s.lo[buf][16 * rt + 4 * lg + i][col] = __builtin_bit_cast(bf16_t, (__bf16)(acc[rt][i] - (float)xh));
    }
}

// acc = rows(s[buf]) x M (+ the additive term already in op.c)
template <int D, int RT>
__device__ __forceinline__ void step_product(const RowPlanes<D, RT>& s, int buf, const StepOps<D, RT>& op,
                                             f32x4 (&acc)[RT], int l16, int lg) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    f32x4 a0 = op.c[rt], a1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const bf16x8 xh = *reinterpret_cast<const bf16x8*>(&s.hi[buf][16 * rt + l16][ks * 32 + lg * 8]);
      const bf16x8 xl = *reinterpret_cast<const bf16x8*>(&s.lo[buf][16 * rt + l16][ks * 32 + lg * 8]);
      a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, op.mh[ks], a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, op.ml[ks], a1, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl, op.mh[ks], a1, 0, 0, 0);
    }
    acc[rt] = a0 + a1;
  }
}

constexpr int kComposeRT = 2;      // 32 rows per compose workgroup

// blockIdx.x = part * RB + rb (part 0: P>, 1: Q>, 2: Q<, 3: P< (decay only)), blockIdx.y = chunk,
// blockIdx.z = head.  mhl holds each frame's step planes (G_f^T by rows, see the inverse kernel).
template <int D>
__global__ __launch_bounds__(D * 4) void vda_compose_kernel(const float* __restrict__ minv,
                                                            const bf16_t* __restrict__ mhl,
                                                            const float* __restrict__ cw,
                                                            const float* __restrict__ alpha,
                                                            bf16_t* __restrict__ pp, float* __restrict__ qq, int T,
                                                            int C, int Nc, int H, int anchors) {
  constexpr int RT = kComposeRT;
  constexpr int RB = D / (16 * RT);
  __shared__ __attribute__((aligned(16))) RowPlanes<D, RT> s;
  const int part = blockIdx.x / RB, rb = blockIdx.x % RB, j = blockIdx.y, h = blockIdx.z;
  const int row0 = rb * 16 * RT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int col = wave * 16 + l16;
  const int64_t DD = (int64_t)D * D;

  const bool is_p = part == 0 || part == 3;
  const bool decreasing = part >= 2;
  // the chunk's scanned frames, in this part's order (P>, Q> increasing; Q<, P< decreasing)
  const int f_lo = j * C, f_hi = min(f_lo + C, T);
  int m = 0;
  for (int f = f_lo; f < f_hi; ++f) m += is_bnd(f, T, anchors) ? 0 : 1;
  auto frame_at = [&](int a) {                       // a-th scanned frame of the chunk in this order
    int f = decreasing ? f_hi - 1 : f_lo;
    const int step = decreasing ? -1 : 1;
    for (int seen = 0;; f += step)
      if (!is_bnd(f, T, anchors) && seen++ == a) return f;
  };

  f32x4 acc[RT];
  if (m == 0) {                                      // identity map: P = I, Q = 0
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[rt][i] = (is_p && row0 + 16 * rt + 4 * lg + i == col) ? 1.f : 0.f;
  } else {
    // first frame's map: rows of G = Diag(alpha) M (row r of M times alpha[r]) or of C
    const int f1 = frame_at(0);
    const float* x0 = (is_p ? minv : cw) + ((int64_t)(1 + f1) * H + h) * DD;
    const float* a1 = (is_p && alpha) ? alpha + ((int64_t)f1 * H + h) * D : nullptr;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row0 + 16 * rt + 4 * lg + i;
        acc[rt][i] = x0[(int64_t)r * D + col] * (a1 ? a1[r] : 1.f);
      }
  }
  int buf = 0;
  put_rows<D, RT>(s, buf, acc, col, lg);
  for (int a = 1; a < m; ++a) {
    StepOps<D, RT> op;
    const int64_t slot = (int64_t)(1 + frame_at(a)) * H + h;
    load_mat<D, RT>(op, mhl + slot * 2 * DD, col, lg);
    if (is_p) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) op.c[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
      load_add<D, RT>(op, cw + slot * DD, row0, col, lg);
    }
    __syncthreads();                                 // rows of s[buf] complete
    step_product<D, RT>(s, buf, op, acc, l16, lg);
    buf ^= 1;
    put_rows<D, RT>(s, buf, acc, col, lg);
  }

  const int64_t ph = (int64_t)j * H + h;
  if (is_p) {
    // pp[chunk][head][layout][plane][D][D]: layout 1 = P>^T (operand of the forward scan),
    // layout 0 = P<^T (reverse scan); without decay P<^T = P>, written by the P> chain directly
    bf16_t* p = pp + ph * 4 * DD;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row0 + 16 * rt + 4 * lg + i;
        const __bf16 xh = (__bf16)acc[rt][i];
        const bf16_t hb = __builtin_bit_cast(bf16_t, xh);
        const bf16_t lb = __builtin_bit_cast(bf16_t, (__bf16)(acc[rt][i] - (float)xh));
        if (part == 0 && !alpha) {
          p[(int64_t)r * D + col] = hb;
          p[DD + (int64_t)r * D + col] = lb;
        }
        bf16_t* t = p + (part == 0 ? 2 * DD : 0);      // transposed planes of this map
        t[(int64_t)col * D + r] = hb;
        t[DD + (int64_t)col * D + r] = lb;
      }
  } else {
    float* q = qq + ((int64_t)(part - 1) * Nc * H + ph) * DD;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) q[(int64_t)(row0 + 16 * rt + 4 * lg + i) * D + col] = acc[rt][i];
  }
}

template <int D>
__global__ __launch_bounds__(D * 4) void vda_chunk_scan_kernel(const float* __restrict__ cw,
                                                               const bf16_t* __restrict__ pp,
                                                               const float* __restrict__ qq,
                                                               float* __restrict__ states, int Nc, int H,
                                                               int n_chains, int per_xcd) {
  constexpr int RB = D / 16;                         // row blocks per (head, direction)
  __shared__ __attribute__((aligned(16))) RowPlanes<D, 1> s;
  // workgroup -> (head, direction, row block), the row blocks of one chain on one XCD
  const int w = blockIdx.x;
  const int L = (w & 7) * per_xcd + (w >> 3);
  if (L >= n_chains * RB) return;
  const int chain = L / RB, rb = L % RB;
  const int h = chain >> 1, dir = chain & 1;
  const int row0 = rb * 16;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int col = wave * 16 + l16;
  const int64_t DD = (int64_t)D * D;

  auto store = [&](int cslot, const f32x4& a) {
    float* dst = states + (((int64_t)dir * (Nc + 1) + cslot) * H + h) * DD + (int64_t)(row0 + 4 * lg) * D + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i * D] = a[i];
  };
  // step k applies chunk j(k) and yields slot j(k) + 2 (forward) / j(k) - 2 (reverse)
  const int n_steps = max(Nc - 2, 0);
  auto load = [&](StepOps<D, 1>& op, int k) {        // past the last step: a harmless reload of step 0
    const int kk = k < n_steps ? k : 0;
    const int j = dir == 0 ? kk : Nc - 1 - kk;
    const int64_t ph = (int64_t)j * H + h;
    // forward applies P> (planes of P>^T give its columns), reverse applies P< (planes of P<^T)
    load_mat<D, 1>(op, pp + ph * 4 * DD + (dir == 0 ? 2 * DD : 0), col, lg);
    load_add<D, 1>(op, qq + ((int64_t)dir * Nc * H + ph) * DD, row0, col, lg);
  };

  f32x4 acca[1], accb[1];
  {
    const float* cp = cw + (int64_t)h * DD + (int64_t)(row0 + 4 * lg) * D + col;   // S0 = C_0
#pragma unroll
    for (int i = 0; i < 4; ++i) accb[0][i] = cp[i * D];
  }
  int buf = 0;
  put_rows<D, 1>(s, buf, accb, col, lg);
  for (int c = 0; c < min(Nc, 2); ++c) store(dir == 0 ? c : Nc - 1 - c, accb[0]);

  // The steps run in pairs with the operands of the next two steps in flight.  Each step issues
  // exactly one store, before the next operand loads, and results alternate between two
  // accumulators (the store of one is never overwritten by the next step): the compiler can then
  // keep the loads in flight across the following steps.  The prologue follows the same pattern
  // (loads, one store, loads).
  StepOps<D, 1> opa, opb;
  load(opa, 0);
  asm volatile("" ::: "memory");
  store(Nc, accb[0]);
  asm volatile("" ::: "memory");
  load(opb, 1);
  asm volatile("" ::: "memory");
  auto apply = [&](const StepOps<D, 1>& op, f32x4 (&acc)[1]) {
    __syncthreads();                                 // rows of s[buf] complete
    step_product<D, 1>(s, buf, op, acc, l16, lg);
    buf ^= 1;
    put_rows<D, 1>(s, buf, acc, col, lg);
  };
  auto slot_after = [&](int k) { return dir == 0 ? k + 2 : Nc - 3 - k; };
  int k = 0;
  for (; k + 1 < n_steps; k += 2) {
    apply(opa, acca);
    asm volatile("" ::"v"(accb[0]));                 // the store of accb may still be reading it
    store(slot_after(k), acca[0]);
    asm volatile("" ::: "memory");
    load(opa, k + 2);
    asm volatile("" ::: "memory");
    apply(opb, accb);
    asm volatile("" ::"v"(acca[0]));
    store(slot_after(k + 1), accb[0]);
    asm volatile("" ::: "memory");
    load(opb, k + 3);
    asm volatile("" ::: "memory");
  }
  if (k < n_steps) {
    apply(opa, acca);
    store(slot_after(k), acca[0]);
  }
}

template <int D>
void launch_t(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  constexpr int RB = D / (16 * kComposeRT);
  const int parts = in.alpha ? 4 : 3;
  vda_compose_kernel<D><<<dim3(parts * RB, s.Nc, s.H), D * 4, 0, st>>>(b.minv, b.mhl, b.cw, in.alpha, b.pp, b.qq, s.T,
                                                                      s.C, s.Nc, s.H, s.anchors);
  // the row blocks of one (head, direction) stay on one XCD: per_xcd is a multiple of D / 16
  const int n_chains = 2 * s.H;
  const int per_xcd = (n_chains + 7) / 8 * (D / 16);
  vda_chunk_scan_kernel<D><<<8 * per_xcd, D * 4, 0, st>>>(b.cw, b.pp, b.qq, b.states, s.Nc, s.H, n_chains, per_xcd);
}

}  // namespace

hipError_t launch_vda_scan_mfma(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  if (s.d == 128) launch_t<128>(s, in, b, st);
  else launch_t<64>(s, in, b, st);
  return hipGetLastError();
}

}  // namespace vdn
