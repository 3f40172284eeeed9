// MFMA state scans of Video Delta Attention (bf16 plans, d in {64, 128}).
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Video Delta
// Attention: A Frame-Wise Solution": each frame updates the state as S <- (S + B_f) M_f =
// S M_f + C_f.  Section "Local Softmax and Long-Range Linear Memory": both directions start from
// the text state S0 = C_0 (the text written from the zero state); the forward state of a query
// frame in chunk c has absorbed, in increasing order, the non-boundary frames of chunks <= c-2, the
// reverse state, in decreasing order, those of chunks >= c+2.
//
// Row r of the new state depends only on row r of the old state (and of C_f), so the rows split
// into independent chains.  One workgroup owns kRows rows of one (head, direction) and walks the
// frames; each of its D/16 waves produces 16 output columns.  The product runs on
// v_mfma_f32_16x16x32_bf16 with both operands in bf16 high and low parts,
// x M ~ xh Mh + xh Ml + xl Mh (relative error ~2^-16): M_f arrives already split (two bf16
// planes, read by rows through M^T = M), and the state is kept in LDS as its two bf16 planes
// (double buffered: one barrier per frame), split once by the wave that produced it; the fp32
// accumulator is what gets stored.  The operands of the next two frames are in flight while the
// current one is multiplied.  The workgroups of one (head, direction) are placed on one XCD so
// each frame's M_f is fetched into that XCD's L2 once for all of them.
#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kRows = 16;          // state rows per workgroup (one 16-row MFMA tile)

// Operands of one frame for one wave: its 16 columns of Mh and Ml (k = ks*32 + lg*8 .. +8) and its
// 4 elements of C_f (rows 4 lg + i, column col).
template <int D>
struct StepOps {
  bf16x8 mh[D / 32], ml[D / 32];
  f32x4 c;
};

template <int D>
__global__ __launch_bounds__(D * 4) void vda_scan_kernel(const bf16_t* __restrict__ mhl, const float* __restrict__ cw,
                                                         float* __restrict__ states, float* __restrict__ sink, int T,
                                                         int C, int Nc, int H, int anchors, int n_chains,
                                                         int per_xcd) {
  constexpr int KS = D / 32;
  constexpr int LDX = D + 8;                          // bf16 row stride of the state planes
  constexpr int RB = D / kRows;                       // row blocks per (head, direction)
  __shared__ __attribute__((aligned(16))) bf16_t s_hi[2][kRows][LDX];
  __shared__ __attribute__((aligned(16))) bf16_t s_lo[2][kRows][LDX];
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
  // next frame this direction writes after f (start: f = -1 forward, T reverse), or -1; only
  // frames 0 and T-1 are ever skipped (the boundary frames)
  auto next_frame = [&](int f) {
    if (dir == 0) {
      int n = f + 1;
      n = (anchors && n == 0) ? 1 : n;
      return (n >= T || (anchors && n == T - 1)) ? -1 : n;
    }
    int n = f - 1;
    n = (anchors && n == T - 1) ? T - 2 : n;
    return (n < 0 || (anchors && n == 0)) ? -1 : n;
  };
  auto load = [&](StepOps<D>& op, int f) {            // past the last frame: a harmless reload
    const int slot = f >= 0 ? 1 + f : 0;
    const bf16_t* mp = mhl + ((int64_t)slot * H + h) * 2 * DD + (int64_t)col * D + lg * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      op.mh[ks] = *reinterpret_cast<const bf16x8*>(mp + ks * 32);
      op.ml[ks] = *reinterpret_cast<const bf16x8*>(mp + DD + ks * 32);
    }
    const float* cp = cw + ((int64_t)slot * H + h) * DD + (int64_t)(row0 + 4 * lg) * D + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) op.c[i] = cp[i * D];
  };

  int buf = 0;
  auto put_state = [&](const f32x4& acc) {             // acc -> planes of s[buf]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 xh = (__bf16)acc[i];
      s_hi[buf][4 * lg + i][col] = __builtin_bit_cast(bf16_t, xh);
      s_lo[buf][4 * lg + i][col] = __builtin_bit_cast(bf16_t, (__bf16)(acc[i] - (float)xh));
    }
  };
  auto store = [&](int cslot, const f32x4& acc) {
    float* dst = states + (((int64_t)dir * (Nc + 1) + cslot) * H + h) * DD + (int64_t)(row0 + 4 * lg) * D + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i * D] = acc[i];
  };
  auto apply = [&](const StepOps<D>& op, f32x4& acc) {
    __syncthreads();                                   // planes of s[buf] complete
    f32x4 a0 = op.c, a1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 xh = *reinterpret_cast<const bf16x8*>(&s_hi[buf][l16][ks * 32 + lg * 8]);
      const bf16x8 xl = *reinterpret_cast<const bf16x8*>(&s_lo[buf][l16][ks * 32 + lg * 8]);
      a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, op.mh[ks], a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, op.ml[ks], a1, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl, op.mh[ks], a1, 0, 0, 0);
    }
    acc = a0 + a1;
    buf ^= 1;
    put_state(acc);
  };

  // S0 = C_0 -> planes and state slot Nc.  Results alternate between two accumulators, so a frame
  // never overwrites the registers that the store of the previous frame's result reads.
  f32x4 acca, accb;
  {
    const float* cp = cw + (int64_t)h * DD + (int64_t)(row0 + 4 * lg) * D + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) accb[i] = cp[i * D];
    put_state(accb);
    store(Nc, accb);
  }

  // Frames are applied in scan order.  A chunk slot is stored as soon as the next frame to apply is
  // not part of its state: forward chunk c holds the scanned frames of chunks <= c-2 (frames
  // < (c-1) C), reverse chunk c those of chunks >= c+2 (frames >= (c+2) C).
  int next_c = dir == 0 ? 0 : Nc - 1;
  auto due = [&](int f) {                              // slot next_c is complete before frame f
    return dir == 0 ? (next_c < Nc && (f < 0 || (next_c - 1) * C <= f))
                    : (next_c >= 0 && (f < 0 || f < (next_c + 2) * C));
  };
  // Inside the frame loop consecutive scanned frames are adjacent (only frames 0 and T-1 are ever
  // skipped), so at most one slot falls due per frame.  Every frame issues exactly one store,
  // to the slot that fell due or else to the sink: a fixed number of memory operations per frame
  // lets the operand loads of the next two frames stay in flight across it.
  auto store_one = [&](int f, const f32x4& acc) {
    const bool take = due(f);
    float* dst = take ? states + (((int64_t)dir * (Nc + 1) + next_c) * H + h) * DD : sink;
    dst += (int64_t)(row0 + 4 * lg) * D + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i * D] = acc[i];
    next_c += take ? (dir == 0 ? 1 : -1) : 0;
  };
  int f0 = next_frame(dir == 0 ? -1 : T);
  while (due(f0)) store(dir == 0 ? next_c++ : next_c--, accb);   // slots holding S0 only
  int f1 = f0 >= 0 ? next_frame(f0) : -1;
  StepOps<D> opa, opb;                                 // operands of f0 and f1
  load(opa, f0);
  {                                                    // the loop's pattern: a store between loads
    float* dst = sink + (int64_t)(row0 + 4 * lg) * D + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i * D] = accb[i];
  }
  asm volatile("" ::: "memory");
  load(opb, f1);
  asm volatile("" ::: "memory");
  // Each frame's store is issued before the next operand loads, and the loop over frame pairs has
  // a single exit: the compiler then keeps those loads in flight across the following frames.
  const int n_frames = anchors ? max(T - 2, 0) : T;
  for (int pair = 0; pair < n_frames / 2; ++pair) {
    const int f2 = f1 >= 0 ? next_frame(f1) : -1;
    apply(opa, acca);
    asm volatile("" ::"v"(accb));                      // the store of accb may still be reading it
    store_one(f1, acca);
    asm volatile("" ::: "memory");                     // memory operations stay in this order
    load(opa, f2);
    asm volatile("" ::: "memory");
    const int f3 = f2 >= 0 ? next_frame(f2) : -1;
    apply(opb, accb);
    asm volatile("" ::"v"(acca));
    store_one(f2, accb);
    asm volatile("" ::: "memory");
    load(opb, f3);
    asm volatile("" ::: "memory");
    f0 = f2;
    f1 = f3;
  }
  if (n_frames & 1) {
    apply(opa, acca);
    accb = acca;
  }
  while (due(-1)) store(dir == 0 ? next_c++ : next_c--, accb);   // accb: the last result
}

template <int D>
void launch_t(const Shape& s, const Buffers& b, hipStream_t st) {
  // the row blocks of one (head, direction) stay on one XCD: per_xcd is a multiple of D / kRows
  const int n_chains = 2 * s.H;
  const int per_xcd = (n_chains + 7) / 8 * (D / kRows);
  vda_scan_kernel<D><<<8 * per_xcd, D * 4, 0, st>>>(b.mhl, b.cw, b.states, b.sink, s.T, s.C, s.Nc, s.H, s.anchors, n_chains,
                                                    per_xcd);
}

}  // namespace

hipError_t launch_vda_scan_mfma(const Shape& s, const Buffers& b, hipStream_t st) {
  if (s.d == 128) launch_t<128>(s, b, st);
  else launch_t<64>(s, b, st);
  return hipGetLastError();
}

}  // namespace vdn
