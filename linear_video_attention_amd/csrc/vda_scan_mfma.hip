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
// so a workgroup owns 16 RT rows (the compose kernel: all D of them) and walks its steps; each of
// its D/16 waves produces 16 output columns with v_mfma_f32_16x16x32_bf16, both operands as bf16
// high and low parts, x M ~ xh Mh + xh Ml + xl Mh (relative error ~2^-16).  The right-hand matrix
// arrives split (two bf16 planes holding its transpose row by row, so a lane's k-run is
// contiguous); the running rows are kept in LDS as their two bf16 planes (double buffered: one
// barrier per step) and the fp32 accumulator is what gets stored.
//   * vda_compose_kernel: every (chunk, head, map part) in parallel, one workgroup over all D rows
//     (each frame's step planes are loaded once, the next frame's during the current step): P>,
//     Q>, Q< (fp32), and P< with a decay gate; the maps are written as the planes of their
//     transposes (the scan's operand layout), P> also as its own planes (= P<^T) without decay.
//     At most C-1 steps each.
//   * vda_chunk_scan_kernel: one workgroup per (head, direction, 16 rows) walks the Nc-2 chunk
//     steps, the next step's matrix copied into LDS (DMA, two stages) during the current step's
//     product, storing one state slot per step.
//     Slot Nc of each direction receives S0 (read by boundary query frames).
#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

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

// blockIdx.x = part (0: P>, 1: Q>, 2: Q<, 3: P< (decay only)), blockIdx.y = chunk, blockIdx.z =
// head; the workgroup computes the whole D x D map, so each frame's step planes are loaded once per
// (chunk, head, part).  mhl holds each frame's step planes (G_f^T by rows, see the inverse kernel).
template <int D>
__global__ __launch_bounds__(D * 4) void vda_compose_kernel(const float* __restrict__ minv,
                                                            const bf16_t* __restrict__ mhl,
                                                            const float* __restrict__ cw,
                                                            const float* __restrict__ alpha,
                                                            bf16_t* __restrict__ pp, float* __restrict__ qq, int T,
                                                            int C, int Nc, int H, int anchors) {
  constexpr int RT = D / 16;                         // every row of the map: D / 16 row tiles per wave
  __shared__ __attribute__((aligned(16))) RowPlanes<D, RT> s;
  const int part = blockIdx.x, j = blockIdx.y, h = blockIdx.z;
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
      for (int i = 0; i < 4; ++i) acc[rt][i] = (is_p && 16 * rt + 4 * lg + i == col) ? 1.f : 0.f;
  } else {
    // first frame's map: rows of G = Diag(alpha) M (row r of M times alpha[r]) or of C
    const int f1 = frame_at(0);
    const float* x0 = (is_p ? minv : cw) + ((int64_t)(1 + f1) * H + h) * DD;
    const float* a1 = (is_p && alpha) ? alpha + ((int64_t)f1 * H + h) * D : nullptr;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * lg + i;
        acc[rt][i] = x0[(int64_t)r * D + col] * (a1 ? a1[r] : 1.f);
      }
  }
  int buf = 0;
  put_rows<D, RT>(s, buf, acc, col, lg);
  StepOps<D, RT> op;
  auto load_step = [&](int a) {                      // operands of frame a of the chain
    const int64_t slot = (int64_t)(1 + frame_at(a)) * H + h;
    load_mat<D, RT>(op, mhl + slot * 2 * DD, col, lg);
    if (is_p) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) op.c[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
      load_add<D, RT>(op, cw + slot * DD, 0, col, lg);
    }
  };
  if (m > 1) load_step(1);
  for (int a = 1; a < m; ++a) {
    lds_barrier();                                   // rows of s[buf] complete (the next operands stay in flight)
    step_product<D, RT>(s, buf, op, acc, l16, lg);
    if (a + 1 < m) load_step(a + 1);                 // the next frame's operands during the stores
    buf ^= 1;
    put_rows<D, RT>(s, buf, acc, col, lg);
  }

  const int64_t ph = (int64_t)j * H + h;
  if (is_p) {
    // pp[chunk][head][layout][plane][D][D]: layout 1 = P>^T (operand of the forward scan),
    // layout 0 = P<^T (reverse scan).  The transposed planes come straight from the accumulators
    // (a lane's four rows are consecutive elements of one transposed row); without decay
    // P<^T = P> is layout 0, copied row by row from the planes of the last step in LDS.
    bf16_t* p = pp + ph * 4 * DD;
    bf16_t* t = p + (part == 0 ? 2 * DD : 0);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      ushort4 hv, lv;
      uint16_t* hp = reinterpret_cast<uint16_t*>(&hv);
      uint16_t* lp = reinterpret_cast<uint16_t*>(&lv);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const __bf16 xh = (__bf16)acc[rt][i];
        hp[i] = __builtin_bit_cast(bf16_t, xh);
        lp[i] = __builtin_bit_cast(bf16_t, (__bf16)(acc[rt][i] - (float)xh));
      }
      const int64_t off = (int64_t)col * D + 16 * rt + 4 * lg;
      *reinterpret_cast<ushort4*>(t + off) = hv;
      *reinterpret_cast<ushort4*>(t + DD + off) = lv;
    }
    if (part == 0 && !alpha) {
      __syncthreads();                               // the last planes of s[buf] complete
      for (int e = tid; e < 2 * D * D / 8; e += D * 4) {
        const int plane = e / (D * D / 8), rem = e % (D * D / 8);
        const int row = rem / (D / 8), c8 = rem % (D / 8);
        const bf16_t* src = plane ? &s.lo[buf][row][c8 * 8] : &s.hi[buf][row][c8 * 8];
        *reinterpret_cast<uint4*>(p + plane * DD + (int64_t)row * D + c8 * 8) = *reinterpret_cast<const uint4*>(src);
      }
    }
  } else {
    float* q = qq + ((int64_t)(part - 1) * Nc * H + ph) * DD;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) q[(int64_t)(16 * rt + 4 * lg + i) * D + col] = acc[rt][i];
  }
}

// Chunk scan operand staging: the step matrix (two bf16 planes of its transpose, 2 D^2 bf16,
// contiguous) is copied into LDS by DMA in whole 256-byte rows (the fragment loads straight from
// global memory touched each 128-byte line with half a line per instruction, so twice the bytes
// crossed into the CU; at 768p the scan spent most of its time there), 16-byte chunk c of row n
// at chunk position c ^ scan_swz(n) so that the 16 rows a 16-lane fragment read covers land on
// distinct banks.
template <int D>
__device__ __forceinline__ int scan_swz(int n) {
  if constexpr (D == 128) return n & 15;
  else return (n >> 1) & 7;
}
template <int D>
struct ScanSmem {
  static constexpr int MAT = 2 * D * D * 2;            // bytes of one step matrix (hi, lo planes)
  static constexpr int STAGES = 2;
  static constexpr int ROWS_OFF = STAGES * MAT;
  static constexpr int TOTAL = ROWS_OFF + (int)sizeof(RowPlanes<D, 1>);
};

template <int D>
__global__ __launch_bounds__(D * 4) void vda_chunk_scan_kernel(const float* __restrict__ cw,
                                                               const bf16_t* __restrict__ pp,
                                                               const float* __restrict__ qq,
                                                               float* __restrict__ states, int Nc, int H,
                                                               int n_chains, int per_xcd) {
  using SM = ScanSmem<D>;
  constexpr int RB = D / 16;                         // row blocks per (head, direction)
  constexpr int NW = D / 16;                         // waves
  constexpr int CHR = D / 8;                         // 16-byte chunks per plane row
  constexpr int ROWS_PER_KB = 1024 / (2 * D);
  constexpr int DMA = SM::MAT / 1024 / NW;           // DMA instructions per wave and step
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  RowPlanes<D, 1>& s = *reinterpret_cast<RowPlanes<D, 1>*>(smem + SM::ROWS_OFF);
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
  auto chunk_of = [&](int k) { return dir == 0 ? k : Nc - 1 - k; };
  // forward applies P> (planes of P>^T give its columns), reverse applies P< (planes of P<^T)
  auto issue_mat = [&](int k) {
    const bf16_t* src = pp + ((int64_t)chunk_of(k) * H + h) * 4 * DD + (dir == 0 ? 2 * DD : 0);
    unsigned char* stg = smem + (k & 1) * SM::MAT;
#pragma unroll
    for (int i = 0; i < DMA; ++i) {
      const int blk = i * NW + wave;
      const int row = blk * ROWS_PER_KB + lane / CHR;          // row of the [2 D][D] plane pair
      const int c = (lane % CHR) ^ scan_swz<D>(row & (D - 1));
      __builtin_amdgcn_global_load_lds((gptr_t)(src + (int64_t)row * D + c * 8), (lptr_t)(stg + blk * 1024), 16,
                                       0, 0);
    }
  };
  auto load_c = [&](f32x4& c, int k) {
    const float* a = qq + ((int64_t)dir * Nc * H + (int64_t)chunk_of(k) * H + h) * DD + (int64_t)(row0 + 4 * lg) * D + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = a[i * D];
  };

  f32x4 acc;
  {
    const float* cp = cw + (int64_t)h * DD + (int64_t)(row0 + 4 * lg) * D + col;   // S0 = C_0
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = cp[i * D];
  }
  int buf = 0;
  {
    f32x4 a1[1] = {acc};
    put_rows<D, 1>(s, buf, a1, col, lg);
  }
  for (int c = 0; c < min(Nc, 2); ++c) store(dir == 0 ? c : Nc - 1 - c, acc);
  store(Nc, acc);
  if (n_steps == 0) return;
  // one step: wait for its matrix (DMA) and additive term, start the next step's copies into
  // the other stage and registers, then the product; the loop runs in pairs so the additive terms
  // alternate between two registers without a copy (a copy would make the compiler wait for the
  // next step's loads too)
  auto step = [&](int k, const f32x4& cur, f32x4& nxt) {
    // only the 4 state stores of step k-1 may be newer than step k's loads (none at k = 0: the
    // prologue's stores came first)
    if (k == 0) __builtin_amdgcn_s_waitcnt(0x0F70);         // vmcnt(0)
    else __builtin_amdgcn_s_waitcnt(0x0F74);                // vmcnt(4)
    lds_barrier();                                          // stage k & 1 and the rows of s[buf] complete
    if (k + 1 < n_steps) {                                  // stage (k+1) & 1 was last read in step k-1
      issue_mat(k + 1);
      load_c(nxt, k + 1);
    }
    asm volatile("" ::: "memory");                          // keep these loads ahead of this step's store
    const unsigned char* stg = smem + (k & 1) * SM::MAT;
    f32x4 a0 = cur, a1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const int ch = ks * 4 + lg;
      const int off = col * (2 * D) + ((ch ^ scan_swz<D>(col)) << 4);
      const bf16x8 mh = *reinterpret_cast<const bf16x8*>(stg + off);
      const bf16x8 ml = *reinterpret_cast<const bf16x8*>(stg + D * D * 2 + off);
      const bf16x8 xh = *reinterpret_cast<const bf16x8*>(&s.hi[buf][l16][ks * 32 + lg * 8]);
      const bf16x8 xl = *reinterpret_cast<const bf16x8*>(&s.lo[buf][l16][ks * 32 + lg * 8]);
      a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, mh, a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, ml, a1, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl, mh, a1, 0, 0, 0);
    }
    f32x4 r1[1] = {a0 + a1};
    buf ^= 1;
    put_rows<D, 1>(s, buf, r1, col, lg);
    store(dir == 0 ? k + 2 : Nc - 3 - k, r1[0]);
  };
  f32x4 ca, cb;
  issue_mat(0);
  load_c(ca, 0);
  for (int k = 0; k < n_steps; k += 2) {
    step(k, ca, cb);
    if (k + 1 < n_steps) step(k + 1, cb, ca);
  }
}

template <int D>
void launch_t(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  const int parts = in.alpha ? 4 : 3;
  vda_compose_kernel<D><<<dim3(parts, s.Nc, s.H), D * 4, 0, st>>>(b.minv, b.mhl, b.cw, in.alpha, b.pp, b.qq, s.T,
                                                                 s.C, s.Nc, s.H, s.anchors);
  // the row blocks of one (head, direction) stay on one XCD: per_xcd is a multiple of D / 16
  const int n_chains = 2 * s.H;
  const int per_xcd = (n_chains + 7) / 8 * (D / 16);
  const size_t smem = ScanSmem<D>::TOTAL;
  (void)hipFuncSetAttribute((const void*)vda_chunk_scan_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)smem);
  vda_chunk_scan_kernel<D><<<8 * per_xcd, D * 4, smem, st>>>(b.cw, b.pp, b.qq, b.states, s.Nc, s.H, n_chains,
                                                             per_xcd);
}

}  // namespace

hipError_t launch_vda_scan_mfma(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  if (s.d == 128) launch_t<128>(s, in, b, st);
  else launch_t<64>(s, in, b, st);
  return hipGetLastError();
}

}  // namespace vdn
