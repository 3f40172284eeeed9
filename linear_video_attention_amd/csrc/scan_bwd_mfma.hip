// Adjoint chain of the frame scan, and the states entering each scanned frame, on CDNA4 matrix
// cores (bf16 plans, d in {64, 128}).
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Video Delta
// Attention: A Frame-Wise Solution": each scanned frame maps the state as
// S <- (S Diag(alpha_f) + B_f) M_f.  Walking the frames of one direction in reverse scan order, the
// adjoint G of the state after frame f (plus the readout adjoints of the chunks that read that
// state) gives dB_f = dR = G M_f^T and the adjoint before the frame, dR Diag(alpha_f); the adjoint
// after every write is kept for the per-frame dM_f and dalpha_f.  After the first frame, the
// adjoint is that of the text state.
//
// The chain is sequential in the frames but its rows are independent (every step multiplies G from
// the right), so the workgroups of one (head, direction) each run it for a block of rows: 16 rows at
// d = 128, 32 at d = 64, eight waves each owning one 16 x 16 output tile.  A step is a rows x d x d
// product on v_mfma_f32_16x16x32_bf16 with both fp32 operands as bf16 hi + lo parts (three
// products, about 2^-16 relative per step).  The block of G stays in LDS in fp32; a wave's B
// fragments (rows of M_f, eight consecutive k per lane) come straight from global memory and the
// next frame's are loaded while the current product runs.
#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kWaves = 8;

__device__ __forceinline__ void split8(float4 a, float4 b, bf16x8& hi, bf16x8& lo) {
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 t = (__bf16)x[i];
    hi[i] = t;
    lo[i] = (__bf16)(x[i] - (float)t);
  }
}

template <int D>
__global__ __launch_bounds__(kWaves * 64) void scan_bwd_mfma_kernel(
    const float* __restrict__ minv, const float* __restrict__ alpha, const float* __restrict__ dread,
    const int* __restrict__ mslot, const int* __restrict__ order, int nscan, int T, int H, int Nc,
    float* __restrict__ dmf, float* __restrict__ dbf, float* __restrict__ ds0) {
  constexpr int KS = D / 32, TJ = D / 16;
  constexpr int RB = 16 * (kWaves / TJ);       // rows of G per workgroup: one row tile per wave
  constexpr int LD = D + 4;                    // LDS row stride (floats)
  constexpr int64_t DD = (int64_t)D * D;
  extern __shared__ __attribute__((aligned(16))) float adj[];   // RB x LD
  const int h = blockIdx.x, dir = blockIdx.y, row0 = blockIdx.z * RB;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int tj = wave % TJ, ti = wave / TJ;
  const int* ms = mslot + dir * (Nc + 2);
  for (int e = tid; e < RB * D; e += kWaves * 64) adj[(e / D) * LD + e % D] = 0.f;
  __syncthreads();
  auto add_reads = [&](int m) {
    for (int c = 0; c < Nc + 2; ++c)
      if (ms[c] == m) {
        const float* gr = dread + ((int64_t)c * H + h) * DD + (int64_t)row0 * D;
        for (int e = tid; e < RB * D; e += kWaves * 64) adj[(e / D) * LD + e % D] += gr[e];
      }
    __syncthreads();
  };
  auto frame_of = [&](int m) { return order[dir == 0 ? m - 1 : nscan - m]; };
  // B fragment of k-step ks: row 16 tj + l16 of M_f, columns 32 ks + 8 g .. + 7
  float4 mb[KS][2];
  auto load_m = [&](int f) {
    const float* mf = minv + ((int64_t)(1 + f) * H + h) * DD + (int64_t)(16 * tj + l16) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      mb[ks][0] = *reinterpret_cast<const float4*>(mf + 32 * ks);
      mb[ks][1] = *reinterpret_cast<const float4*>(mf + 32 * ks + 4);
    }
  };
  const int col = 16 * tj + l16;
  if (nscan >= 1) load_m(frame_of(nscan));
  for (int m = nscan; m >= 1; --m) {
    add_reads(m);
    const int f = frame_of(m);
    bf16x8 bh[KS], bl[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) split8(mb[ks][0], mb[ks][1], bh[ks], bl[ks]);
    if (m > 1) load_m(frame_of(m - 1));      // the next frame's fragments, in flight during this step
    // dR = G M_f^T: dR[i][j] = sum_k G[i][k] M_f[j][k]
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float* ar = adj + (16 * ti + l16) * LD + 32 * ks + 8 * g;
      bf16x8 ah, al;
      split8(*reinterpret_cast<const float4*>(ar), *reinterpret_cast<const float4*>(ar + 4), ah, al);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh[ks], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl[ks], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh[ks], acc, 0, 0, 0);
    }
    // keep the adjoint after the write (for dM_f, dalpha_f) and dB_f = dR
    float* dmo = dmf + (((int64_t)dir * T + f) * H + h) * DD + (int64_t)row0 * D;
    float* dbo = dbf + (((int64_t)dir * T + f) * H + h) * DD + (int64_t)row0 * D;
    for (int e = tid; e < RB * D; e += kWaves * 64) dmo[e] = adj[(e / D) * LD + e % D];
#pragma unroll
    for (int i = 0; i < 4; ++i) dbo[(int64_t)(16 * ti + 4 * g + i) * D + col] = acc[i];
    __syncthreads();                             // every wave is done reading G
    const float a = alpha ? alpha[((int64_t)f * H + h) * D + col] : 1.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) adj[(16 * ti + 4 * g + i) * LD + col] = acc[i] * a;
    __syncthreads();
  }
  add_reads(0);
  float* o = ds0 + ((int64_t)dir * H + h) * DD + (int64_t)row0 * D;
  for (int e = tid; e < RB * D; e += kWaves * 64) o[e] = adj[(e / D) * LD + e % D];
}

// States entering the scanned frames, walked per (chunk, head, direction) from the forward's chunk
// state like the generic frame_states_kernel: Z <- (Z Diag(alpha_f) + B_f) M_f frame by frame (M_f
// symmetric, so row j of M_f is column j), storing Z before every frame of the chunk.  Rows evolve
// independently, so each workgroup walks a block of rows with the chain's layout; the block of Z
// lives in LDS in fp32.
template <int D>
__global__ __launch_bounds__(kWaves * 64) void frame_states_mfma_kernel(
    const float* __restrict__ states, const float* __restrict__ minv, const float* __restrict__ bw,
    const float* __restrict__ alpha, int T, int C, int anchors, int H, int Nc, float* __restrict__ zin) {
  constexpr int KS = D / 32, TJ = D / 16;
  constexpr int RB = 16 * (kWaves / TJ);
  constexpr int LD = D + 4;
  constexpr int64_t DD = (int64_t)D * D;
  extern __shared__ __attribute__((aligned(16))) float z[];   // RB x LD
  const int c = blockIdx.x, h = blockIdx.y, dir = blockIdx.z / (D / RB), row0 = (blockIdx.z % (D / RB)) * RB;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int tj = wave % TJ, ti = wave / TJ;
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
  const float* s0 = states + ((int64_t)(dir * (Nc + 1) + slot) * H + h) * DD + (int64_t)row0 * D;
  for (int e = tid; e < RB * D; e += kWaves * 64) z[(e / D) * LD + e % D] = s0[e];
  __syncthreads();
  const int step = dir == 0 ? 1 : -1;
  const int col = 16 * tj + l16;
  for (int f = f_first;; f += step) {
    if (!(anchors && (f == 0 || f == T - 1))) {
      if (f / C == c) {
        float* zo = zin + (((int64_t)dir * T + f) * H + h) * DD + (int64_t)row0 * D;
        for (int e = tid; e < RB * D; e += kWaves * 64) zo[e] = z[(e / D) * LD + e % D];
      }
      const float* af = alpha ? alpha + ((int64_t)f * H + h) * D : nullptr;
      const float* bf = bw + ((int64_t)(1 + f) * H + h) * DD + (int64_t)row0 * D;
      const float* mf = minv + ((int64_t)(1 + f) * H + h) * DD + (int64_t)col * D + 8 * g;
      bf16x8 bh[KS], bl[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        split8(*reinterpret_cast<const float4*>(mf + 32 * ks), *reinterpret_cast<const float4*>(mf + 32 * ks + 4),
               bh[ks], bl[ks]);
      __syncthreads();                           // the copy-out of Z is done
      for (int e = tid; e < RB * D; e += kWaves * 64) {
        const int r = e / D, cc = e % D;
        z[r * LD + cc] = z[r * LD + cc] * (af ? af[cc] : 1.f) + bf[e];
      }
      __syncthreads();
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const float* ar = z + (16 * ti + l16) * LD + 32 * ks + 8 * g;
        bf16x8 ah, al;
        split8(*reinterpret_cast<const float4*>(ar), *reinterpret_cast<const float4*>(ar + 4), ah, al);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh[ks], acc, 0, 0, 0);
      }
      __syncthreads();                           // every wave is done reading the right-hand side
#pragma unroll
      for (int i = 0; i < 4; ++i) z[(16 * ti + 4 * g + i) * LD + col] = acc[i];
      __syncthreads();
    }
    if (f == f_last) break;
  }
}

}  // namespace

template <int D>
static hipError_t launch_t(const Shape& s, const Inputs& in, const Buffers& b, const BwdBuffers& w, hipStream_t st) {
  constexpr int RB = 16 * (kWaves / (D / 16));   // rows of the adjoint per workgroup
  constexpr size_t sm = (size_t)RB * (D + 4) * 4;
  scan_bwd_mfma_kernel<D><<<dim3(s.H, 2, D / RB), kWaves * 64, sm, st>>>(
      b.minv, in.alpha, w.dread, w.mslot, w.order, w.nscan, s.T, s.H, s.Nc, w.dmf, w.dbf, w.ds0);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_fs(const Shape& s, const Inputs& in, const Buffers& b, const BwdBuffers& w, hipStream_t st) {
  constexpr int RB = 16 * (kWaves / (D / 16));
  constexpr size_t sm = (size_t)RB * (D + 4) * 4;
  frame_states_mfma_kernel<D><<<dim3(s.Nc, s.H, 2 * (D / RB)), kWaves * 64, sm, st>>>(
      b.states, b.minv, b.bw, in.alpha, s.T, s.C, s.anchors, s.H, s.Nc, w.zin);
  return hipGetLastError();
}

hipError_t launch_frame_states_mfma(const Shape& s, const Inputs& in, const Buffers& b, const BwdBuffers& w,
                                   hipStream_t st) {
  if (s.d == 128) return launch_fs<128>(s, in, b, w, st);
  if (s.d == 64) return launch_fs<64>(s, in, b, w, st);
  return hipErrorInvalidValue;
}

hipError_t launch_scan_bwd_mfma(const Shape& s, const Inputs& in, const Buffers& b, const BwdBuffers& w,
                                hipStream_t st) {
  if (s.d == 128) return launch_t<128>(s, in, b, w, st);
  if (s.d == 64) return launch_t<64>(s, in, b, w, st);
  return hipErrorInvalidValue;
}

}  // namespace vdn
