// MFMA state scans of Video Delta Attention (d in {64, 128}).
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Video Delta
// Attention: A Frame-Wise Solution": each frame updates the state as S <- (S + B_f) M_f with
// M_f = (I + A_f)^-1.  Section "Local Softmax and Long-Range Linear Memory": both directions start
// from the text state S0; the forward state of a query frame in chunk c has absorbed, in
// increasing order, the non-boundary frames of chunks <= c-2, the reverse state, in decreasing
// order, those of chunks >= c+2.
//
// Row r of the new state depends only on row r of the old state and of B_f, so the rows split into
// independent chains: one workgroup owns 32 rows of one (head, direction) and walks all frames;
// wave w produces output columns [32w, 32w + 32).  The product x M_f (x = s + B_f) runs on
// v_mfma_f32_32x32x16_bf16 with both operands split into bf16 high and low parts,
// x M ~ xh Mh + xh Ml + xl Mh (relative error ~2^-16, i.e. close to fp32), M_f read by rows thanks
// to its symmetry (M^T = M).  The state lives in LDS (fp32) between frames; B_f and M_f of the next
// frame are prefetched into registers while the current frame is multiplied.  Slot Nc of each
// direction receives S0 (read by boundary query frames).
#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kRows = 32;

template <int D>
__global__ __launch_bounds__(D * 2) void vda_scan_mfma_kernel(const float* __restrict__ minv,
                                                              const float* __restrict__ bw,
                                                              float* __restrict__ states, int T, int C, int Nc, int H,
                                                              int anchors) {
  constexpr int KS = D / 16;               // k-steps of 16
  constexpr int LDS_STRIDE = D + 4;
  __shared__ __attribute__((aligned(16))) float s_lds[kRows][LDS_STRIDE];
  const int row0 = blockIdx.x * kRows, dir = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hl = lane >> 5;
  const int col = wave * 32 + l32;          // output column of this lane (B-operand column)
  const int64_t DD = (int64_t)D * D;

  for (int e = tid; e < kRows * LDS_STRIDE; e += blockDim.x) (&s_lds[0][0])[e] = 0.f;

  // operand prefetch registers: B rows (A operand side) and M rows (B operand side, by symmetry)
  f32x4 breg[KS][2], mreg[KS][2];
  auto prefetch = [&](int slot) {
    const float* bsl = bw + ((int64_t)slot * H + h) * DD + (int64_t)(row0 + l32) * D + hl * 8;
    const float* msl = minv + ((int64_t)slot * H + h) * DD + (int64_t)col * D + hl * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      breg[ks][0] = *reinterpret_cast<const f32x4*>(bsl + ks * 16);
      breg[ks][1] = *reinterpret_cast<const f32x4*>(bsl + ks * 16 + 4);
      mreg[ks][0] = *reinterpret_cast<const f32x4*>(msl + ks * 16);
      mreg[ks][1] = *reinterpret_cast<const f32x4*>(msl + ks * 16 + 4);
    }
  };
  auto split = [](const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = e < 4 ? a[e] : b[e - 4];
      const __bf16 xh = (__bf16)x;
      hi[e] = xh;
      lo[e] = (__bf16)(x - (float)xh);
    }
  };
  // apply the frame whose operands sit in breg/mreg; the result replaces the state in LDS
  f32x16 acc;
  auto apply = [&]() {
    __syncthreads();                         // state of the previous step visible to every wave
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(&s_lds[l32][ks * 16 + hl * 8]);
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(&s_lds[l32][ks * 16 + hl * 8 + 4]);
      bf16x8 xh, xl, mh, ml;
      split(s0 + breg[ks][0], s1 + breg[ks][1], xh, xl);
      split(mreg[ks][0], mreg[ks][1], mh, ml);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, mh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, ml, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xl, mh, acc, 0, 0, 0);
    }
    __syncthreads();                         // every wave has read the old state
#pragma unroll
    for (int i = 0; i < 16; ++i) s_lds[8 * (i / 4) + 4 * hl + (i % 4)][col] = acc[i];
  };
  auto store = [&](int cslot) {
    float* dst = states + (((int64_t)dir * (Nc + 1) + cslot) * H + h) * DD + (int64_t)row0 * D + col;
#pragma unroll
    for (int i = 0; i < 16; ++i) dst[(int64_t)(8 * (i / 4) + 4 * hl + (i % 4)) * D] = acc[i];
  };
  auto boundary = [&](int f) { return anchors && (f == 0 || f == T - 1); };

  // ordered list of frame slots this direction applies, walked with a one-step prefetch
  auto next_frame = [&](int f, int step) {            // next scanned frame after f, or -1
    for (f += step; f >= 0 && f < T; f += step)
      if (!boundary(f)) return f;
    return -1;
  };

  prefetch(0);
  apply();                                   // text, written from the zero state
  store(Nc);                                 // S0
  if (dir == 0) {
    // forward: chunk c stores the state after every non-boundary frame of chunks <= c-2
    int f = next_frame(-1, 1);
    if (f >= 0) prefetch(1 + f);
    for (int c = 0; c < Nc; ++c) {
      if (c >= 2) {
        const int f_end = min((c - 1) * C, T);
        while (f >= 0 && f < f_end) {
          const int nf = next_frame(f, 1);
          apply();
          if (nf >= 0) prefetch(1 + nf);
          f = nf;
        }
      }
      store(c);
    }
  } else {
    int f = next_frame(T, -1);
    if (f >= 0) prefetch(1 + f);
    for (int c = Nc - 1; c >= 0; --c) {
      if (c + 2 <= Nc - 1) {
        const int f_lo = (c + 2) * C;
        while (f >= 0 && f >= f_lo) {
          const int nf = next_frame(f, -1);
          apply();
          if (nf >= 0) prefetch(1 + nf);
          f = nf;
        }
      }
      store(c);
    }
  }
}

template <int D>
void launch_t(const Shape& s, const Buffers& b, hipStream_t st) {
  dim3 grid(D / kRows, 2, s.H);
  vda_scan_mfma_kernel<D><<<grid, D * 2, 0, st>>>(b.minv, b.bw, b.states, s.T, s.C, s.Nc, s.H, s.anchors);
}

}  // namespace

hipError_t launch_vda_scan_mfma(const Shape& s, const Buffers& b, hipStream_t st) {
  if (s.d == 128) launch_t<128>(s, b, st);
  else launch_t<64>(s, b, st);
  return hipGetLastError();
}

}  // namespace vdn
