// MFMA epilogue of the VDN layer (bf16 plans, d in {64, 128}): linear readout, RMSNorm, the two
// sigmoid gates, the two output projections and their sum.
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Local Softmax and
// Long-Range Linear Memory": o_l = (S_fwd + S_rev) q.  Section "Gating the Softmax and Linear Branch
// Outputs": out = (sigmoid(q Wg0) * o_s) Wp0 + (sigmoid(q Wg1) * RMSNorm(o_l)) Wp1 (gate input q,
// weights [in][out] shared by the heads, RMSNorm eps 1e-6 with unit weight).
//
// All products are computed transposed (channels x tokens) with v_mfma_f32_16x16x32_bf16, so the
// small operand that is the same for every token of the workgroup -- the combined state S of the
// frame's chunk and the four weight matrices -- is the A operand and stays in registers:
//   * one workgroup = up to 512 tokens of one frame and one head, D/16 waves; wave w owns output
//     channels [16w, 16w + 16) and holds rows [16w, 16w+16) of S (as bf16 hi + lo parts, so the
//     readout keeps ~16 mantissa bits) and of Wg0^T, Wg1^T, Wp0^T, Wp1^T (pre-transposed once per
//     forward by prep_weights_kernel);
//   * tokens stream through LDS in tiles of 64 whose global operands (q, the o_s slice) are fetched
//     two tiles ahead: q^T is the shared B operand of the readout and of both gates; the per-token
//     RMS needs all channels, so each wave's partial sum of squares is exchanged through LDS; the
//     gated branches x_s, x_l are exchanged through LDS, as bf16 hi + lo parts, as the B operand
//     of the two projections.
#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kTileTok = 64;
#ifndef VDN_EPI_TOK
#define VDN_EPI_TOK 512
#endif
constexpr int kTokPerWG = VDN_EPI_TOK;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// W^T for gate_w[0], gate_w[1], proj_w[0], proj_w[1]: wt[m][j][i] = W_m[i][j]
__global__ __launch_bounds__(256) void prep_weights_kernel(const bf16_t* __restrict__ gate_w,
                                                           const bf16_t* __restrict__ proj_w,
                                                           bf16_t* __restrict__ wt, int D) {
  const int m = blockIdx.y;
  const bf16_t* src = m < 2 ? gate_w + (int64_t)m * D * D : proj_w + (int64_t)(m - 2) * D * D;
  for (int e = blockIdx.x * 256 + threadIdx.x; e < D * D; e += gridDim.x * 256) {
    const int j = e / D, i = e % D;
    wt[(int64_t)m * D * D + e] = src[(int64_t)i * D + j];
  }
}

template <int D>
__global__ __launch_bounds__(D * 4) void epilogue_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ o_s, const float* __restrict__ states,
    const bf16_t* __restrict__ wt, bf16_t* __restrict__ out, int T, int N, int H, int C, int Nc, int anchors,
    int wg_per_frame) {
  constexpr int NW = D / 16;              // waves
  constexpr int KS = D / 32;              // k-steps of 32
  constexpr int NT = kTileTok / 16;       // 16-token column tiles per tile
  constexpr int NTHR = NW * 64;
  constexpr int QCH = kTileTok * D / 8;   // 16-byte chunks of a q tile
  constexpr int QPT = (QCH + NTHR - 1) / NTHR;
  __shared__ __attribute__((aligned(16))) bf16_t qtile[kTileTok][D + 8];
  __shared__ __attribute__((aligned(16))) bf16_t xtile[4][kTileTok][D + 8];   // x_s hi, x_s lo, x_l hi, x_l lo
  __shared__ float part[NW][kTileTok];

  const int wg = blockIdx.x;
  const int h = blockIdx.y;
  const int t = wg / wg_per_frame;
  const int tok_begin = (wg % wg_per_frame) * kTokPerWG;
  const int tok_end = min(N, tok_begin + kTokPerWG);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lg = lane >> 4;         // lane group 0..3
  const int j0 = wave * 16;

  const bool bnd = anchors && (t == 0 || t == T - 1);
  const int slot = bnd ? Nc : t / C;
  const int64_t DD = (int64_t)D * D;
  const float* sf = states + ((int64_t)slot * H + h) * DD;
  const float* sr = states + (((int64_t)(Nc + 1) + slot) * H + h) * DD;

  // ---- A fragments: row j0 + l16, k = ks*32 + lg*8 .. +8 ----
  bf16x8 s_hi[KS], s_lo[KS], wg0[KS], wg1[KS], wp0[KS], wp1[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int j = j0 + l16, i0 = ks * 32 + lg * 8;
    const f32x4* a = reinterpret_cast<const f32x4*>(sf + (int64_t)j * D + i0);
    const f32x4* b = reinterpret_cast<const f32x4*>(sr + (int64_t)j * D + i0);
    const f32x4 a0 = a[0], a1 = a[1], b0 = b[0], b1 = b[1];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sv = e < 4 ? a0[e] + b0[e] : a1[e - 4] + b1[e - 4];
      const __bf16 hi = (__bf16)sv;
      s_hi[ks][e] = hi;
      s_lo[ks][e] = (__bf16)(sv - (float)hi);
    }
    wg0[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(wt + 0 * DD + (int64_t)j * D + i0));
    wg1[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(wt + 1 * DD + (int64_t)j * D + i0));
    wp0[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(wt + 2 * DD + (int64_t)j * D + i0));
    wp1[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(wt + 3 * DD + (int64_t)j * D + i0));
  }

  // Global operands of a tile (q tile chunks, this lane's o_s slice), fetched two tiles ahead.
  struct Pre {
    u32x4 q[QPT];
    uint2 os[NT];
  };
  auto fetch = [&](int tok0, Pre& pr) {
#pragma unroll
    for (int c = 0; c < QPT; ++c) {
      const int e = c * NTHR + tid;
      u32x4 val = {0, 0, 0, 0};
      if (e < QCH) {
        const int r = e / (D / 8), cc = e % (D / 8);
        const int n = tok0 + r;
        if (n < tok_end) val = *reinterpret_cast<const u32x4*>(q + (((int64_t)t * N + n) * H + h) * D + cc * 8);
      }
      pr.q[c] = val;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = tok0 + nt * 16 + l16;
      pr.os[nt] = n < tok_end ? *reinterpret_cast<const uint2*>(o_s + (((int64_t)t * N + n) * H + h) * D + j0 + lg * 4)
                              : make_uint2(0, 0);
    }
  };

  auto process = [&](int tok0, const Pre& pr) {
#pragma unroll
    for (int c = 0; c < QPT; ++c) {
      const int e = c * NTHR + tid;
      if (e < QCH) {
        const int r = e / (D / 8), cc = e % (D / 8);
        *reinterpret_cast<u32x4*>(&qtile[r][cc * 8]) = pr.q[c];
      }
    }
    __syncthreads();                                         // q tile ready (previous tile's readers
                                                             // passed the previous 2nd and 3rd barrier)
    f32x4 ol[NT], gs[NT], gl[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      ol[nt] = f32x4{0, 0, 0, 0};
      gs[nt] = f32x4{0, 0, 0, 0};
      gl[nt] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 qb = as_bf16x8(*reinterpret_cast<const u32x4*>(&qtile[nt * 16 + l16][ks * 32 + lg * 8]));
        ol[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s_hi[ks], qb, ol[nt], 0, 0, 0);
        ol[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s_lo[ks], qb, ol[nt], 0, 0, 0);
        gs[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wg0[ks], qb, gs[nt], 0, 0, 0);
        gl[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wg1[ks], qb, gl[nt], 0, 0, 0);
      }
    }
    // partial sums of squares of o_l over this wave's 16 channels, per token
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float ss = ol[nt][0] * ol[nt][0] + ol[nt][1] * ol[nt][1] + ol[nt][2] * ol[nt][2] + ol[nt][3] * ol[nt][3];
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      if (lg == 0) part[wave][nt * 16 + l16] = ss;
    }
    __syncthreads();                                         // partial sums ready
    // gated branches, as bf16 hi + lo parts (the projection weights are exact bf16, so the two
    // projections keep ~fp32 accuracy)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float ss = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) ss += part[ww][nt * 16 + l16];
      const float rinv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + 1e-6f);
      __bf16 xsh[4], xsl[4], xlh[4], xll[4];
      const uint32_t o01 = pr.os[nt].x, o23 = pr.os[nt].y;
      const float osv[4] = {__uint_as_float(o01 << 16), __uint_as_float(o01 & 0xFFFF0000u),
                            __uint_as_float(o23 << 16), __uint_as_float(o23 & 0xFFFF0000u)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float xs = fast_sigmoid(gs[nt][e]) * osv[e];
        const float xl = fast_sigmoid(gl[nt][e]) * ol[nt][e] * rinv;
        xsh[e] = (__bf16)xs;
        xsl[e] = (__bf16)(xs - (float)xsh[e]);
        xlh[e] = (__bf16)xl;
        xll[e] = (__bf16)(xl - (float)xlh[e]);
      }
      const int row = nt * 16 + l16, c0 = j0 + lg * 4;
      *reinterpret_cast<uint2*>(&xtile[0][row][c0]) = __builtin_bit_cast(uint2, xsh);
      *reinterpret_cast<uint2*>(&xtile[1][row][c0]) = __builtin_bit_cast(uint2, xsl);
      *reinterpret_cast<uint2*>(&xtile[2][row][c0]) = __builtin_bit_cast(uint2, xlh);
      *reinterpret_cast<uint2*>(&xtile[3][row][c0]) = __builtin_bit_cast(uint2, xll);
    }
    __syncthreads();                                         // gated branches ready
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 o = {0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int row = nt * 16 + l16, k0 = ks * 32 + lg * 8;
        o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            wp0[ks], as_bf16x8(*reinterpret_cast<const u32x4*>(&xtile[0][row][k0])), o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            wp0[ks], as_bf16x8(*reinterpret_cast<const u32x4*>(&xtile[1][row][k0])), o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            wp1[ks], as_bf16x8(*reinterpret_cast<const u32x4*>(&xtile[2][row][k0])), o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            wp1[ks], as_bf16x8(*reinterpret_cast<const u32x4*>(&xtile[3][row][k0])), o, 0, 0, 0);
      }
      const int n = tok0 + nt * 16 + l16;
      if (n < tok_end) {
        __bf16 ov[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (__bf16)o[e];
        *reinterpret_cast<uint2*>(out + (((int64_t)t * N + n) * H + h) * D + j0 + lg * 4) = __builtin_bit_cast(uint2, ov);
      }
    }
  };

  // two register sets, fetched two tiles ahead of their use
  Pre pa, pb;
  fetch(tok_begin, pa);
  fetch(tok_begin + kTileTok, pb);
  for (int tok0 = tok_begin; tok0 < tok_end; tok0 += 2 * kTileTok) {
    process(tok0, pa);
    if (tok0 + 2 * kTileTok < tok_end) fetch(tok0 + 2 * kTileTok, pa);
    if (tok0 + kTileTok < tok_end) {
      process(tok0 + kTileTok, pb);
      if (tok0 + 3 * kTileTok < tok_end) fetch(tok0 + 3 * kTileTok, pb);
    }
  }
}

template <int D>
void launch_t(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  const int wg_per_frame = (s.N + kTokPerWG - 1) / kTokPerWG;
  dim3 grid(s.T * wg_per_frame, s.H);
  epilogue_mfma_kernel<D><<<grid, D * 4, 0, st>>>((const bf16_t*)in.q, (const bf16_t*)b.os, b.states, b.wt,
                                                  (bf16_t*)in.out, s.T, s.N, s.H, s.C, s.Nc, s.anchors,
                                                  wg_per_frame);
}

}  // namespace

hipError_t launch_prep_weights(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  dim3 grid((s.d * s.d + 255) / 256, 4);
  prep_weights_kernel<<<grid, 256, 0, st>>>((const bf16_t*)in.gate_w, (const bf16_t*)in.proj_w, b.wt, s.d);
  return hipGetLastError();
}

hipError_t launch_epilogue_mfma(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  if (s.d == 128) launch_t<128>(s, in, b, st);
  else launch_t<64>(s, in, b, st);
  return hipGetLastError();
}

}  // namespace vdn
