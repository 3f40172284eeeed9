// Generic (SIMT) epilogue of the VDN layer: linear readout, RMSNorm, the two sigmoid gates, the
// two output projections and their sum.
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Local Softmax and
// Long-Range Linear Memory": the query reads both directional states and adds the two readouts,
// o_l = (S_fwd + S_rev) q.  Section "Gating the Softmax and Linear Branch Outputs": each branch is
// gated by a content-dependent sigmoid gate and has its own output projection; the linear branch
// is RMS-normalised first; the two projected branches are summed.  Gate input is q (per head),
// weights are [in][out] and shared by the heads, RMSNorm eps = 1e-6 with unit weight.
//
// One block per (16 tokens of one frame, head); thread j computes output channel j.  The frame's
// combined state S = S_fwd[c] + S_rev[c] (slot Nc = S0 for boundary frames) is staged in LDS.
#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

constexpr int kTok = 16;

template <typename Tin, int D>
__global__ __launch_bounds__(D < 64 ? 64 : D) void epilogue_simt_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ o_s, const float* __restrict__ states,
    const Tin* __restrict__ gate_w, const Tin* __restrict__ proj_w, Tin* __restrict__ out, int T, int N, int H,
    int C, int Nc, int anchors) {
  const int t = blockIdx.y, h = blockIdx.z;
  const int n0 = blockIdx.x * kTok;
  const int j = threadIdx.x;
  const bool active = j < D;
  const int jj = active ? j : 0;
  __shared__ float S[D][D + 1];
  __shared__ float qs[kTok][D], os[kTok][D], ol[kTok][D], xa[kTok][D], xb[kTok][D];
  __shared__ float rinv[kTok];

  const bool bnd = anchors && (t == 0 || t == T - 1);
  const int slot = bnd ? Nc : t / C;
  const int64_t DD = (int64_t)D * D;
  const float* sf = states + ((int64_t)slot * H + h) * DD;
  const float* sr = states + (((int64_t)(Nc + 1) + slot) * H + h) * DD;
  for (int e = threadIdx.x; e < D * D; e += blockDim.x) S[e / D][e % D] = sf[e] + sr[e];
  for (int e = threadIdx.x; e < kTok * D; e += blockDim.x) {
    const int tt = e / D, i = e % D;
    const int n = n0 + tt;
    float qv = 0.f, ov = 0.f;
    if (n < N) {
      const int64_t off = (((int64_t)t * N + n) * H + h) * D + i;
      qv = to_f32(q[off]);
      ov = to_f32(o_s[off]);
    }
    qs[tt][i] = qv;
    os[tt][i] = ov;
  }
  __syncthreads();

  float acc_l[kTok], acc_gs[kTok], acc_gl[kTok];
#pragma unroll
  for (int tt = 0; tt < kTok; ++tt) { acc_l[tt] = 0.f; acc_gs[tt] = 0.f; acc_gl[tt] = 0.f; }
  for (int i = 0; i < D; ++i) {
    const float sji = S[jj][i];
    const float g0 = to_f32(gate_w[(int64_t)i * D + jj]);
    const float g1 = to_f32(gate_w[DD + (int64_t)i * D + jj]);
#pragma unroll
    for (int tt = 0; tt < kTok; ++tt) {
      const float qi = qs[tt][i];
      acc_l[tt] += sji * qi;
      acc_gs[tt] += qi * g0;
      acc_gl[tt] += qi * g1;
    }
  }
  if (active) {
#pragma unroll
    for (int tt = 0; tt < kTok; ++tt) ol[tt][j] = acc_l[tt];
  }
  __syncthreads();
  if (threadIdx.x < kTok) {
    float ss = 0.f;
    for (int i = 0; i < D; ++i) ss += ol[threadIdx.x][i] * ol[threadIdx.x][i];
    rinv[threadIdx.x] = 1.0f / sqrtf(ss / D + 1e-6f);
  }
  __syncthreads();
  if (active) {
#pragma unroll
    for (int tt = 0; tt < kTok; ++tt) {
      xa[tt][j] = sigmoidf_(acc_gs[tt]) * os[tt][j];
      xb[tt][j] = sigmoidf_(acc_gl[tt]) * ol[tt][j] * rinv[tt];
    }
  }
  __syncthreads();
  float acc[kTok];
#pragma unroll
  for (int tt = 0; tt < kTok; ++tt) acc[tt] = 0.f;
  for (int i = 0; i < D; ++i) {
    const float p0 = to_f32(proj_w[(int64_t)i * D + jj]);
    const float p1 = to_f32(proj_w[DD + (int64_t)i * D + jj]);
#pragma unroll
    for (int tt = 0; tt < kTok; ++tt) acc[tt] += xa[tt][i] * p0 + xb[tt][i] * p1;
  }
  if (active) {
#pragma unroll
    for (int tt = 0; tt < kTok; ++tt) {
      const int n = n0 + tt;
      if (n < N) store_elt(out + (((int64_t)t * N + n) * H + h) * D + j, acc[tt]);
    }
  }
}

template <typename Tin, int D>
void launch_t(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  dim3 grid((s.N + kTok - 1) / kTok, s.T, s.H);
  const int threads = D < 64 ? 64 : D;
  epilogue_simt_kernel<Tin, D><<<grid, threads, 0, st>>>(
      (const Tin*)in.q, (const Tin*)b.os, b.states, (const Tin*)in.gate_w, (const Tin*)in.proj_w, (Tin*)in.out,
      s.T, s.N, s.H, s.C, s.Nc, s.anchors);
}

template <typename Tin>
void launch_d(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  switch (s.d) {
    case 16: launch_t<Tin, 16>(s, in, b, st); break;
    case 32: launch_t<Tin, 32>(s, in, b, st); break;
    case 64: launch_t<Tin, 64>(s, in, b, st); break;
    default: launch_t<Tin, 128>(s, in, b, st); break;
  }
}

}  // namespace

hipError_t launch_epilogue(const Shape& s, const Inputs& in, const Buffers& b, bool /*mfma*/, hipStream_t st) {
  if (s.dtype == VDN_BF16) launch_d<bf16_t>(s, in, b, st);
  else launch_d<float>(s, in, b, st);
  return hipGetLastError();
}

}  // namespace vdn
