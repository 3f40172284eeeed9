// Generic (SIMT) kernel of the softmax branch: any d in {16,32,64,128}, fp32 or bf16 inputs.
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Local Softmax and
// Long-Range Linear Memory": each video query attends, under one softmax with scale 1/sqrt(d), to
// the text keys, the keys of its chunk and of the two neighbouring chunks, and the boundary anchor
// frames.  "Video DeltaNet speeds MiniMax H3 video generation 14.5x" (summary): interactions with
// text or audio stay full softmax attention, so audio keys join the text keys, and the text and
// audio query rows attend to every token.  The key set of a row group is a short list of
// contiguous ranges (built on the host) in the key space [text, audio (padded) | video tokens].
//
// One thread per query token: the 64 threads of a block are 64 consecutive tokens of one frame
// and one head, so they walk the same keys in lock step and every key/value load is a broadcast.
// Online softmax in base 2 with fp32 statistics and accumulator.
#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

// Row group g = blockIdx.y holds nq query rows (q and o are [groups][nq][H][D]) and uses key-range
// row t0 + g: video frames (t0 = 0, nq = N) or the context rows (t0 = T, nq = n_ctx, one group).
template <typename Tin, int D>
__global__ __launch_bounds__(64) void softmax_simt_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const Tin* __restrict__ ctx_kv, Tin* __restrict__ o, const int* __restrict__ ranges,
    const int* __restrict__ nranges, int nq, int t0, int H, int n_ctx, int ctx_pad, float scale_log2,
    float* __restrict__ lse) {
  const int t = t0 + blockIdx.y, h = blockIdx.z;
  const int n = blockIdx.x * 64 + threadIdx.x;
  if (n >= nq) return;
  const int64_t tok = (int64_t)blockIdx.y * nq + n;
  const Tin* qp = q + (tok * H + h) * D;
  float qr[D], acc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) { qr[i] = to_f32(qp[i]) * scale_log2; acc[i] = 0.f; }
  float m = -INFINITY, l = 0.f;
  const Tin* ctx_v = ctx_kv + (int64_t)n_ctx * H * D;
  const int nr = nranges[t];
  for (int r = 0; r < nr; ++r) {
    const int a = ranges[t * 2 * kMaxRanges + 2 * r], b = ranges[t * 2 * kMaxRanges + 2 * r + 1];
    for (int j = a; j < b; ++j) {
      const Tin *kp, *vp;
      if (j < ctx_pad) {
        kp = ctx_kv + ((int64_t)j * H + h) * D;
        vp = ctx_v + ((int64_t)j * H + h) * D;
      } else {
        const int64_t vt = j - ctx_pad;
        kp = k + (vt * H + h) * D;
        vp = v + (vt * H + h) * D;
      }
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) s += qr[i] * to_f32(kp[i]);
      if (s > m) {
        const float alpha = exp2f(m - s);
        l *= alpha;
#pragma unroll
        for (int i = 0; i < D; ++i) acc[i] *= alpha;
        m = s;
      }
      const float p = exp2f(s - m);
      l += p;
#pragma unroll
      for (int i = 0; i < D; ++i) acc[i] += p * to_f32(vp[i]);
    }
  }
  const float inv = 1.f / l;
  if (lse) lse[tok * H + h] = m + __log2f(l);         // scores are in base-2 units here
  Tin* op = o + (tok * H + h) * D;
#pragma unroll
  for (int i = 0; i < D; ++i) store_elt(op + i, acc[i] * inv);
}

template <typename Tin, int D>
void launch_t(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  softmax_simt_kernel<Tin, D><<<dim3((s.N + 63) / 64, s.T, s.H), 64, 0, st>>>(
      (const Tin*)in.q, (const Tin*)in.k, (const Tin*)in.v, (const Tin*)in.text_kv, (Tin*)b.os, b.ranges,
      b.nranges, s.N, 0, s.H, s.n_ctx, s.ctx_pad, scale_log2, b.lse);
  if (in.ctx_out)
    softmax_simt_kernel<Tin, D><<<dim3((s.n_ctx + 63) / 64, 1, s.H), 64, 0, st>>>(
        (const Tin*)in.ctx_q, (const Tin*)in.k, (const Tin*)in.v, (const Tin*)in.text_kv, (Tin*)in.ctx_out,
        b.ranges, b.nranges, s.n_ctx, s.T, s.H, s.n_ctx, s.ctx_pad, scale_log2,
        b.lse ? b.lse + (int64_t)s.T * s.N * s.H : nullptr);   // context rows after the video rows
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

hipError_t launch_softmax_simt(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  if (s.dtype == VDN_BF16) launch_d<bf16_t>(s, in, b, st);
  else launch_d<float>(s, in, b, st);
  return hipGetLastError();
}

}  // namespace vdn
