// Packing of keys and values for the FP8 (E4M3) softmax kernel, d = 128.
//
// FP8 variant of the softmax branch of "Video DeltaNet: Near-Lossless Hybrid Attention for Video
// Models" (section "Local Softmax and Long-Range Linear Memory"; the pages run their production
// kernels with FP8, section "Adapting the Pretrained H3 backbone").  Every operand is rounded to
// OCP E4M3 after a power-of-two scale 2^(8 - e), e the binary exponent of the largest magnitude
// (m = f 2^e, f in [0.5, 1)), so the scaled values stay below 256:
//   K8 [H][Ls8][128]  e4m3(s_k k), row per key          s_k from max |k| over the head's keys
//   V8 [H][128][Ls8]  e4m3(s_v v), transposed            s_v from max |v| over the head's values
// in the same key space as the bf16 path (global keys padded to 64, then the video tokens; keys
// Lk .. Ls8 stay zero, so a 128-key tile never leaves the buffer).  Three launches: per 64-key
// block the largest |k|, |v| and key norm; per head the scales and the largest key norm (the
// softmax's exponent bound); the packing itself.
#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

constexpr int D = 128;

__device__ __forceinline__ float pow2_scale(float m) {
  if (!(m > 0.f)) return 1.f;
  int e;
  (void)frexpf(m, &e);
  return ldexpf(1.f, 8 - e);
}

// key j of the head's key space: pointers to its d keys and values, or null for a padding key
__device__ __forceinline__ void key_src(const bf16_t* k, const bf16_t* v, const bf16_t* ctx_kv, int64_t j, int h,
                                        int H, int n_ctx, int ctx_pad, int64_t Lk, const bf16_t*& kp,
                                        const bf16_t*& vp) {
  kp = vp = nullptr;
  if (j >= Lk) return;
  if (j < n_ctx) {
    kp = ctx_kv + (j * H + h) * D;
    vp = ctx_kv + ((int64_t)n_ctx * H + j * H + h) * D;
  } else if (j >= ctx_pad) {
    kp = k + ((j - ctx_pad) * H + h) * D;
    vp = v + ((j - ctx_pad) * H + h) * D;
  }
}

// one block = 64 keys of one head; thread = (key tid / 4, quarter tid % 4 of its 128 channels)
__global__ __launch_bounds__(256) void amax_fp8_kernel(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                                       const bf16_t* __restrict__ ctx_kv, float* __restrict__ part,
                                                       int H, int n_ctx, int ctx_pad, int64_t Lk) {
  const int h = blockIdx.y, tid = threadIdx.x;
  const int64_t j = (int64_t)blockIdx.x * 64 + tid / 4;
  const int q0 = (tid % 4) * 32;
  const bf16_t *kp, *vp;
  key_src(k, v, ctx_kv, j, h, H, n_ctx, ctx_pad, Lk, kp, vp);
  float mk = 0.f, mv = 0.f, ss = 0.f;
  if (kp) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 kk = *reinterpret_cast<const uint4*>(kp + q0 + 8 * c);
      const uint4 vv = *reinterpret_cast<const uint4*>(vp + q0 + 8 * c);
      const bf16_t* ke = reinterpret_cast<const bf16_t*>(&kk);
      const bf16_t* ve = reinterpret_cast<const bf16_t*>(&vv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float a = to_f32(ke[i]), b = to_f32(ve[i]);
        mk = fmaxf(mk, fabsf(a));
        mv = fmaxf(mv, fabsf(b));
        ss += a * a;
      }
    }
  }
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
  float mn = sqrtf(ss);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    mk = fmaxf(mk, __shfl_xor(mk, off));
    mv = fmaxf(mv, __shfl_xor(mv, off));
    mn = fmaxf(mn, __shfl_xor(mn, off));
  }
  __shared__ float red[4][3];
  if ((tid & 63) == 0) {
    red[tid / 64][0] = mk;
    red[tid / 64][1] = mv;
    red[tid / 64][2] = mn;
  }
  __syncthreads();
  if (tid < 3) {
    const float m = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
    part[((int64_t)h * gridDim.x + blockIdx.x) * 3 + tid] = m;
  }
}

// one block per head: scales [H][2] (s_k, s_v) and the largest key norm kmax [H]
__global__ __launch_bounds__(256) void scales_fp8_kernel(const float* __restrict__ part, float* __restrict__ scale,
                                                         float* __restrict__ kmax, int nblk) {
  const int h = blockIdx.x, tid = threadIdx.x;
  float m[3] = {0.f, 0.f, 0.f};
  for (int i = tid; i < nblk; i += 256)
#pragma unroll
    for (int c = 0; c < 3; ++c) m[c] = fmaxf(m[c], part[((int64_t)h * nblk + i) * 3 + c]);
  __shared__ float red[3][256];
#pragma unroll
  for (int c = 0; c < 3; ++c) red[c][tid] = m[c];
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s)
#pragma unroll
      for (int c = 0; c < 3; ++c) red[c][tid] = fmaxf(red[c][tid], red[c][tid + s]);
    __syncthreads();
  }
  if (tid == 0) {
    scale[2 * h] = pow2_scale(red[0][0]);
    scale[2 * h + 1] = pow2_scale(red[1][0]);
    kmax[h] = red[2][0];
  }
}

// four E4M3 bytes (round to nearest even) of s * x[0..3]
__device__ __forceinline__ uint32_t e4m3x4(float s, float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(s * a, s * b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(s * c, s * d, w, true);
  return (uint32_t)w;
}

// one block = 64 keys of one head: K8 rows straight through (thread = key, quarter); V8 through
// LDS for the transpose (thread = channel row, 16-key chunk; two items per thread)
__global__ __launch_bounds__(256) void pack_fp8_kernel(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                                       const bf16_t* __restrict__ ctx_kv,
                                                       const float* __restrict__ scale, uint8_t* __restrict__ k8,
                                                       uint8_t* __restrict__ v8, int H, int n_ctx, int ctx_pad,
                                                       int64_t Lk, int64_t Ls8) {
  const int h = blockIdx.y, tid = threadIdx.x;
  const int64_t key0 = (int64_t)blockIdx.x * 64;
  const float sk = scale[2 * h], sv = scale[2 * h + 1];
  __shared__ bf16_t tile[64][D + 8];
  {
    const int r = tid / 4, q0 = (tid % 4) * 32;
    const bf16_t *kp, *vp;
    key_src(k, v, ctx_kv, key0 + r, h, H, n_ctx, ctx_pad, Lk, kp, vp);
    uint32_t out[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 kk = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (kp) {
        kk = *reinterpret_cast<const uint4*>(kp + q0 + 8 * c);
        vv = *reinterpret_cast<const uint4*>(vp + q0 + 8 * c);
      }
      const bf16_t* ke = reinterpret_cast<const bf16_t*>(&kk);
      out[2 * c] = e4m3x4(sk, to_f32(ke[0]), to_f32(ke[1]), to_f32(ke[2]), to_f32(ke[3]));
      out[2 * c + 1] = e4m3x4(sk, to_f32(ke[4]), to_f32(ke[5]), to_f32(ke[6]), to_f32(ke[7]));
      *reinterpret_cast<uint4*>(&tile[r][q0 + 8 * c]) = vv;
    }
    uint8_t* dst = k8 + ((int64_t)h * Ls8 + key0 + r) * D + q0;
    *reinterpret_cast<uint4*>(dst) = make_uint4(out[0], out[1], out[2], out[3]);
    *reinterpret_cast<uint4*>(dst + 16) = make_uint4(out[4], out[5], out[6], out[7]);
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int e = tid + 256 * it;
    const int dr = e / 4, c = e % 4;                // channel row, 16-key chunk
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = e4m3x4(sv, to_f32(tile[16 * c + 4 * i][dr]), to_f32(tile[16 * c + 4 * i + 1][dr]),
                    to_f32(tile[16 * c + 4 * i + 2][dr]), to_f32(tile[16 * c + 4 * i + 3][dr]));
    *reinterpret_cast<uint4*>(v8 + ((int64_t)h * D + dr) * Ls8 + key0 + 16 * c) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

hipError_t launch_prep_fp8(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  if (s.d != D) return hipErrorInvalidValue;
  const int nblk = (int)((s.Lk + 63) / 64);
  const dim3 grid(nblk, s.H);
  amax_fp8_kernel<<<grid, 256, 0, st>>>((const bf16_t*)in.k, (const bf16_t*)in.v, (const bf16_t*)in.text_kv, b.part8,
                                        s.H, s.n_ctx, s.ctx_pad, s.Lk);
  scales_fp8_kernel<<<s.H, 256, 0, st>>>(b.part8, b.scale8, b.kmax, nblk);
  pack_fp8_kernel<<<grid, 256, 0, st>>>((const bf16_t*)in.k, (const bf16_t*)in.v, (const bf16_t*)in.text_kv, b.scale8,
                                        b.k8, b.v8, s.H, s.n_ctx, s.ctx_pad, s.Lk, s.Ls8);
  return hipGetLastError();
}

}  // namespace vdn
