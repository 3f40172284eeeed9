// Packing of keys and values for the MFMA softmax kernel.
//
// The softmax branch reads, for every query chunk, a few contiguous ranges of keys of one head
// (global keys, window, anchors).  Packing once per forward gives every head one contiguous key
// space [text, audio (padded together to 64) | video tokens] so each key tile is one dense 64 x d
// block:
//   Kp [H][Ls][d]   keys, bf16, row per key
//   Vt [H][d][Ls]   values transposed, bf16, so that the P.V contraction (over keys) reads
//                   key-contiguous 16-byte fragments
// Ls = Lk + 128: a tile of zero keys past the end (zeroed at plan creation, never written here)
// so that a tile load never leaves the buffer.  Padding keys (n_ctx <= j < ctx_pad) are zero;
// the softmax kernel masks them.
// The same pass records the largest key norm of each 64-key block; a second tiny kernel reduces
// them to the largest key norm of each head, which bounds every score of the head
// (|q.k| <= |q| max|k|) and serves the softmax kernel as a fixed exponent reference.
//
// One block per (64-key tile, head): 256 threads copy the 64 x d keys straight through and
// transpose the matching 64 x d values through LDS, 64 dims at a time.
#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

__global__ __launch_bounds__(256) void prep_kv_kernel(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                                      const bf16_t* __restrict__ ctx_kv, bf16_t* __restrict__ kp,
                                                      bf16_t* __restrict__ vt, float* __restrict__ kmax_part, int H,
                                                      int D, int n_ctx, int ctx_pad, int64_t Lk, int64_t Ls) {
  const int64_t key0 = (int64_t)blockIdx.x * 64;
  const int h = blockIdx.y;
  __shared__ bf16_t tile[64][64 + 2];
  __shared__ float sq[64][9];
  const int tid = threadIdx.x;
  float ssq[2] = {0.f, 0.f};
  for (int d0 = 0; d0 < D; d0 += 64) {
    // 64 keys x 64 dims = 512 chunks of 8 bf16
    for (int e = tid, it = 0; e < 512; e += 256, ++it) {
      const int r = e / 8, c = e % 8;
      const int64_t j = key0 + r;
      uint4 kk = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (j < Lk) {
        if (j < n_ctx) {
          const int64_t off = (j * H + h) * D + d0 + c * 8;
          kk = *reinterpret_cast<const uint4*>(ctx_kv + off);
          vv = *reinterpret_cast<const uint4*>(ctx_kv + (int64_t)n_ctx * H * D + off);
        } else if (j >= ctx_pad) {
          const int64_t off = ((j - ctx_pad) * H + h) * D + d0 + c * 8;
          kk = *reinterpret_cast<const uint4*>(k + off);
          vv = *reinterpret_cast<const uint4*>(v + off);
        }
        *reinterpret_cast<uint4*>(kp + ((int64_t)h * Ls + j) * D + d0 + c * 8) = kk;
      }
      const bf16_t* ke = reinterpret_cast<const bf16_t*>(&kk);
      const bf16_t* ve = reinterpret_cast<const bf16_t*>(&vv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        tile[r][c * 8 + i] = ve[i];
        const float kf = to_f32(ke[i]);
        ssq[it] += kf * kf;
      }
    }
    __syncthreads();
    for (int e = tid; e < 512; e += 256) {
      const int dr = e / 8, c = e % 8;
      const int64_t j = key0 + c * 8;
      if (j < Lk) {
        alignas(16) bf16_t buf[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) buf[i] = tile[c * 8 + i][dr];
        *reinterpret_cast<uint4*>(vt + ((int64_t)h * D + d0 + dr) * Ls + j) = *reinterpret_cast<const uint4*>(buf);
      }
    }
    __syncthreads();
  }
  // per-key squared norms: thread (e = tid + 256 it) covered key e / 8, chunk e % 8
  sq[tid / 8][tid % 8] = ssq[0];
  sq[32 + tid / 8][tid % 8] = ssq[1];
  __syncthreads();
  if (tid < 64) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) s += sq[tid][c];
    float m = sqrtf(s);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (tid == 0) kmax_part[(int64_t)h * gridDim.x + blockIdx.x] = m;
  }
}

__global__ __launch_bounds__(256) void kmax_reduce_kernel(const float* __restrict__ kmax_part,
                                                          float* __restrict__ kmax, int nblk) {
  const int h = blockIdx.x;
  __shared__ float red[256];
  float m = 0.f;
  for (int i = threadIdx.x; i < nblk; i += 256) m = fmaxf(m, kmax_part[(int64_t)h * nblk + i]);
  red[threadIdx.x] = m;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0) kmax[h] = red[0];
}

}  // namespace

hipError_t launch_prep_kv(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  const int nblk = (int)((s.Lk + 63) / 64);
  prep_kv_kernel<<<dim3(nblk, s.H), 256, 0, st>>>((const bf16_t*)in.k, (const bf16_t*)in.v,
                                                  (const bf16_t*)in.text_kv, b.kp, b.vt, b.kmax_part, s.H, s.d,
                                                  s.n_ctx, s.ctx_pad, s.Lk, s.Ls);
  kmax_reduce_kernel<<<s.H, 256, 0, st>>>(b.kmax_part, b.kmax, nblk);
  return hipGetLastError();
}

}  // namespace vdn
