// Packing of keys and values for the MFMA softmax kernel.
//
// The softmax branch reads, for every query chunk, a few contiguous ranges of keys of one head
// (text, window, anchors).  Packing once per forward gives every head one contiguous key space
// [text (padded to 64) | video tokens] so each key tile is one dense 64 x d block:
//   Kp [H][Lk][d]   keys, bf16, row per key
//   Vt [H][d][Lk]   values transposed, bf16, so that the P.V contraction (over keys) reads
//                   key-contiguous 16-byte fragments
// Padding keys (n_text <= j < text_pad) are zero; the softmax kernel masks them.
//
// One block per (64-key tile, 64-dim slice, head): 256 threads move 64 x 64 bf16 of K straight
// through and transpose the matching 64 x 64 block of V through LDS.
#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

__global__ __launch_bounds__(256) void prep_kv_kernel(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                                      const bf16_t* __restrict__ text_kv, bf16_t* __restrict__ kp,
                                                      bf16_t* __restrict__ vt, int H, int D, int n_text, int text_pad,
                                                      int64_t Lk) {
  const int64_t key0 = (int64_t)blockIdx.x * 64;
  const int d0 = blockIdx.y * 64;
  const int h = blockIdx.z;
  __shared__ bf16_t tile[64][64 + 2];
  const int tid = threadIdx.x;
  // 64 keys x 64 dims = 512 chunks of 8 bf16
  for (int e = tid; e < 512; e += 256) {
    const int r = e / 8, c = e % 8;
    const int64_t j = key0 + r;
    uint4 kk = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (j < Lk) {
      if (j < n_text) {
        const int64_t off = (j * H + h) * D + d0 + c * 8;
        kk = *reinterpret_cast<const uint4*>(text_kv + off);
        vv = *reinterpret_cast<const uint4*>(text_kv + (int64_t)n_text * H * D + off);
      } else if (j >= text_pad) {
        const int64_t off = ((j - text_pad) * H + h) * D + d0 + c * 8;
        kk = *reinterpret_cast<const uint4*>(k + off);
        vv = *reinterpret_cast<const uint4*>(v + off);
      }
      *reinterpret_cast<uint4*>(kp + ((int64_t)h * Lk + j) * D + d0 + c * 8) = kk;
    }
    const bf16_t* ve = reinterpret_cast<const bf16_t*>(&vv);
#pragma unroll
    for (int i = 0; i < 8; ++i) tile[r][c * 8 + i] = ve[i];
  }
  __syncthreads();
  // write Vt rows d0..d0+63, keys key0..key0+63 (8 keys per chunk)
  for (int e = tid; e < 512; e += 256) {
    const int dr = e / 8, c = e % 8;
    const int64_t j = key0 + c * 8;
    if (j < Lk) {
      alignas(16) bf16_t buf[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) buf[i] = tile[c * 8 + i][dr];
      *reinterpret_cast<uint4*>(vt + ((int64_t)h * D + d0 + dr) * Lk + j) = *reinterpret_cast<const uint4*>(buf);
    }
  }
}

}  // namespace

hipError_t launch_prep_kv(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  dim3 grid((unsigned)((s.Lk + 63) / 64), s.d / 64, s.H);
  prep_kv_kernel<<<grid, 256, 0, st>>>((const bf16_t*)in.k, (const bf16_t*)in.v, (const bf16_t*)in.text_kv, b.kp,
                                       b.vt, s.H, s.d, s.n_text, s.text_pad, s.Lk);
  return hipGetLastError();
}

}  // namespace vdn
