// Inverse of I + A and the scan operands of Video Delta Attention (bf16 plans, d in {64, 128}).
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Video Delta
// Attention: A Frame-Wise Solution": a frame updates the state as S <- (S + B)(I + A)^-1 =
// S M + C with M = (I + A)^-1 and C = B M.  Per (frame or text, head) one workgroup
//   1. inverts I + A (written by the statistics kernel into the M buffer) in place by Gauss-Jordan
//      elimination in registers (16 x 16 threads, R x R elements each);
//   2. keeps M in LDS as two bf16 planes, M = Mh + Ml to ~2^-16;
//   3. forms C = B M on v_mfma_f32_16x16x32_bf16 with B split the same way,
//      B M ~ Bh Mh + Bh Ml + Bl Mh, and writes C (fp32);
//   4. writes the frame's step matrix for the scans as two bf16 planes holding its transpose row
//      by row: the step is S <- S G + C with G = Diag(alpha_f) M (the decay gate on the inherited
//      state's key channels; alpha = 1 without it), and G^T = M Diag(alpha_f), so plane row n is
//      row n of M with column k scaled by alpha_f[k] (row n of M itself when there is no decay).
// Boundary frames are never written into a state and are skipped.
#include "dev_common.h"
#include "vda_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__device__ __forceinline__ void split8(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = e < 4 ? a[e] : b[e - 4];
    const __bf16 xh = (__bf16)x;
    hi[e] = xh;
    lo[e] = (__bf16)(x - (float)xh);
  }
}

template <int D>
__global__ __launch_bounds__(256, 2) void vda_invert_kernel(float* __restrict__ minv, const float* __restrict__ bw,
                                                         const float* __restrict__ alpha, float* __restrict__ cw,
                                                         bf16_t* __restrict__ mhl, int T, int H, int anchors) {
  constexpr int R = D / 16;
  constexpr int LDM = D + 8;                 // bf16 row stride of the M planes in LDS
  constexpr int KS = D / 32;                 // k-steps of the 16x16x32 products
  constexpr int RT = D / 64;                 // 16-row tiles of C per wave (4 waves)
  constexpr int CT = D / 16;                 // 16-column tiles of C
  __shared__ __attribute__((aligned(16))) bf16_t mp[2][D][LDM];
  __shared__ __attribute__((aligned(16))) float rowbuf[2 * D], colbuf[2 * D];

  const int slot = blockIdx.x, h = blockIdx.y;
  if (slot > 0 && anchors && (slot - 1 == 0 || slot - 1 == T - 1)) return;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int64_t DD = (int64_t)D * D;
  const int64_t mbase = ((int64_t)slot * H + h) * DD;

  // 1. M = (I + A)^-1
  float g[R][R];
#pragma unroll
  for (int ii = 0; ii < R; ++ii)
#pragma unroll
    for (int j4 = 0; j4 < R / 4; ++j4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(minv + mbase + (int64_t)(ty * R + ii) * D + tx * R + 4 * j4);
#pragma unroll
      for (int e = 0; e < 4; ++e) g[ii][4 * j4 + e] = x[e];
    }
  gauss_jordan_inverse<D>(g, rowbuf, colbuf, ty, tx);

  // 2. M (fp32) out, M planes into LDS
  const float* af = (alpha && slot > 0) ? alpha + ((int64_t)(slot - 1) * H + h) * D + tx * R : nullptr;
#pragma unroll
  for (int ii = 0; ii < R; ++ii) {
#pragma unroll
    for (int j4 = 0; j4 < R / 4; ++j4) {
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = g[ii][4 * j4 + e];
      *reinterpret_cast<f32x4*>(minv + mbase + (int64_t)(ty * R + ii) * D + tx * R + 4 * j4) = x;
    }
#pragma unroll
    for (int jj = 0; jj < R; ++jj) {
      const __bf16 xh = (__bf16)g[ii][jj];
      mp[0][ty * R + ii][tx * R + jj] = __builtin_bit_cast(bf16_t, xh);
      mp[1][ty * R + ii][tx * R + jj] = __builtin_bit_cast(bf16_t, (__bf16)(g[ii][jj] - (float)xh));
    }
  }
  __syncthreads();
  bf16_t* mout = mhl + ((int64_t)slot * H + h) * 2 * DD;
  auto write_planes = [&]() {
    for (int e = tid; e < 2 * D * D / 8; e += 256) {
      const int plane = e / (D * D / 8), rem = e % (D * D / 8);
      const int row = rem / (D / 8), c8 = rem % (D / 8);
      *reinterpret_cast<u32x4*>(mout + plane * DD + (int64_t)row * D + c8 * 8) =
          *reinterpret_cast<const u32x4*>(&mp[plane][row][c8 * 8]);
    }
  };
  if (!af) write_planes();                 // step planes = M planes

  // 3. C = B M: wave w owns rows [RT*16*w, RT*16*(w+1)), all columns
  const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const float* brow = bw + mbase + (int64_t)(RT * 16 * wave + l16) * D + lg * 8;
  f32x4 acc[RT][CT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    bf16x8 xh[RT], xl[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float* bp = brow + (int64_t)rt * 16 * D + ks * 32;
      split8(*reinterpret_cast<const f32x4*>(bp), *reinterpret_cast<const f32x4*>(bp + 4), xh[rt], xl[rt]);
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      // B operand element (k, n) = M[k][n] = M[n][k]: row n of the planes, k contiguous
      const bf16x8 mh = *reinterpret_cast<const bf16x8*>(&mp[0][ct * 16 + l16][ks * 32 + lg * 8]);
      const bf16x8 ml = *reinterpret_cast<const bf16x8*>(&mp[1][ct * 16 + l16][ks * 32 + lg * 8]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh[rt], mh, acc[rt][ct], 0, 0, 0);
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh[rt], ml, acc[rt][ct], 0, 0, 0);
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl[rt], mh, acc[rt][ct], 0, 0, 0);
      }
    }
  }
  // output element (16 rt + 4 lg + i, 16 ct + l16) of the wave's rows
  float* cout = cw + mbase + (int64_t)(RT * 16 * wave + 4 * lg) * D + l16;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) cout[(int64_t)(16 * rt + i) * D + 16 * ct] = acc[rt][ct][i];

  // 4. with a decay gate: step planes = M Diag(alpha_f), rebuilt in LDS once C no longer needs M.
  // Each thread reads back the fp32 elements of M it wrote in step 2 (its own writes, so no fence
  // is needed), which keeps M out of registers across step 3.
  if (af) {
    float a[R];
#pragma unroll
    for (int jj = 0; jj < R; ++jj) a[jj] = af[jj];
    __syncthreads();                       // every wave is done reading the M planes
#pragma unroll
    for (int ii = 0; ii < R; ++ii)
#pragma unroll
      for (int j4 = 0; j4 < R / 4; ++j4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(minv + mbase + (int64_t)(ty * R + ii) * D + tx * R + 4 * j4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int jj = 4 * j4 + e;
          const float gv = x[e] * a[jj];
          const __bf16 xh = (__bf16)gv;
          mp[0][ty * R + ii][tx * R + jj] = __builtin_bit_cast(bf16_t, xh);
          mp[1][ty * R + ii][tx * R + jj] = __builtin_bit_cast(bf16_t, (__bf16)(gv - (float)xh));
        }
      }
    __syncthreads();
    write_planes();
  }
}

}  // namespace

hipError_t launch_vda_invert_mfma(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  const dim3 grid(s.T + 1, s.H);
  if (s.d == 128)
    vda_invert_kernel<128><<<grid, 256, 0, st>>>(b.minv, b.bw, in.alpha, b.cw, b.mhl, s.T, s.H, s.anchors);
  else
    vda_invert_kernel<64><<<grid, 256, 0, st>>>(b.minv, b.bw, in.alpha, b.cw, b.mhl, s.T, s.H, s.anchors);
  return hipGetLastError();
}

}  // namespace vdn
