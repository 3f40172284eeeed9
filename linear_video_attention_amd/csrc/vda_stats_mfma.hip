// MFMA statistics of Video Delta Attention (bf16 plans, d in {64, 128}): per (frame or text, head)
// the weighted key Gram A = sum_u beta_u k_u k_u^T and write matrix B = sum_u beta_u v_u k_u^T,
// written as I + A (inverted in place by the next kernel) and B.
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Video Delta
// Attention: A Frame-Wise Solution": a frame's tokens jointly update the state as
// S <- (S + B)(I + A)^-1.  Section "Local Softmax and Long-Range Linear Memory": the text enters
// once, at half strength in each direction (weights beta/2), as one joint update from S = 0.
//
// [A; B] = [K V]^T Diag(beta) K is one (2d x d) product with the frame's tokens as the reduction
// dimension.  Tokens stream through LDS 64 at a time, written transposed (feature rows, token
// columns) so both MFMA operands are read as token-contiguous 16-byte fragments:
//   X^T = [K V]^T (2d rows, exact: the inputs are bf16), Y^T = (Diag(beta) K)^T held as two bf16
//   parts hi + lo (beta * k = hi + lo to ~2^-16), so A and B keep near-fp32 accuracy and A stays
//   symmetric (the scan reads M = (I + A)^-1 by rows using M^T = M).
// Feature f = 8c + e of a 16-byte chunk c is stored at row e * (d/8) + c, so the eight 2-byte
// LDS writes of one chunk land in different banks for neighbouring chunks; the MFMA row and column
// order is free, and the mapping is undone when the result is written.  4 waves: waves 0-1 own the
// rows of A, waves 2-3 those of B.  HBM-bound: every K/V/beta byte of the frame is read once.
#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kTU = 64;             // tokens per tile
constexpr int kLDT = kTU + 8;       // token stride of the transposed tiles (bf16 elements)

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

template <int D>
struct GramSmem {
  static constexpr int CH = D / 8;
  static constexpr int X_BYTES = 2 * D * kLDT * 2;
  static constexpr int Y_BYTES = 2 * D * kLDT * 2;       // hi and lo parts
  static constexpr int A_BYTES = D * (D + 1) * 4;
  static constexpr int TILE_BYTES = X_BYTES + Y_BYTES;
  static constexpr int MAIN = TILE_BYTES > A_BYTES ? TILE_BYTES : A_BYTES;
  static constexpr int TOTAL = MAIN;
};

template <int D>
__device__ __forceinline__ int feat_of_row(int p) {   // inverse of row(f) = (f % 8) * (D/8) + f / 8
  constexpr int CH = D / 8;
  return (p % CH) * 8 + p / CH;
}

template <int D>
__global__ __launch_bounds__(256) void vda_gram_mfma_kernel(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                                            const float* __restrict__ beta,
                                                            const bf16_t* __restrict__ text_kv,
                                                            float* __restrict__ minv, float* __restrict__ bw, int T,
                                                            int N, int H, int n_text, int anchors) {
  using SM = GramSmem<D>;
  constexpr int CH = SM::CH;
  constexpr int MT = 2 * D / 32 / 4;        // M tiles (32 rows of X^T) per wave
  constexpr int NT = D / 32;                // N tiles (32 rows of Y^T)
  constexpr int CHUNKS = kTU * CH;          // 16-byte chunks per matrix per tile
  constexpr int CPT = 2 * CHUNKS / 256;     // chunks per thread (K and V)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16_t* xt = reinterpret_cast<bf16_t*>(smem);
  bf16_t* yt = reinterpret_cast<bf16_t*>(smem + SM::X_BYTES);          // hi part
  bf16_t* yl = yt + D * kLDT;                                           // lo part

  const int slot = blockIdx.x, h = blockIdx.y;
  if (slot > 0 && anchors && (slot - 1 == 0 || slot - 1 == T - 1)) return;   // boundary frames are never written
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hl = lane >> 5;

  const int U = slot == 0 ? n_text : N;
  const int64_t tok0 = slot == 0 ? 0 : (int64_t)(slot - 1) * N;
  const bf16_t* kbase = slot == 0 ? text_kv : k;
  const bf16_t* vbase = slot == 0 ? text_kv + (int64_t)n_text * H * D : v;
  const float wscale = slot == 0 ? 0.5f : 1.0f;
  const int64_t brow0 = slot == 0 ? 0 : n_text + tok0;

  u32x4 reg[CPT];
  float wreg[CPT];
  auto load = [&](int u0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int e = i * 256 + tid;
      const int m = e / CHUNKS, rem = e % CHUNKS;     // m: 0 = K, 1 = V
      const int tok = rem / CH, c = rem % CH;
      const int u = u0 + tok;
      u32x4 val = {0, 0, 0, 0};
      float wv = 0.f;
      if (u < U) {
        const int64_t off = ((tok0 + u) * H + h) * D + c * 8;
        val = *reinterpret_cast<const u32x4*>((m == 0 ? kbase : vbase) + off);
        if (m == 0) wv = wscale * beta[(brow0 + u) * H + h];
      }
      reg[i] = val;
      wreg[i] = wv;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int e = i * 256 + tid;
      const int m = e / CHUNKS, rem = e % CHUNKS;
      const int tok = rem / CH, c = rem % CH;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int row = q * CH + c;
        const bf16_t el = (bf16_t)((q & 1) ? (reg[i][q >> 1] >> 16) : (reg[i][q >> 1] & 0xFFFFu));
        xt[(m * D + row) * kLDT + tok] = el;
        if (m == 0) {
          const float wk = wreg[i] * to_f32(el);
          const __bf16 wh = (__bf16)wk;
          const __bf16 wl = (__bf16)(wk - (float)wh);
          yt[row * kLDT + tok] = __builtin_bit_cast(bf16_t, wh);
          yl[row * kLDT + tok] = __builtin_bit_cast(bf16_t, wl);
        }
      }
    }
  };

  f32x16 acc[MT][NT];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  if (U > 0) load(0);
  for (int u0 = 0; u0 < U; u0 += kTU) {
    __syncthreads();                        // previous tile fully consumed
    store();
    __syncthreads();
    if (u0 + kTU < U) load(u0 + kTU);
#pragma unroll
    for (int ks = 0; ks < kTU / 16; ++ks) {
      bf16x8 bfr[NT], bfl[NT];
#pragma unroll
      for (int b = 0; b < NT; ++b) {
        bfr[b] = as_bf16x8(*reinterpret_cast<const u32x4*>(yt + (b * 32 + l32) * kLDT + ks * 16 + hl * 8));
        bfl[b] = as_bf16x8(*reinterpret_cast<const u32x4*>(yl + (b * 32 + l32) * kLDT + ks * 16 + hl * 8));
      }
#pragma unroll
      for (int a = 0; a < MT; ++a) {
        const int xrow = (wave * MT + a) * 32 + l32;
        const bf16x8 afr = as_bf16x8(*reinterpret_cast<const u32x4*>(xt + xrow * kLDT + ks * 16 + hl * 8));
#pragma unroll
        for (int b = 0; b < NT; ++b) {
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr, bfr[b], acc[a][b], 0, 0, 0);
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr, bfl[b], acc[a][b], 0, 0, 0);
        }
      }
    }
  }
  __syncthreads();                          // tiles no longer needed: the LDS now holds I + A

  float* af = reinterpret_cast<float*>(smem);           // [D][D + 1]
  const int64_t DD = (int64_t)D * D;
  const int64_t mbase = ((int64_t)slot * H + h) * DD;
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int prow = (wave * MT + a) * 32 + 8 * (r / 4) + 4 * hl + (r % 4);
        const int j = feat_of_row<D>(b * 32 + l32);
        if (prow < D) {
          const int i = feat_of_row<D>(prow);
          af[i * (D + 1) + j] = acc[a][b][r] + (i == j ? 1.0f : 0.0f);
        } else {
          const int i = feat_of_row<D>(prow - D);
          bw[mbase + (int64_t)i * D + j] = acc[a][b][r];
        }
      }
  __syncthreads();
  for (int e = tid; e < D * D; e += 256) minv[mbase + e] = af[(e / D) * (D + 1) + e % D];   // I + A, inverted later
}

template <int D>
void launch_t(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  const size_t smem = GramSmem<D>::TOTAL;
  (void)hipFuncSetAttribute((const void*)vda_gram_mfma_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)smem);
  hipLaunchKernelGGL(vda_gram_mfma_kernel<D>, dim3(s.T + 1, s.H), dim3(256), smem, st, (const bf16_t*)in.k,
                     (const bf16_t*)in.v, in.beta, (const bf16_t*)in.text_kv, b.minv, b.bw, s.T, s.N, s.H, s.n_text,
                     s.anchors);
}

}  // namespace

hipError_t launch_vda_stats_mfma(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  if (s.d == 128) launch_t<128>(s, in, b, st);
  else launch_t<64>(s, in, b, st);
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : launch_vda_invert_mfma(s, b, st);
}

}  // namespace vdn
