// MFMA statistics of Video Delta Attention (bf16 plans, d in {64, 128}): per (frame or text, head)
// the weighted key Gram A = sum_u beta_u k_u k_u^T and write matrix B = sum_u beta_u v_u k_u^T,
// written as I + A (inverted in place by the next kernel) and B.
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Video Delta
// Attention: A Frame-Wise Solution": a frame's tokens jointly update the state as
// S <- (S + B)(I + A)^-1.  Section "Local Softmax and Long-Range Linear Memory": the text enters
// once, at half strength in each direction (weights beta/2), as one joint update from S = 0.
//
// [A; B] = [K V]^T Diag(beta) K is one (2d x d) product with the tokens as the reduction
// dimension, run on v_mfma_f32_32x32x16_bf16:
//   * tokens stream through LDS 32 (d = 128) or 64 at a time, copied straight from global memory in their natural
//     token-major layout (global_load_lds, three stages: two tiles in flight while one is used),
//     16-byte chunks XOR-swizzled per row; beta comes along the same way;
//   * Y = Diag(beta) K is formed once per tile in LDS as two bf16 parts, beta k = Yh + Yl to
//     ~2^-16, so A and B keep near-fp32 accuracy (X = [K V] is exact: the inputs are bf16);
//   * both MFMA operands need eight consecutive tokens of one feature per lane: they are read
//     with ds_read_b64_tr_b16, which hands lane j of each 16-lane group the 4 values at column j
//     of the 4 x 16 block that the group's 16 addresses describe (two reads per fragment);
//   * 8 waves: wave w owns X rows [32 MT (w % 4), +32 MT) (K features for w % 4 < 2, V features
//     otherwise) and Y columns [32 NT (w / 4), +32 NT), MT = NT = d / 64.
// Every K/V/beta byte of the frame is read once.
#include <type_traits>

#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 lds_bf16x4;

// tokens per tile: 32 at d = 128 (70 KB of LDS, two workgroups per CU, so every frame of a 768p
// layer is resident at once: 0.207 -> 0.180 ms with the inverse), 64 at d = 64 (a DMA instruction
// per wave needs 8 KB tiles)
#ifndef VDN_GRAM_TU
#define VDN_GRAM_TU 32
#endif
template <int D>
constexpr int tile_tokens() { return D == 128 ? VDN_GRAM_TU : 64; }
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

// 16-byte chunk c of token row r sits at chunk position c ^ swz(r).  The transposed reads of one
// half-wave cover 4 consecutive rows x 64 bytes; the swizzle spreads them over all 64 banks.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return 4 * (r & 3);
  else return 4 * ((r >> 1) & 1);
}

constexpr int kStages = 3;

template <int D>
struct GramSmem {
  static constexpr int ROW = 2 * D;                    // bytes per token row
  static constexpr int kTU = tile_tokens<D>();
  static constexpr int TILE = kTU * ROW;               // one matrix, one tile
  static constexpr int BETA = 2 * TILE;                // beta: wave w's 256 bytes hold tokens 8w..8w+7
  static constexpr int STAGE = BETA + kWaves * 256;    // K, V, beta
  static constexpr int Y_OFF = kStages * STAGE;
  static constexpr int TOTAL = Y_OFF + 2 * TILE;       // Yh, Yl
};

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
  return (uint32_t)(size_t)((const __attribute__((address_space(3))) unsigned char*)p);
}
__device__ __forceinline__ bf16x8 cat2(u32x2 a, u32x2 b) {
  return cat(__builtin_bit_cast(bf16x4, a), __builtin_bit_cast(bf16x4, b));
}

// The transposed fragment reads of one k-step (ds_read_b64_tr_b16) as one asm block that waits for
// its own reads.  Issued through the builtin, each such read gets a vmcnt(0) from the compiler
// while any LDS DMA copy is in flight (it cannot tell the read from the stage being filled), which
// completed the tiles in flight before every k-step and left the copies of later tiles no time to
// overlap the products.  A fragment is two reads, rows r and r + 4 of the block (R4 bytes apart);
// the Y operand has the high and low planes TILE bytes apart.
//   d = 128 (two Y and two X fragments per wave): ya[nt], xa[mt] are the fragment base addresses
//   without the k-step offset KB.
template <int KB, int TILE, int R4>
__device__ __forceinline__ void ks_frags(const uint32_t (&ya)[2], const uint32_t (&xa)[2], bf16x8 (&yf)[2][2],
                                         bf16x8 (&xf)[2]) {
  u32x2 r0, r1, r2, r3, r4, r5, r6, r7, r8, r9, r10, r11;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %12 offset:%c16\n\t"
      "ds_read_b64_tr_b16 %1, %12 offset:%c17\n\t"
      "ds_read_b64_tr_b16 %2, %12 offset:%c18\n\t"
      "ds_read_b64_tr_b16 %3, %12 offset:%c19\n\t"
      "ds_read_b64_tr_b16 %4, %13 offset:%c16\n\t"
      "ds_read_b64_tr_b16 %5, %13 offset:%c17\n\t"
      "ds_read_b64_tr_b16 %6, %13 offset:%c18\n\t"
      "ds_read_b64_tr_b16 %7, %13 offset:%c19\n\t"
      "ds_read_b64_tr_b16 %8, %14 offset:%c16\n\t"
      "ds_read_b64_tr_b16 %9, %14 offset:%c17\n\t"
      "ds_read_b64_tr_b16 %10, %15 offset:%c16\n\t"
      "ds_read_b64_tr_b16 %11, %15 offset:%c17\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7), "=&v"(r8),
        "=&v"(r9), "=&v"(r10), "=&v"(r11)
      : "v"(ya[0]), "v"(ya[1]), "v"(xa[0]), "v"(xa[1]), "i"(KB), "i"(KB + R4), "i"(TILE + KB), "i"(TILE + KB + R4));
  yf[0][0] = cat2(r0, r1);
  yf[0][1] = cat2(r2, r3);
  yf[1][0] = cat2(r4, r5);
  yf[1][1] = cat2(r6, r7);
  xf[0] = cat2(r8, r9);
  xf[1] = cat2(r10, r11);
}
//   d = 64 (one Y and one X fragment per wave)
template <int KB, int TILE, int R4>
__device__ __forceinline__ void ks_frags(const uint32_t (&ya)[1], const uint32_t (&xa)[1], bf16x8 (&yf)[1][2],
                                         bf16x8 (&xf)[1]) {
  u32x2 r0, r1, r2, r3, r4, r5;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %6 offset:%c8\n\t"
      "ds_read_b64_tr_b16 %1, %6 offset:%c9\n\t"
      "ds_read_b64_tr_b16 %2, %6 offset:%c10\n\t"
      "ds_read_b64_tr_b16 %3, %6 offset:%c11\n\t"
      "ds_read_b64_tr_b16 %4, %7 offset:%c8\n\t"
      "ds_read_b64_tr_b16 %5, %7 offset:%c9\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5)
      : "v"(ya[0]), "v"(xa[0]), "i"(KB), "i"(KB + R4), "i"(TILE + KB), "i"(TILE + KB + R4));
  yf[0][0] = cat2(r0, r1);
  yf[0][1] = cat2(r2, r3);
  xf[0] = cat2(r4, r5);
}

template <int D>
__global__ __launch_bounds__(kThreads) void vda_gram_mfma_kernel(const bf16_t* __restrict__ k,
                                                                 const bf16_t* __restrict__ v,
                                                                 const float* __restrict__ beta,
                                                                 const bf16_t* __restrict__ text_kv,
                                                                 float* __restrict__ minv, float* __restrict__ bw,
                                                                 int T, int N, int H, int n_text, int n_ctx,
                                                                 int anchors) {
  using SM = GramSmem<D>;
  constexpr int CH = D / 8;                 // 16-byte chunks per token row
  constexpr int ROWS_PER_KB = 1024 / SM::ROW;
  constexpr int DMA = SM::TILE / 1024 / kWaves;   // DMA instructions per wave per matrix and tile
  constexpr int kTU = SM::kTU;
  constexpr int YCH = kTU * CH / kThreads;        // Y chunks per thread per tile
  constexpr int MT = D / 64, NT = D / 64;
  constexpr int kVmcntTile = 0x0F70 | (2 * DMA + 1);   // s_waitcnt vmcnt(one tile's loads of a wave)
  static_assert(2 * DMA + 1 < 16, "vmcnt field");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int slot = blockIdx.x, h = blockIdx.y;
  if (slot > 0 && anchors && (slot - 1 == 0 || slot - 1 == T - 1)) return;   // boundary frames are never written
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  const int U = slot == 0 ? n_text : N;
  const int64_t tok0 = slot == 0 ? 0 : (int64_t)(slot - 1) * N;
  const bf16_t* kbase = slot == 0 ? text_kv : k;
  const bf16_t* vbase = slot == 0 ? text_kv + (int64_t)n_ctx * H * D : v;   // V half of [2][n_ctx][H][d]
  const float wscale = slot == 0 ? 0.5f : 1.0f;
  const int64_t brow0 = slot == 0 ? 0 : n_text + tok0;
  const int ntiles = (U + kTU - 1) / kTU;

  // DMA: instruction i of wave w fills token rows (i*kWaves + w)*ROWS_PER_KB + lane / CH; lane
  // writes chunk position lane % CH, so it fetches chunk (lane % CH) ^ swz(row).  Rows past the
  // last token re-read the last token; beta is read for tokens 8w + lane % 8 (clamped the same
  // way) and zeroed past the last token when Y is formed.  Every wave issues 2 DMA + 1 loads per
  // tile and nothing else, so one explicit vmcnt per tile covers them.
  auto issue_tile = [&](int u0, int stage) {
    unsigned char* kb = smem + stage * SM::STAGE;
#pragma unroll
    for (int i = 0; i < DMA; ++i) {
      const int blk = i * kWaves + wave;
      const int row = blk * ROWS_PER_KB + lane / CH;
      const int u = min(u0 + row, U - 1);
      const int c = (lane % CH) ^ swz<D>(row);
      const int64_t off = ((tok0 + u) * H + h) * D + c * 8;
      __builtin_amdgcn_global_load_lds((gptr_t)(kbase + off), (lptr_t)(kb + blk * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gptr_t)(vbase + off), (lptr_t)(kb + SM::TILE + blk * 1024), 16, 0, 0);
    }
    const int ub = min(u0 + 8 * wave + (lane & 7), U - 1);
    __builtin_amdgcn_global_load_lds((gptr_t)(beta + (brow0 + ub) * H + h), (lptr_t)(kb + SM::BETA + wave * 256), 4,
                                     0, 0);
  };

  // transposed-read lane offsets: lane (g = lane / 16, i = lane % 16) addresses token
  // 8 (g / 2) + (i / 4) (+ 4 for the second read) and feature 16 (g % 2) + 4 (i % 4) of a
  // 16-token x 32-feature fragment block
  const int g = lane >> 4, li = lane & 15;
  const int tr_tok = 8 * (g >> 1) + (li >> 2);
  const int tr_feat = 16 * (g & 1) + 4 * (li & 3);
  auto tr_off = [&](int f0) {                         // byte offset for feature block f0, token 0
    const int f = f0 + tr_feat;
    return tr_tok * SM::ROW + (((f >> 3) ^ swz<D>(tr_tok)) << 4) + (f & 7) * 2;
  };
  const int xg = wave & 3, yh = wave >> 2;
  int xoff[MT], yoff[NT];
  bool xv[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int xr = (xg * MT + mt) * 32;                 // X row = K feature (< D) or D + V feature
    xv[mt] = xr >= D;
    xoff[mt] = tr_off(xv[mt] ? xr - D : xr);
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) yoff[nt] = tr_off((yh * NT + nt) * 32);

  f32x16 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.f;

  if (ntiles > 0) issue_tile(0, 0);
  if (ntiles > 1) issue_tile(kTU, 1);
  unsigned char* yb = smem + SM::Y_OFF;
  for (int it = 0; it < ntiles; ++it) {
    if (it + 1 < ntiles) __builtin_amdgcn_s_waitcnt(kVmcntTile);   // tile it landed, it+1 in flight
    else __builtin_amdgcn_s_waitcnt(0x0F70);                       // vmcnt(0)
    lds_barrier();                         // ... for every wave; Y and stage (it+2)%3 (tile it-1) are free
    if (it + 2 < ntiles) issue_tile((it + 2) * kTU, (it + 2) % kStages);
    const unsigned char* kb = smem + (it % kStages) * SM::STAGE;
    // Y = beta k as hi + lo, same chunk positions as K (chunk e = tid + s * kThreads, token e / CH)
#pragma unroll
    for (int s = 0; s < YCH; ++s) {
      const int e = tid + s * kThreads;
      const int tok = e / CH;
      const float bt = it * kTU + tok < U ? wscale * *reinterpret_cast<const float*>(
                                                          kb + SM::BETA + (tok >> 3) * 256 + (tok & 7) * 4)
                                          : 0.f;
      const bf16x8 kv = *reinterpret_cast<const bf16x8*>(kb + e * 16);
      bf16x8 yhv, ylv;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float y = bt * (float)kv[q];
        const __bf16 hi = (__bf16)y;
        yhv[q] = hi;
        ylv[q] = (__bf16)(y - (float)hi);
      }
      *reinterpret_cast<bf16x8*>(yb + e * 16) = yhv;
      *reinterpret_cast<bf16x8*>(yb + SM::TILE + e * 16) = ylv;
    }
    lds_barrier();                                    // Y ready
    uint32_t ya[NT], xa[MT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) ya[nt] = lds_addr(yb) + yoff[nt];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xa[mt] = lds_addr(kb) + (xv[mt] ? SM::TILE : 0) + xoff[mt];
    auto kstep = [&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      bf16x8 yf[NT][2], xf[MT];
      ks_frags<ks * 16 * SM::ROW, SM::TILE, 4 * SM::ROW>(ya, xa, yf, xf);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf[mt], yf[nt][0], acc[mt][nt], 0, 0, 0);
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf[mt], yf[nt][1], acc[mt][nt], 0, 0, 0);
        }
    };
    kstep(std::integral_constant<int, 0>{});
    kstep(std::integral_constant<int, 1>{});
    if constexpr (kTU / 16 > 2) {
      kstep(std::integral_constant<int, 2>{});
      kstep(std::integral_constant<int, 3>{});
    }
  }

  // acc[mt][nt][r]: X row 32 (xg MT + mt) + 8 (r / 4) + 4 (lane / 32) + r % 4, Y column
  // 32 (yh NT + nt) + lane % 32
  const int64_t DD = (int64_t)D * D;
  const int64_t mbase = ((int64_t)slot * H + h) * DD;
  const int l32 = lane & 31, hl = lane >> 5;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int xr = (xg * MT + mt) * 32 + 8 * (r / 4) + 4 * hl + (r % 4);
        const int j = (yh * NT + nt) * 32 + l32;
        if (xr < D) minv[mbase + (int64_t)xr * D + j] = acc[mt][nt][r] + (xr == j ? 1.0f : 0.0f);   // I + A
        else bw[mbase + (int64_t)(xr - D) * D + j] = acc[mt][nt][r];
      }
}

template <int D>
void launch_t(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  const size_t smem = GramSmem<D>::TOTAL;
  (void)hipFuncSetAttribute((const void*)vda_gram_mfma_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)smem);
  hipLaunchKernelGGL(vda_gram_mfma_kernel<D>, dim3(s.T + 1, s.H), dim3(kThreads), smem, st, (const bf16_t*)in.k,
                     (const bf16_t*)in.v, in.beta, (const bf16_t*)in.text_kv, b.minv, b.bw, s.T, s.N, s.H, s.n_text,
                     s.n_ctx, s.anchors);
}

}  // namespace

hipError_t launch_vda_stats_mfma(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  if (s.d == 128) launch_t<128>(s, in, b, st);
  else launch_t<64>(s, in, b, st);
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : launch_vda_invert_mfma(s, in, b, st);
}

}  // namespace vdn
