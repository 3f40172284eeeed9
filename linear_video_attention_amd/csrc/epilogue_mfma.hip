// MFMA epilogue of the VDN layer (bf16 plans, d in {64, 128}): linear readout, RMSNorm, the two
// sigmoid gates, the two output projections and their sum.
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Local Softmax and
// Long-Range Linear Memory": o_l = (S_fwd + S_rev) q.  Section "Gating the Softmax and Linear Branch
// Outputs": out = (sigmoid(q Wg0) * o_s) Wp0 + (sigmoid(q Wg1) * RMSNorm(o_l)) Wp1 (gate input q,
// weights [in][out] shared by the heads, RMSNorm eps 1e-6 with unit weight).
//
// RMSNorm scales each token's o_l by one number r = 1/sqrt(mean(o_l^2) + eps), and that scalar
// commutes with the projection: (g_l * o_l * r) Wp1 = r ((g_l * o_l) Wp1).  So the work splits into
// two stages that never wait for each other inside a tile:
//   * readout waves (0-3): per 64-token tile, o_l^T, (q Wg0)^T, (q Wg1)^T = [S; Wg0^T; Wg1^T] q^T,
//     then x_s = sigmoid(q Wg0) * o_s and z_l = sigmoid(q Wg1) * o_l, written to LDS (z_l as bf16
//     hi + lo parts), plus each wave's partial sum of o_l^2 per token;
//   * projection waves (4-7): one tile behind, out^T = Wp0^T x_s^T + r (Wp1^T z_l^T), with r from
//     the four partial sums, stored as bf16.
// One barrier per tile hands the tile over (double-buffered x planes and partials); it orders LDS
// only, so the q copies, o_s loads and output stores in flight stay in flight across it.  Every product
// is computed transposed (channels x tokens) with v_mfma_f32_16x16x32_bf16 so that the matrix
// shared by all tokens -- S (as bf16 hi + lo, since the readout needs ~16 mantissa bits) and the
// pre-transposed weights -- is the A operand and stays in registers: each wave owns 16 CT
// channels.  q tiles are copied straight into LDS (global_load_lds, three buffers, issued two
// tiles ahead by the readout waves, which are their only readers); all LDS tiles are token rows
// with 16-byte chunks XOR-swizzled so the 16-lane fragment reads are bank-conflict free.
//
// MXFP8 variant (MX = true, d = 128): the four d x d products take E4M3 operands in blocks of 32
// along the contraction axis, each block with a power-of-two scale 2^X, X = max(e - 8, -127) for
// a largest magnitude f 2^e (f in [0.5, 1)), on v_mfma_scale_f32_16x16x128_f8f6f4 (the whole
// contraction in one instruction; the block scales are its E8M0 scale operands).  The readout
// stays split bf16.  In that instruction lane group g (lanes 16g .. 16g+15) holds k = 16g .. +15
// in its first 16 bytes and k = 64 + 16g .. +15 in its last 16, and supplies the scale of k block
// g: each readout lane quantises its own two q half-blocks (block maxima from the partner lane
// group) and fetches the scale it must supply from the lane group that holds that block's first
// half.  x_s and z_l are quantised per token and 32-channel block -- exactly one readout wave's
// channels -- and handed over as two E4M3 planes plus one scale byte per token and block.
#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

constexpr int kTileTok = 64;
constexpr int kSub = kTileTok / 16;      // 16-token column tiles per tile
#ifndef VDN_EPI_TOKENS
#define VDN_EPI_TOKENS 768
#endif
constexpr int kTokPerWG = VDN_EPI_TOKENS;   // tokens of one frame and head per workgroup (384: 11 %, 1536: 19 % slower)
constexpr int kQBufs = 3;

// 16-byte chunk c of token row r sits at chunk position c ^ swz(r): the 16 rows read by one
// 16-lane fragment load then cover all 64 banks.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return r & 15;
  else return (r >> 1) & 7;
}

template <int D, bool MX>
struct EpiSmem {
  static constexpr int ROW = 2 * D;                          // bytes per token row
  static constexpr int PLANE = kTileTok * ROW;
  static constexpr int PLANE8 = kTileTok * D;                // E4M3 planes (MX)
  static constexpr int Q_OFF = 0;                            // kQBufs q tiles
  static constexpr int X_OFF = kQBufs * PLANE;               // [2][3] planes: x_s, z_l hi, z_l lo
                                                             // (MX: [2][2] E4M3 planes x_s, z_l)
  static constexpr int SC_OFF = X_OFF + (MX ? 4 * PLANE8 : 6 * PLANE);  // MX: [2][2][kTileTok][4] scale bytes
  static constexpr int P_OFF = SC_OFF + (MX ? 2 * 2 * kTileTok * 4 : 0);  // [2][4 waves][kTileTok] floats
  static constexpr int TOTAL = P_OFF + 2 * 4 * kTileTok * 4;
};

// Block exponent of the MX format: X = max(e - 8, -127) for m = f 2^e (f in [0.5, 1)), 0 for
// m = 0 (m >= 0; every subnormal m gives -127).
__device__ __forceinline__ int mx_exponent(float m) {
  const int E = (int)((__float_as_uint(m) >> 23) & 0xFFu);
  if (E == 0) return m > 0.f ? -127 : 0;
  return max(E - 134, -127);
}

// 2^x for -126 <= x <= 127
__device__ __forceinline__ float exp2i(int x) { return __uint_as_float((uint32_t)(x + 127) << 23); }

// four floats, already scaled into the block's range, as E4M3 codes (nearest, ties to even)
__device__ __forceinline__ int pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// MX weights: wt8[m][j][i] = E4M3 code of W_m[i][j] / 2^X and wsc8[m][j][b] = X + 127, X the
// exponent of block b = i / 32 of column j (gate_w[0], gate_w[1], proj_w[0], proj_w[1])
__global__ __launch_bounds__(512) void prep_weights_mx_kernel(const bf16_t* __restrict__ gate_w,
                                                              const bf16_t* __restrict__ proj_w,
                                                              uint8_t* __restrict__ wt8, uint8_t* __restrict__ wsc8,
                                                              int D) {
  const int m = blockIdx.y;
  const bf16_t* src = m < 2 ? gate_w + (int64_t)m * D * D : proj_w + (int64_t)(m - 2) * D * D;
  const int nb = D / 32;
  for (int e = blockIdx.x * 512 + threadIdx.x; e < D * nb; e += gridDim.x * 512) {
    const int j = e % D, b = e / D;           // consecutive threads: consecutive columns (coalesced reads)
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      v[t] = __uint_as_float((uint32_t)src[(int64_t)(32 * b + t) * D + j] << 16);
      amax = fmaxf(amax, fabsf(v[t]));
    }
    const int X = mx_exponent(amax);
    const float sc = exp2i(-X);
    uint8_t* dst = wt8 + ((int64_t)m * D + j) * D + 32 * b;
#pragma unroll
    for (int i4 = 0; i4 < 8; ++i4)
      reinterpret_cast<int*>(dst)[i4] = pack4_e4m3(v[4 * i4] * sc, v[4 * i4 + 1] * sc, v[4 * i4 + 2] * sc, v[4 * i4 + 3] * sc);
    wsc8[((int64_t)m * D + j) * nb + b] = (uint8_t)(X + 127);
  }
}

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

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

template <int D, bool MX>
__global__ __launch_bounds__(512) void epilogue_mfma_kernel(const bf16_t* __restrict__ q,
                                                            const bf16_t* __restrict__ o_s,
                                                            const float* __restrict__ states,
                                                            const bf16_t* __restrict__ wt,
                                                            const uint8_t* __restrict__ wt8,
                                                            const uint8_t* __restrict__ wsc8, bf16_t* __restrict__ out,
                                                            int T, int N, int H, int C, int Nc, int anchors,
                                                            int wg_per_frame) {
  using SM = EpiSmem<D, MX>;
  static_assert(!MX || D == 128, "MX epilogue: d = 128 (one readout wave per 32-channel block)");
  constexpr int CT = D / 64;              // 16-channel tiles per wave (4 waves per stage cover D)
  constexpr int KS = D / 32;              // k-steps of 32
  constexpr int CH = D / 8;               // 16-byte chunks per token row
  constexpr int ROWS_PER_KB = 1024 / SM::ROW;
  constexpr int QDMA = SM::PLANE / 1024 / 4;      // q DMA instructions per readout wave per tile
  constexpr int kVmcntTile = 0x0F70 | QDMA;       // s_waitcnt vmcnt(one tile's q loads of a wave)
  static_assert(QDMA < 16, "vmcnt field");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int wg = blockIdx.x, h = blockIdx.y;
  const int t = wg / wg_per_frame;
  const int tok_begin = (wg % wg_per_frame) * kTokPerWG;
  const int tok_end = min(N, tok_begin + kTokPerWG);
  const int ntiles = (tok_end - tok_begin + kTileTok - 1) / kTileTok;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  const bool readout = wave < 4;
  const int sw = wave & 3;                 // wave index within its stage
  const int64_t DD = (int64_t)D * D;
  auto tok_row = [&](int n) { return ((int64_t)t * N + n) * H + h; };

  // fragment byte offset of (token row r, channels k0 .. k0+7) in a swizzled tile
  auto frag_off = [&](int r, int k0) { return r * SM::ROW + (((k0 >> 3) ^ swz<D>(r)) << 4); };
  // byte offset of (token row r, channels 16 c .. 16 c + 15) in an E4M3 plane (MX)
  auto off8 = [&](int r, int c) { return r * D + ((c ^ (r & 7)) << 4); };
  // MX weight fragment (A operand) of matrix m, row j, for this lane's group, and its scale
  auto wfrag8 = [&](int m, int j, i32x8& a, int& sc) {
    const uint8_t* row = wt8 + ((int64_t)m * D + j) * D;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(row + 16 * lg);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(row + 64 + 16 * lg);
    a = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    sc = wsc8[((int64_t)m * D + j) * (D / 32) + lg];
  };

  // q DMA (readout waves): instruction i of stage wave sw fills token rows
  // (i*4 + sw)*ROWS_PER_KB + lane / CH; the lane fetches chunk (lane % CH) ^ swz(row).  Rows past the
  // last token re-read the last token (their results are never stored).
  auto issue_q = [&](int it) {
    unsigned char* qb = smem + SM::Q_OFF + (it % kQBufs) * SM::PLANE;
    const int tok0 = tok_begin + it * kTileTok;
#pragma unroll
    for (int i = 0; i < QDMA; ++i) {
      const int blk = i * 4 + sw;
      const int row = blk * ROWS_PER_KB + lane / CH;
      const int n = min(tok0 + row, tok_end - 1);
      const int c = (lane % CH) ^ swz<D>(row);
      __builtin_amdgcn_global_load_lds((gptr_t)(q + tok_row(n) * D + c * 8), (lptr_t)(qb + blk * 1024), 16, 0, 0);
    }
  };

  if (readout) {
    // ---- readout waves: channels [16 CT sw, +16 CT) ----
    // o_s of this lane's outputs of a tile: channels 16 (sw CT + ct) + 4 lg .. +4, token 16 sub + l16
    auto fetch_os = [&](int it, uint2 (&os)[CT][kSub]) {
      const int tok0 = tok_begin + it * kTileTok;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int sub = 0; sub < kSub; ++sub) {
          const int n = min(tok0 + sub * 16 + l16, tok_end - 1);
          os[ct][sub] = *reinterpret_cast<const uint2*>(o_s + tok_row(n) * D + (sw * CT + ct) * 16 + lg * 4);
        }
    };
    // the first tiles' loads go out before the (once per workgroup) state and weight loads
    uint2 osa[CT][kSub], osb[CT][kSub];
    issue_q(0);
    fetch_os(0, osa);
    if (ntiles > 1) issue_q(1);
    const bool bnd = anchors && (t == 0 || t == T - 1);
    const int slot = bnd ? Nc : t / C;
    const float* sf = states + ((int64_t)slot * H + h) * DD;
    const float* sr = states + (((int64_t)(Nc + 1) + slot) * H + h) * DD;
    bf16x8 s_hi[CT][KS], s_lo[CT][KS], wg0[MX ? 1 : CT][MX ? 1 : KS], wg1[MX ? 1 : CT][MX ? 1 : KS];
    i32x8 wg8[2][CT];                       // MX gate weights and their block scales
    int wgs[2][CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int j = (sw * CT + ct) * 16 + l16, i0 = ks * 32 + lg * 8;
        const f32x4* a = reinterpret_cast<const f32x4*>(sf + (int64_t)j * D + i0);
        const f32x4* b = reinterpret_cast<const f32x4*>(sr + (int64_t)j * D + i0);
        const f32x4 a0 = a[0], a1 = a[1], b0 = b[0], b1 = b[1];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float sv = e < 4 ? a0[e] + b0[e] : a1[e - 4] + b1[e - 4];
          const __bf16 hi = (__bf16)sv;
          s_hi[ct][ks][e] = hi;
          s_lo[ct][ks][e] = (__bf16)(sv - (float)hi);
        }
        if constexpr (!MX) {
          wg0[ct][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(wt + 0 * DD + (int64_t)j * D + i0));
          wg1[ct][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(wt + 1 * DD + (int64_t)j * D + i0));
        }
      }
      if constexpr (MX) {
        const int j = (sw * CT + ct) * 16 + l16;
        wfrag8(0, j, wg8[0][ct], wgs[0][ct]);
        wfrag8(1, j, wg8[1][ct], wgs[1][ct]);
      }
    }
    // Issue order per tile: the o_s loads of the next tile, then the q DMA of the tile after; the
    // wait for those o_s loads (before their registers are used) then leaves the DMA in flight.
    __builtin_amdgcn_s_waitcnt(0x0F70);                // q tiles 0 (and 1) landed
    lds_barrier();                                     // q tile 0 complete for every wave
    for (int it = 0; it <= ntiles; ++it) {
      if (it < ntiles) {
        if (it + 1 < ntiles) fetch_os(it + 1, osb);
        if (it + 2 < ntiles) issue_q(it + 2);          // its buffer held tile it-1, read in the last iteration
        const unsigned char* qb = smem + SM::Q_OFF + (it % kQBufs) * SM::PLANE;
        unsigned char* xb = smem + SM::X_OFF + (it & 1) * (MX ? 2 * SM::PLANE8 : 3 * SM::PLANE);
        float* part = reinterpret_cast<float*>(smem + SM::P_OFF) + (it & 1) * 4 * kTileTok + sw * kTileTok;
#pragma unroll
        for (int sub = 0; sub < kSub; ++sub) {
          const int r = sub * 16 + l16;
          f32x4 ol[CT], gs[CT], gl[CT];
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) ol[ct] = gs[ct] = gl[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 qf = *reinterpret_cast<const bf16x8*>(qb + frag_off(r, ks * 32 + lg * 8));
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              ol[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s_hi[ct][ks], qf, ol[ct], 0, 0, 0);
              ol[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s_lo[ct][ks], qf, ol[ct], 0, 0, 0);
              if constexpr (!MX) {
                gs[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wg0[ct][ks], qf, gs[ct], 0, 0, 0);
                gl[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wg1[ct][ks], qf, gl[ct], 0, 0, 0);
              }
            }
          }
          if constexpr (MX) {
            // q of token r as the B operand: k = 16 lg .. +15 (half A, block lg / 2) and
            // k = 64 + 16 lg .. +15 (half B, block 2 + lg / 2), each half quantised with its block
            uint32_t h[2][8];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              const u32x4 c0 = *reinterpret_cast<const u32x4*>(qb + frag_off(r, 64 * hf + 16 * lg));
              const u32x4 c1 = *reinterpret_cast<const u32x4*>(qb + frag_off(r, 64 * hf + 16 * lg + 8));
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                h[hf][i] = c0[i];
                h[hf][4 + i] = c1[i];
              }
            }
            float am[2];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              float m = 0.f;
#pragma unroll
              for (int i = 0; i < 8; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(h[hf][i])), fabsf(bf16_hi(h[hf][i]))));
              am[hf] = fmaxf(m, __shfl_xor(m, 16));          // both halves of the block
            }
            const int xa = mx_exponent(am[0]), xb = mx_exponent(am[1]);
            // lane group g supplies block g's scale: block 0 and 2 sit in group 0, block 1 in
            // group 2 (half A), block 3 in group 3 (half B)
            const int both = (xa + 127) | ((xb + 127) << 8);
            const int got = __shfl(both, l16 + 16 * ((0xC8 >> (2 * lg)) & 3));
            const int qsc = lg < 2 ? (got & 0xFF) : ((got >> 8) & 0xFF);
            i32x8 q8;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              const float sc = exp2i(-(hf ? xb : xa));
#pragma unroll
              for (int i = 0; i < 4; ++i)
                q8[4 * hf + i] = pack4_e4m3(bf16_lo(h[hf][2 * i]) * sc, bf16_hi(h[hf][2 * i]) * sc,
                                            bf16_lo(h[hf][2 * i + 1]) * sc, bf16_hi(h[hf][2 * i + 1]) * sc);
            }
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              gs[ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wg8[0][ct], q8, z, 0, 0, 0, wgs[0][ct], 0, qsc);
              gl[ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wg8[1][ct], q8, z, 0, 0, 0, wgs[1][ct], 0, qsc);
            }
          }
          // outputs: channel 16 (sw CT + ct) + 4 lg + e, token row r
          float ss = 0.f;
          float xsv[CT][4], zlv[CT][4];
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const uint32_t o01 = osa[ct][sub].x, o23 = osa[ct][sub].y;
            const float osv[4] = {bf16_lo(o01), bf16_hi(o01), bf16_lo(o23), bf16_hi(o23)};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              ss += ol[ct][e] * ol[ct][e];
              xsv[ct][e] = fast_sigmoid(gs[ct][e]) * osv[e];
              zlv[ct][e] = fast_sigmoid(gl[ct][e]) * ol[ct][e];
            }
          }
          if constexpr (MX) {
            // this wave's 32 channels are block sw of token r: maxima over the lane's 8 values and
            // the four lane groups, then E4M3 codes and the block's scale byte
            float mx = 0.f, mz = 0.f;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                mx = fmaxf(mx, fabsf(xsv[ct][e]));
                mz = fmaxf(mz, fabsf(zlv[ct][e]));
              }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            mz = fmaxf(mz, __shfl_xor(mz, 16));
            mz = fmaxf(mz, __shfl_xor(mz, 32));
            const int ex = mx_exponent(mx), ez = mx_exponent(mz);
            const float sx = exp2i(-ex), sz = exp2i(-ez);
            unsigned char* x8 = xb;                      // [2][PLANE8]: x_s, z_l
            uint8_t* scb = reinterpret_cast<uint8_t*>(smem + SM::SC_OFF) + (it & 1) * 2 * kTileTok * 4;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              const int off = off8(r, sw * CT + ct) + 4 * lg;
              *reinterpret_cast<int*>(x8 + off) =
                  pack4_e4m3(xsv[ct][0] * sx, xsv[ct][1] * sx, xsv[ct][2] * sx, xsv[ct][3] * sx);
              *reinterpret_cast<int*>(x8 + SM::PLANE8 + off) =
                  pack4_e4m3(zlv[ct][0] * sz, zlv[ct][1] * sz, zlv[ct][2] * sz, zlv[ct][3] * sz);
            }
            if (lg == 0) {
              scb[r * 4 + sw] = (uint8_t)(ex + 127);
              scb[kTileTok * 4 + r * 4 + sw] = (uint8_t)(ez + 127);
            }
          } else {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              bf16x4 xs, zh, zl;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                xs[e] = (__bf16)xsv[ct][e];
                zh[e] = (__bf16)zlv[ct][e];
                zl[e] = (__bf16)(zlv[ct][e] - (float)zh[e]);
              }
              const int ch = (sw * CT + ct) * 16 + lg * 4;
              const int off = frag_off(r, ch) + (ch & 4) * 2;
              *reinterpret_cast<bf16x4*>(xb + off) = xs;
              *reinterpret_cast<bf16x4*>(xb + SM::PLANE + off) = zh;
              *reinterpret_cast<bf16x4*>(xb + 2 * SM::PLANE + off) = zl;
            }
          }
          ss += __shfl_xor(ss, 16);
          ss += __shfl_xor(ss, 32);
          if (lg == 0) part[r] = ss;
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int sub = 0; sub < kSub; ++sub) osa[ct][sub] = osb[ct][sub];
      }
      if (it + 2 < ntiles) __builtin_amdgcn_s_waitcnt(kVmcntTile);   // q tile it+1 landed
      else __builtin_amdgcn_s_waitcnt(0x0F70);
      lds_barrier();                                   // tile it handed over; q tile it+1 complete
    }
  } else {
    // ---- projection waves: channels [16 CT sw, +16 CT) ----
    bf16x8 wp0[MX ? 1 : CT][MX ? 1 : KS], wp1[MX ? 1 : CT][MX ? 1 : KS];
    i32x8 wp8[2][CT];                       // MX projection weights and their block scales
    int wps[2][CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int j = (sw * CT + ct) * 16 + l16;
      if constexpr (MX) {
        wfrag8(2, j, wp8[0][ct], wps[0][ct]);
        wfrag8(3, j, wp8[1][ct], wps[1][ct]);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int i0 = ks * 32 + lg * 8;
          wp0[ct][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(wt + 2 * DD + (int64_t)j * D + i0));
          wp1[ct][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(wt + 3 * DD + (int64_t)j * D + i0));
        }
      }
    }
    lds_barrier();
    for (int it = 0; it <= ntiles; ++it) {
      if (it >= 1) {
        const int pt = it - 1;                         // the tile handed over at the last barrier
        const unsigned char* xb = smem + SM::X_OFF + (pt & 1) * (MX ? 2 * SM::PLANE8 : 3 * SM::PLANE);
        const uint8_t* scb = reinterpret_cast<const uint8_t*>(smem + SM::SC_OFF) + (pt & 1) * 2 * kTileTok * 4;
        const float* part = reinterpret_cast<const float*>(smem + SM::P_OFF) + (pt & 1) * 4 * kTileTok;
        const int tok0 = tok_begin + pt * kTileTok;
#pragma unroll
        for (int sub = 0; sub < kSub; ++sub) {
          const int r = sub * 16 + l16;
          f32x4 as[CT], al[CT];
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) as[ct] = al[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
          if constexpr (MX) {
            // B operands: token r, channels 16 lg .. +15 and 64 + 16 lg .. +15; scale of block lg
            i32x8 x8[2];
#pragma unroll
            for (int pl = 0; pl < 2; ++pl) {
              const unsigned char* pb = xb + pl * SM::PLANE8;
              const u32x4 lo = *reinterpret_cast<const u32x4*>(pb + off8(r, lg));
              const u32x4 hi = *reinterpret_cast<const u32x4*>(pb + off8(r, 4 + lg));
              x8[pl] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
            const int sx = scb[r * 4 + lg], sz = scb[kTileTok * 4 + r * 4 + lg];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              as[ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wp8[0][ct], x8[0], as[ct], 0, 0, 0, wps[0][ct], 0, sx);
              al[ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wp8[1][ct], x8[1], al[ct], 0, 0, 0, wps[1][ct], 0, sz);
            }
          } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              const int off = frag_off(r, ks * 32 + lg * 8);
              const bf16x8 xs = *reinterpret_cast<const bf16x8*>(xb + off);
              const bf16x8 zh = *reinterpret_cast<const bf16x8*>(xb + SM::PLANE + off);
              const bf16x8 zl = *reinterpret_cast<const bf16x8*>(xb + 2 * SM::PLANE + off);
#pragma unroll
              for (int ct = 0; ct < CT; ++ct) {
                as[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wp0[ct][ks], xs, as[ct], 0, 0, 0);
                al[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wp1[ct][ks], zh, al[ct], 0, 0, 0);
                al[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wp1[ct][ks], zl, al[ct], 0, 0, 0);
              }
            }
          }
          const float ss = part[r] + part[kTileTok + r] + part[2 * kTileTok + r] + part[3 * kTileTok + r];
          const float rinv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + 1e-6f);
          const int n = tok0 + r;
          if (n < tok_end) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              bf16x4 ov;
#pragma unroll
              for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(as[ct][e] + rinv * al[ct][e]);
              *reinterpret_cast<bf16x4*>(out + tok_row(n) * D + (sw * CT + ct) * 16 + lg * 4) = ov;
            }
          }
        }
      }
      lds_barrier();
    }
  }
}

template <int D, bool MX>
void launch_t(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  const int wg_per_frame = (s.N + kTokPerWG - 1) / kTokPerWG;
  const size_t smem = EpiSmem<D, MX>::TOTAL;
  (void)hipFuncSetAttribute((const void*)epilogue_mfma_kernel<D, MX>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)smem);
  hipLaunchKernelGGL((epilogue_mfma_kernel<D, MX>), dim3(s.T * wg_per_frame, s.H), dim3(512), smem, st,
                     (const bf16_t*)in.q, (const bf16_t*)b.os, b.states, b.wt, b.wt8, b.wsc8, (bf16_t*)in.out, s.T,
                     s.N, s.H, s.C, s.Nc, s.anchors, wg_per_frame);
}

}  // namespace

hipError_t launch_prep_weights(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  dim3 grid((s.d * s.d + 255) / 256, 4);
  prep_weights_kernel<<<grid, 256, 0, st>>>((const bf16_t*)in.gate_w, (const bf16_t*)in.proj_w, b.wt, s.d);
  return hipGetLastError();
}

hipError_t launch_prep_weights_mx(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  if (s.d != 128 || !b.wt8 || !b.wsc8) return hipErrorInvalidValue;
  prep_weights_mx_kernel<<<dim3(1, 4), 512, 0, st>>>((const bf16_t*)in.gate_w, (const bf16_t*)in.proj_w, b.wt8, b.wsc8,
                                                     s.d);
  return hipGetLastError();
}

hipError_t launch_epilogue_mfma(const Shape& s, const Inputs& in, const Buffers& b, bool mx, hipStream_t st) {
  if (mx) {
    if (s.d != 128 || !b.wt8 || !b.wsc8) return hipErrorInvalidValue;
    launch_t<128, true>(s, in, b, st);
  } else if (s.d == 128) {
    launch_t<128, false>(s, in, b, st);
  } else {
    launch_t<64, false>(s, in, b, st);
  }
  return hipGetLastError();
}

}  // namespace vdn
