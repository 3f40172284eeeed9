// Softmax-branch backward on CDNA4 matrix cores (bf16 operands, fp32 accumulate), d in {64, 128}.
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Local Softmax and
// Long-Range Linear Memory": o = P V with P = softmax(tau q K^T) over each query frame's key set.
// Its transpose, with P rebuilt from the forward's saved base-2 normaliser lse (P = 2^(c q.k - lse),
// c = tau log2 e) and Dq = rowsum(do * o):
//   dS = P (dP - Dq) tau,  dP = do V^T,   dq = dS K,   dK = dS^T q,   dV = P^T do.
// Two kernels, both on v_mfma_f32_16x16x32_bf16 with operand tiles staged in XOR-swizzled LDS by
// global_load_lds (two stages):
//   * softmax_dkv_mfma: one workgroup = 128 keys of one key slot (the text or one frame) and head,
//     16 keys per wave; it walks every 64-query tile of the query frames that see the slot.  Keys
//     stay in registers (K, V as B operands); per query tile it forms S = Q K^T and dP = dO V^T
//     with the query rows permuted so that a lane's values of two 16-row tiles are 8 consecutive
//     queries, which makes P and dS directly the B operands of dV^T += dO^T P and dK^T += Q^T dS
//     (dO^T, Q^T tiles from transposed copies).
//   * softmax_dq_mfma: one workgroup = 256 queries of one frame and head, 32 per wave, walking the
//     frame's key ranges like the forward; S^T = K Q^T and dP^T = V dO^T with the key rows
//     permuted the same way, then dQ^T += K^T dS^T.
#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

constexpr int kWaves = 8;
// VDN_DKV_WIDE 1: the dK/dV kernel with 4 waves x 32 keys (softmax_dkv_wide_kernel); 0 (default):
// 8 waves x 16 keys, two waves per SIMD (2.5 % faster at 768p once both stage the tile's
// normalisers in LDS and fold the offsets into the accumulators)
#ifndef VDN_DKV_WIDE
#define VDN_DKV_WIDE 0
#endif
constexpr int kVmcntZero = 0x0F70;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
// swizzles: rows read 8 lanes at a time as {8a + b : a in {0,1}, b in 0..3} + const (row-major
// tiles) or 8 consecutive rows (transposed tiles)
__device__ __forceinline__ int r_swz(int row) { return (row & 3) | ((row >> 1) & 4); }
__device__ __forceinline__ int t_swz(int row) { return row & 7; }
// row of a 16-row tile u (of a 32-row k-step pair) that lane l16 addresses: 8 (l16/4) + 4 (u%2) + l16%4
__device__ __forceinline__ int perm_row(int u, int l16) { return 32 * (u >> 1) + 8 * (l16 >> 2) + 4 * (u & 1) + (l16 & 3); }

// ---------------------------------------------------------------------------------------------
// Packing for the backward: transposed copies [H][D][ld] of token-major [rows][H][D] arrays, and
// head-major row copies [H][ld][D].  Pad columns/rows are zeroed once at allocation.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_t_kernel(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst,
                                                     int64_t rows, int H, int D, int64_t ld, int64_t col0) {
  __shared__ bf16_t tile[64][64 + 2];
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int h = blockIdx.y, d0 = blockIdx.z * 64;
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int r = e / 64, c = e % 64;
    tile[r][c] = (r0 + r < rows) ? src[((r0 + r) * H + h) * D + d0 + c] : (bf16_t)0;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int c = e / 64, r = e % 64;
    if (r0 + r < rows) dst[((int64_t)h * D + d0 + c) * ld + col0 + r0 + r] = tile[r][c];
  }
}

__global__ __launch_bounds__(256) void pack_rows_kernel(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst,
                                                        int64_t rows, int H, int D, int64_t ld, int64_t row0) {
  const int64_t r = (int64_t)blockIdx.x;
  const int h = blockIdx.y;
  if (r >= rows) return;
  for (int c = threadIdx.x; c < D; c += 256) dst[((int64_t)h * ld + row0 + r) * D + c] = src[(r * H + h) * D + c];
}

// ---------------------------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------------------------
struct DkvParams {
  const bf16_t *q, *dout, *qt, *dot;    // q, do_s [TN][H][D]; their transposes [H][D][Lq]
  const bf16_t *k, *v, *text_kv;        // [TN][H][D]; [2][n_text][H][D]
  const float *lse, *dsum;              // [TN][H]
  const int *qranges, *nqranges;        // per key slot: query-frame ranges
  const int2* blocks;                   // per workgroup: (key slot, first key of the slot)
  float *dk, *dv, *dtext;               // fp32 outputs (accumulated)
  int T, N, H, n_text;
  int64_t Lq;
  float tau, c;
};

template <int D>
struct DkvSmem {
  static constexpr int ROW = 64 * D * 2;          // one 64-query row-major tile (Q or dO)
  static constexpr int STAGE = 4 * ROW + 512;     // Q, dO, Q^T, dO^T, then lse[64], dsum[64]
};

template <int D>
__global__ __launch_bounds__(kWaves * 64, 1) void softmax_dkv_mfma_kernel(DkvParams P) {
  using SM = DkvSmem<D>;
  constexpr int KS = D / 32, DT = D / 16, KCH = D / 8;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int2 blk = P.blocks[blockIdx.x];
  const int slot = blk.x, h = blockIdx.y;
  const int N = P.N, H = P.H;
  const int U = slot == 0 ? P.n_text : N;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int key = blk.y + 16 * wave + l16;                     // this lane's key within the slot
  const bool kvalid = key < U;
  const int kc = kvalid ? key : U - 1;
  const bf16_t* kbase = slot == 0 ? P.text_kv + ((int64_t)kc * H + h) * D
                                  : P.k + (((int64_t)(slot - 1) * N + kc) * H + h) * D;
  const bf16_t* vbase = slot == 0 ? P.text_kv + (((int64_t)P.n_text + kc) * H + h) * D
                                  : P.v + (((int64_t)(slot - 1) * N + kc) * H + h) * D;
  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kf[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(kbase + ks * 32 + g * 8));
    vf[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(vbase + ks * 32 + g * 8));
#pragma unroll
    for (int e = 0; e < 8; ++e) kf[ks][e] = (__bf16)((float)kf[ks][e] * P.c);   // scores in log2 units
  }
  f32x4 dvt[DT], dkt[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dvt[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dkt[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // query tiles: every 64-row tile of every frame in the slot's ranges
  const int* qr = P.qranges + slot * 2 * kMaxRanges;
  const int nr = uniform(P.nqranges[slot]);
  const int tpf = (N + 63) / 64;
  int nfr = 0;
  for (int r = 0; r < nr; ++r) nfr += qr[2 * r + 1] - qr[2 * r];
  const int ntiles = uniform(nfr * tpf);
  auto tile_at = [&](int it, int& t, int& q0) {
    int fi = it / tpf;
    q0 = (it % tpf) * 64;
    t = 0;
    for (int r = 0; r < nr; ++r) {
      const int len = qr[2 * r + 1] - qr[2 * r];
      if (fi < len) { t = qr[2 * r] + fi; break; }
      fi -= len;
    }
  };
  // DMA: Q and dO tiles [64][D] (row-major, rows clamped to the frame), Q^T and dO^T tiles [D][64]
  constexpr int R_ROWS_PER_KB = 1024 / (D * 2);
  constexpr int R_INSTR = SM::ROW / 1024 / kWaves;           // per wave, per row-major tile
  constexpr int T_INSTR = SM::ROW / 1024 / kWaves;           // per wave, per transposed tile
  auto issue_tile = [&](int t, int q0, int stage) {
    unsigned char* base = smem + stage * SM::STAGE;
#pragma unroll
    for (int i = 0; i < R_INSTR; ++i) {
      const int blkid = i * kWaves + wave;
      const int row = blkid * R_ROWS_PER_KB + lane / KCH;
      const int c = (lane % KCH) ^ r_swz(row);
      const int qrow = min(q0 + row, N - 1);
      const int64_t off = (((int64_t)t * N + qrow) * H + h) * D + c * 8;
      __builtin_amdgcn_global_load_lds((gptr_t)(P.q + off), (lptr_t)(base + blkid * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gptr_t)(P.dout + off), (lptr_t)(base + SM::ROW + blkid * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < T_INSTR; ++i) {
      const int blkid = i * kWaves + wave;
      const int row = blkid * 8 + lane / 8;                    // d row
      const int c = (lane % 8) ^ t_swz(row);
      const int64_t off = ((int64_t)h * D + row) * P.Lq + (int64_t)t * N + q0 + c * 8;
      __builtin_amdgcn_global_load_lds((gptr_t)(P.qt + off), (lptr_t)(base + 2 * SM::ROW + blkid * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gptr_t)(P.dot + off), (lptr_t)(base + 3 * SM::ROW + blkid * 1024), 16, 0, 0);
    }
    if (wave < 2) {                              // the tile's normalisers (wave 0) and D values (wave 1)
      const int64_t rr = ((int64_t)t * N + min(q0 + lane, N - 1)) * H + h;
      __builtin_amdgcn_global_load_lds((gptr_t)((wave == 0 ? P.lse : P.dsum) + rr),
                                       (lptr_t)(base + 4 * SM::ROW + wave * 256), 4, 0, 0);
    }
  };

  [[maybe_unused]] const float c = P.c;
  const float tau = P.tau;
  if (ntiles > 0) {
    int t, q0;
    tile_at(0, t, q0);
    issue_tile(t, q0, 0);
  }
  for (int it = 0; it < ntiles; ++it) {
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
    __syncthreads();
    if (it + 1 < ntiles) {
      int t1, q1;
      tile_at(it + 1, t1, q1);
      issue_tile(t1, q1, (it + 1) & 1);
    }
    int t, q0;
    tile_at(it, t, q0);
    const unsigned char* qs = smem + (it & 1) * SM::STAGE;
    const unsigned char* os = qs + SM::ROW;
    const unsigned char* qts = qs + 2 * SM::ROW;
    const unsigned char* ots = qs + 3 * SM::ROW;
    const float* lse_s = reinterpret_cast<const float*>(qs + 4 * SM::ROW);
    const float* dsum_s = lse_s + 64;
    bf16x8 pj[2], sj[2];                                     // P and dS of the two 32-query k-steps
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // accumulators start at -lse and -D of the lane's four query rows
      f32x4 s, dp;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qi = 32 * (u >> 1) + 8 * g + 4 * (u & 1) + i;
        s[i] = -lse_s[qi];
        dp[i] = -dsum_s[qi];
      }
      const int row = perm_row(u, l16);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ch = ks * 4 + g;
        const int boff = row * (D * 2) + ((ch ^ r_swz(row)) * 16);
        const bf16x8 qa = as_bf16x8(*reinterpret_cast<const u32x4*>(qs + boff));
        const bf16x8 oa = as_bf16x8(*reinterpret_cast<const u32x4*>(os + boff));
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kf[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa, vf[ks], dp, 0, 0, 0);
      }
      // lane holds rows 4 g + i of tile u = queries 32 (u/2) + 8 g + 4 (u%2) + i, key l16
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qi = 32 * (u >> 1) + 8 * g + 4 * (u & 1) + i;
        float p = 0.f, ds = 0.f;
        if (q0 + qi < N) {
          p = __builtin_amdgcn_exp2f(s[i]);
          ds = p * dp[i];                          // tau applied to dK at the end
        }
        pj[u >> 1][4 * (u & 1) + i] = (__bf16)p;
        sj[u >> 1][4 * (u & 1) + i] = (__bf16)ds;
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int trow = dt * 16 + l16;
        const int ch = j * 4 + g;
        const int boff = trow * 128 + ((ch ^ t_swz(trow)) * 16);
        const bf16x8 ot = as_bf16x8(*reinterpret_cast<const u32x4*>(ots + boff));
        const bf16x8 qtv = as_bf16x8(*reinterpret_cast<const u32x4*>(qts + boff));
        dvt[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ot, pj[j], dvt[dt], 0, 0, 0);
        dkt[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qtv, sj[j], dkt[dt], 0, 0, 0);
      }
  }
  // lane holds dV^T / dK^T rows d = 16 dt + 4 g + i of key l16
  if (kvalid) {
    float* dkp = slot == 0 ? P.dtext + ((int64_t)key * H + h) * D : P.dk + (((int64_t)(slot - 1) * N + key) * H + h) * D;
    float* dvp = slot == 0 ? P.dtext + (((int64_t)P.n_text + key) * H + h) * D
                           : P.dv + (((int64_t)(slot - 1) * N + key) * H + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x4* a = reinterpret_cast<f32x4*>(dkp + dt * 16 + g * 4);
      f32x4* b = reinterpret_cast<f32x4*>(dvp + dt * 16 + g * 4);
      *a = *a + dkt[dt] * tau;
      *b = *b + dvt[dt];
    }
  }
}

// Wide variant: 4 waves x 32 keys (two 16-key tiles per wave), one wave per SIMD.  Every Q, dO,
// Q^T and dO^T fragment a wave reads from LDS feeds two MFMAs (one per key tile), which halves
// the LDS reads per MFMA of the 16-key layout, and the tile's normalisers and D values come
// through LDS with the tile instead of per-element global loads.
constexpr int kDkvWaves = 4;
// VDN_DKV_FOLD 1: keys enter as bf16(c k) and the score and dP accumulators start at -lse and -D
#ifndef VDN_DKV_FOLD
#define VDN_DKV_FOLD 1
#endif
#ifndef VDN_DKV_MINBLOCKS
#define VDN_DKV_MINBLOCKS 1
#endif

template <int D>
struct DkvWideSmem {
  static constexpr int ROW = 64 * D * 2;
  static constexpr int STAGE = 4 * ROW + 512;     // Q, dO, Q^T, dO^T, then lse[64], dsum[64]
};

template <int D>
__global__ __launch_bounds__(kDkvWaves * 64, VDN_DKV_MINBLOCKS) void softmax_dkv_wide_kernel(DkvParams P) {
  using SM = DkvWideSmem<D>;
  constexpr int KS = D / 32, DT = D / 16, KCH = D / 8;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int2 blk = P.blocks[blockIdx.x];
  const int slot = blk.x, h = blockIdx.y;
  const int N = P.N, H = P.H;
  const int U = slot == 0 ? P.n_text : N;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  bf16x8 kf[2][KS], vf[2][KS];
  int keyk[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = blk.y + 32 * wave + 16 * kt + l16;        // this lane's key of tile kt
    keyk[kt] = key;
    const int kc = key < U ? key : U - 1;
    const bf16_t* kbase = slot == 0 ? P.text_kv + ((int64_t)kc * H + h) * D
                                    : P.k + (((int64_t)(slot - 1) * N + kc) * H + h) * D;
    const bf16_t* vbase = slot == 0 ? P.text_kv + (((int64_t)P.n_text + kc) * H + h) * D
                                    : P.v + (((int64_t)(slot - 1) * N + kc) * H + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[kt][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(kbase + ks * 32 + g * 8));
      vf[kt][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(vbase + ks * 32 + g * 8));
#if VDN_DKV_FOLD
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[kt][ks][e] = (__bf16)((float)kf[kt][ks][e] * P.c);
#endif
    }
  }
  f32x4 dvt[2][DT], dkt[2][DT];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      dvt[kt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dkt[kt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  const int* qr = P.qranges + slot * 2 * kMaxRanges;
  const int nr = uniform(P.nqranges[slot]);
  const int tpf = (N + 63) / 64;
  int nfr = 0;
  for (int r = 0; r < nr; ++r) nfr += qr[2 * r + 1] - qr[2 * r];
  const int ntiles = uniform(nfr * tpf);
  constexpr int R_ROWS_PER_KB = 1024 / (D * 2);
  constexpr int R_INSTR = SM::ROW / 1024 / kDkvWaves;
  constexpr int T_INSTR = SM::ROW / 1024 / kDkvWaves;

  [[maybe_unused]] const float c = P.c;
  const float tau = P.tau;
  int t_next = 0, q_next = 0;
#define VDN_DKV_TILE_AT(it_, t_, q0_)                                  \
  {                                                                    \
    int fi_ = (it_) / tpf;                                             \
    q0_ = ((it_) % tpf) * 64;                                          \
    t_ = 0;                                                            \
    for (int r_ = 0; r_ < nr; ++r_) {                                  \
      const int len_ = qr[2 * r_ + 1] - qr[2 * r_];                    \
      if (fi_ < len_) { t_ = qr[2 * r_] + fi_; break; }                \
      fi_ -= len_;                                                     \
    }                                                                  \
  }
#define VDN_DKV_ISSUE(t_, q0_, stage_)                                                                      \
  {                                                                                                         \
    unsigned char* base_ = smem + (stage_) * SM::STAGE;                                                     \
    _Pragma("unroll") for (int i_ = 0; i_ < R_INSTR; ++i_) {                                                \
      const int blkid_ = i_ * kDkvWaves + wave;                                                             \
      const int row_ = blkid_ * R_ROWS_PER_KB + lane / KCH;                                                 \
      const int c_ = (lane % KCH) ^ r_swz(row_);                                                            \
      const int qrow_ = min((q0_) + row_, N - 1);                                                           \
      const int64_t off_ = (((int64_t)(t_) * N + qrow_) * H + h) * D + c_ * 8;                              \
      __builtin_amdgcn_global_load_lds((gptr_t)(P.q + off_), (lptr_t)(base_ + blkid_ * 1024), 16, 0, 0);   \
      __builtin_amdgcn_global_load_lds((gptr_t)(P.dout + off_), (lptr_t)(base_ + SM::ROW + blkid_ * 1024), \
                                       16, 0, 0);                                                           \
    }                                                                                                       \
    _Pragma("unroll") for (int i_ = 0; i_ < T_INSTR; ++i_) {                                                \
      const int blkid_ = i_ * kDkvWaves + wave;                                                             \
      const int row_ = blkid_ * 8 + lane / 8;                                                               \
      const int c_ = (lane % 8) ^ t_swz(row_);                                                              \
      const int64_t off_ = ((int64_t)h * D + row_) * P.Lq + (int64_t)(t_) * N + (q0_) + c_ * 8;           \
      __builtin_amdgcn_global_load_lds((gptr_t)(P.qt + off_), (lptr_t)(base_ + 2 * SM::ROW + blkid_ * 1024), \
                                       16, 0, 0);                                                           \
      __builtin_amdgcn_global_load_lds((gptr_t)(P.dot + off_), (lptr_t)(base_ + 3 * SM::ROW + blkid_ * 1024), \
                                       16, 0, 0);                                                           \
    }                                                                                                       \
    if (wave < 2) {                                                                                         \
      const int64_t rr_ = ((int64_t)(t_) * N + min((q0_) + lane, N - 1)) * H + h;                           \
      __builtin_amdgcn_global_load_lds((gptr_t)((wave == 0 ? P.lse : P.dsum) + rr_),                        \
                                       (lptr_t)(base_ + 4 * SM::ROW + wave * 256), 4, 0, 0);                \
    }                                                                                                       \
  }
  if (ntiles > 0) {
    VDN_DKV_TILE_AT(0, t_next, q_next)
    VDN_DKV_ISSUE(t_next, q_next, 0)
  }
  for (int it = 0; it < ntiles; ++it) {
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
    __syncthreads();
    [[maybe_unused]] int t;
    int q0;
    VDN_DKV_TILE_AT(it, t, q0)
    if (it + 1 < ntiles) {
      VDN_DKV_TILE_AT(it + 1, t_next, q_next)
      VDN_DKV_ISSUE(t_next, q_next, (it + 1) & 1)
    }
    const unsigned char* qs = smem + (it & 1) * SM::STAGE;
    const unsigned char* os = qs + SM::ROW;
    const unsigned char* qts = qs + 2 * SM::ROW;
    const unsigned char* ots = qs + 3 * SM::ROW;
    const float* lse_s = reinterpret_cast<const float*>(qs + 4 * SM::ROW);
    const float* dsum_s = lse_s + 64;
    bf16x8 pj[2][2], sj[2][2];                               // [key tile][32-query k-step]
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f32x4 sc[2], dp[2];
#if VDN_DKV_FOLD
      // accumulators start at -lse and -D of the lane's four query rows
      f32x4 l0, d0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qi = 32 * (u >> 1) + 8 * g + 4 * (u & 1) + i;
        l0[i] = -lse_s[qi];
        d0[i] = -dsum_s[qi];
      }
#endif
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#if VDN_DKV_FOLD
        sc[kt] = l0;
        dp[kt] = d0;
#else
        sc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#endif
      }
      const int row = perm_row(u, l16);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ch = ks * 4 + g;
        const int boff = row * (D * 2) + ((ch ^ r_swz(row)) * 16);
        const bf16x8 qa = as_bf16x8(*reinterpret_cast<const u32x4*>(qs + boff));
        const bf16x8 oa = as_bf16x8(*reinterpret_cast<const u32x4*>(os + boff));
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          sc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kf[kt][ks], sc[kt], 0, 0, 0);
          dp[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa, vf[kt][ks], dp[kt], 0, 0, 0);
        }
      }
      // lane holds rows 4 g + i of tile u = queries 32 (u/2) + 8 g + 4 (u%2) + i, key l16 of tile kt
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qi = 32 * (u >> 1) + 8 * g + 4 * (u & 1) + i;
        const bool ok = q0 + qi < N;
#if !VDN_DKV_FOLD
        const float l = lse_s[qi], dd = dsum_s[qi];
#endif
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#if VDN_DKV_FOLD
          const float p = ok ? __builtin_amdgcn_exp2f(sc[kt][i]) : 0.f;
          const float ds = p * dp[kt][i];                       // tau applied to dK at the end
#else
          const float p = ok ? __builtin_amdgcn_exp2f(fmaf(sc[kt][i], c, -l)) : 0.f;
          const float ds = p * (dp[kt][i] - dd) * tau;
#endif
          pj[kt][u >> 1][4 * (u & 1) + i] = (__bf16)p;
          sj[kt][u >> 1][4 * (u & 1) + i] = (__bf16)ds;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int trow = dt * 16 + l16;
        const int ch = j * 4 + g;
        const int boff = trow * 128 + ((ch ^ t_swz(trow)) * 16);
        const bf16x8 ot = as_bf16x8(*reinterpret_cast<const u32x4*>(ots + boff));
        const bf16x8 qtv = as_bf16x8(*reinterpret_cast<const u32x4*>(qts + boff));
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          dvt[kt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ot, pj[kt][j], dvt[kt][dt], 0, 0, 0);
          dkt[kt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qtv, sj[kt][j], dkt[kt][dt], 0, 0, 0);
        }
      }
  }
#undef VDN_DKV_TILE_AT
#undef VDN_DKV_ISSUE
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = keyk[kt];
    if (key >= U) continue;
    float* dkp = slot == 0 ? P.dtext + ((int64_t)key * H + h) * D : P.dk + (((int64_t)(slot - 1) * N + key) * H + h) * D;
    float* dvp = slot == 0 ? P.dtext + (((int64_t)P.n_text + key) * H + h) * D
                           : P.dv + (((int64_t)(slot - 1) * N + key) * H + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x4* a = reinterpret_cast<f32x4*>(dkp + dt * 16 + g * 4);
      f32x4* b = reinterpret_cast<f32x4*>(dvp + dt * 16 + g * 4);
#if VDN_DKV_FOLD
      *a = *a + dkt[kt][dt] * tau;
#else
      *a = *a + dkt[kt][dt];
#endif
      *b = *b + dvt[kt][dt];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------------------------
struct DqParams {
  const bf16_t *q, *dout;               // q, do_s [TN][H][D]
  const bf16_t *kp, *vp, *kt;           // [H][Ls][D], [H][Ls][D], [H][D][Ls]
  const float *lse, *dsum;
  const int *ranges, *nranges;
  float* dq;                            // fp32 [TN][H][D] (accumulated)
  int T, N, H, QT;
  int64_t Ls;
  float tau, c;
};

template <int D>
struct DqSmem {
  static constexpr int TILE = 64 * D * 2;
  static constexpr int STAGE = 3 * TILE;          // K, V (key-major), K^T
};

// VDN_DQ_WAVES, VDN_DQ_QT: waves per workgroup and 16-query column tiles per wave (8 x 2: two waves
// per SIMD; 4 x 4: one wave per SIMD, each K, V and K^T fragment read feeding four MFMAs)
#ifndef VDN_DQ_WAVES
#define VDN_DQ_WAVES 8
#endif
// VDN_DQ_FOLD 1: queries enter as bf16(c q) and the score and dP accumulators start at -lse and -D,
// so dS = exp2(S') dP' needs no multiply-adds (tau is applied once to dQ)
#ifndef VDN_DQ_FOLD
#define VDN_DQ_FOLD 1
#endif
#ifndef VDN_DQ_QT
#define VDN_DQ_QT 2
#endif
constexpr int kDqWaves = VDN_DQ_WAVES;
constexpr int kDqQT = VDN_DQ_QT;                  // 16-query column tiles per wave
constexpr int kDqBQ = kDqWaves * 16 * kDqQT;      // queries per workgroup

template <int D>
__global__ __launch_bounds__(kDqWaves * 64, 1) void softmax_dq_mfma_kernel(DqParams P) {
  using SM = DqSmem<D>;
  constexpr int KS = D / 32, DT = D / 16, KCH = D / 8;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int w = blockIdx.x;
  const int qt = w % P.QT, t = (w / P.QT) % P.T, h = w / (P.QT * P.T);
  const int N = P.N, H = P.H;
  const int64_t Ls = P.Ls;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int n_base = qt * kDqBQ + wave * 16 * kDqQT;
  bf16x8 qf[kDqQT][KS], of[kDqQT][KS];
  float lse[kDqQT], dsm[kDqQT];
  bool qv[kDqQT];
#pragma unroll
  for (int j = 0; j < kDqQT; ++j) {
    const int n = n_base + 16 * j + l16;
    qv[j] = n < N;
    const int64_t rr = ((int64_t)t * N + min(n, N - 1)) * H + h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[j][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(P.q + rr * D + ks * 32 + g * 8));
      of[j][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(P.dout + rr * D + ks * 32 + g * 8));
#if VDN_DQ_FOLD
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[j][ks][e] = (__bf16)((float)qf[j][ks][e] * P.c);
#endif
    }
    lse[j] = P.lse[rr];
    dsm[j] = P.dsum[rr];
  }
  f32x4 dqt[DT][kDqQT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int j = 0; j < kDqQT; ++j) dqt[dt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // key tiles of the frame's ranges: full tiles first, then each range's partial tile
  const int* rg = P.ranges + t * 2 * kMaxRanges;
  const int nr = uniform(P.nranges[t]);
  int rs[kMaxRanges], rl[kMaxRanges];
  int nfull = 0, npart = 0;
#pragma unroll
  for (int r = 0; r < kMaxRanges; ++r) {
    rs[r] = r < nr ? uniform(rg[2 * r]) : 0;
    rl[r] = r < nr ? uniform(rg[2 * r + 1]) - rs[r] : 0;
    nfull += rl[r] / 64;
    npart += (rl[r] % 64) != 0;
  }
  const int ntiles = nfull + npart;
  auto tile_at = [&](int it, int& key0, int& valid) {
    if (it < nfull) {
      valid = 64;
#pragma unroll
      for (int r = 0; r < kMaxRanges; ++r) {
        const int nf = rl[r] / 64;
        if (it < nf) { key0 = rs[r] + it * 64; return; }
        it -= nf;
      }
    }
    it -= nfull;
#pragma unroll
    for (int r = 0; r < kMaxRanges; ++r) {
      if (rl[r] % 64) {
        if (it == 0) { key0 = rs[r] + (rl[r] / 64) * 64; valid = rl[r] % 64; return; }
        --it;
      }
    }
    key0 = 0;
    valid = 0;
  };
  const unsigned char* kh = reinterpret_cast<const unsigned char*>(P.kp + (int64_t)h * Ls * D);
  const unsigned char* vh = reinterpret_cast<const unsigned char*>(P.vp + (int64_t)h * Ls * D);
  const unsigned char* th = reinterpret_cast<const unsigned char*>(P.kt + (int64_t)h * D * Ls);
  constexpr int R_ROWS_PER_KB = 1024 / (D * 2);
  constexpr int R_INSTR = SM::TILE / 1024 / kDqWaves;
  auto issue_tile = [&](int key0, int stage) {
    unsigned char* base = smem + stage * SM::STAGE;
#pragma unroll
    for (int i = 0; i < R_INSTR; ++i) {
      const int blkid = i * kDqWaves + wave;
      const int row = blkid * R_ROWS_PER_KB + lane / KCH;
      const int c = (lane % KCH) ^ r_swz(row);
      const int64_t off = ((int64_t)(key0 + row) * D + c * 8) * 2;
      __builtin_amdgcn_global_load_lds((gptr_t)(kh + off), (lptr_t)(base + blkid * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gptr_t)(vh + off), (lptr_t)(base + SM::TILE + blkid * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < R_INSTR; ++i) {
      const int blkid = i * kDqWaves + wave;
      const int row = blkid * 8 + lane / 8;                    // d row
      const int c = (lane % 8) ^ t_swz(row);
      const int64_t off = ((int64_t)row * Ls + key0 + c * 8) * 2;
      __builtin_amdgcn_global_load_lds((gptr_t)(th + off), (lptr_t)(base + 2 * SM::TILE + blkid * 1024), 16, 0, 0);
    }
  };

  [[maybe_unused]] const float c = P.c;
  const float tau = P.tau;
  if (ntiles > 0) {
    int key0, valid;
    tile_at(0, key0, valid);
    issue_tile(key0, 0);
  }
  for (int it = 0; it < ntiles; ++it) {
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
    __syncthreads();
    if (it + 1 < ntiles) {
      int k1, v1;
      tile_at(it + 1, k1, v1);
      issue_tile(k1, (it + 1) & 1);
    }
    int key0, valid;
    tile_at(it, key0, valid);
    const unsigned char* ks_ = smem + (it & 1) * SM::STAGE;
    const unsigned char* vs_ = ks_ + SM::TILE;
    const unsigned char* ts_ = ks_ + 2 * SM::TILE;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      bf16x8 dsf[kDqQT];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        // S^T and dP^T of 16-key row tile u: key rows 8 (l16/4) + 4 u + l16%4 of the half
        const int row = half * 32 + 8 * (l16 >> 2) + 4 * u + (l16 & 3);
        f32x4 s[kDqQT], dp[kDqQT];
#pragma unroll
        for (int j = 0; j < kDqQT; ++j) {
#if VDN_DQ_FOLD
          s[j] = f32x4{-lse[j], -lse[j], -lse[j], -lse[j]};
          dp[j] = f32x4{-dsm[j], -dsm[j], -dsm[j], -dsm[j]};
#else
          s[j] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#endif
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int ch = ks * 4 + g;
          const int boff = row * (D * 2) + ((ch ^ r_swz(row)) * 16);
          const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(ks_ + boff));
          const bf16x8 va = as_bf16x8(*reinterpret_cast<const u32x4*>(vs_ + boff));
#pragma unroll
          for (int j = 0; j < kDqQT; ++j) {
            s[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[j][ks], s[j], 0, 0, 0);
            dp[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, of[j][ks], dp[j], 0, 0, 0);
          }
        }
        // lane holds keys half*32 + 8 g + 4 u + i of query l16 (column tile j)
#pragma unroll
        for (int j = 0; j < kDqQT; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kl = half * 32 + 8 * g + 4 * u + i;
            float ds = 0.f;
            if (kl < valid && qv[j]) {
#if VDN_DQ_FOLD
              ds = __builtin_amdgcn_exp2f(s[j][i]) * dp[j][i];     // tau applied to dQ at the end
#else
              const float p = exp2f(s[j][i] * c - lse[j]);
              ds = p * (dp[j][i] - dsm[j]) * tau;
#endif
            }
            dsf[j][4 * u + i] = (__bf16)ds;
          }
      }
      // dQ^T += K^T dS^T: K^T rows d = 16 dt + l16, keys half*32 + 8 g .. +8
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int trow = dt * 16 + l16;
        const int ch = half * 4 + g;
        const bf16x8 kt = as_bf16x8(*reinterpret_cast<const u32x4*>(ts_ + trow * 128 + ((ch ^ t_swz(trow)) * 16)));
#pragma unroll
        for (int j = 0; j < kDqQT; ++j) dqt[dt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt, dsf[j], dqt[dt][j], 0, 0, 0);
      }
    }
  }
  // lane holds dQ^T rows d = 16 dt + 4 g + i of query l16 of tile j
#pragma unroll
  for (int j = 0; j < kDqQT; ++j) {
    if (!qv[j]) continue;
    float* dqp = P.dq + (((int64_t)t * N + n_base + 16 * j + l16) * H + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x4* a = reinterpret_cast<f32x4*>(dqp + dt * 16 + g * 4);
#if VDN_DQ_FOLD
      *a = *a + dqt[dt][j] * tau;
#else
      *a = *a + dqt[dt][j];
#endif
    }
  }
}

template <int D>
hipError_t run_t(const Shape& s, const Inputs& in, const Buffers& b, const BwdBuffers& w, const BwdOutputs& o,
                 hipStream_t st) {
  const int T = s.T, N = s.N, H = s.H;
  const int64_t TN = (int64_t)T * N;
  const float tau = 1.0f / sqrtf((float)D);
  // packing (do_s arrives in bf16 from the merge): Q^T, dO_s^T [H][D][Lq]; K^T [H][D][Ls]; V
  // key-major [H][Ls][D]
  pack_t_kernel<<<dim3((int)((TN + 63) / 64), H, D / 64), 256, 0, st>>>((const bf16_t*)in.q, w.qt, TN, H, D, w.Lq, 0);
  pack_t_kernel<<<dim3((int)((TN + 63) / 64), H, D / 64), 256, 0, st>>>(w.dos16, w.dot, TN, H, D, w.Lq, 0);
  if (s.n_text > 0) {
    pack_t_kernel<<<dim3((s.n_text + 63) / 64, H, D / 64), 256, 0, st>>>((const bf16_t*)in.text_kv, w.kt, s.n_text, H,
                                                                         D, s.Ls, 0);
    pack_rows_kernel<<<dim3(s.n_text, H), 256, 0, st>>>((const bf16_t*)in.text_kv + (int64_t)s.n_text * H * D, w.vp,
                                                        s.n_text, H, D, s.Ls, 0);
  }
  pack_t_kernel<<<dim3((int)((TN + 63) / 64), H, D / 64), 256, 0, st>>>((const bf16_t*)in.k, w.kt, TN, H, D, s.Ls,
                                                                       s.ctx_pad);
  pack_rows_kernel<<<dim3((unsigned)TN, H), 256, 0, st>>>((const bf16_t*)in.v, w.vp, TN, H, D, s.Ls, s.ctx_pad);
  // dK, dV
  {
    DkvParams p{};
    p.q = (const bf16_t*)in.q;
    p.dout = w.dos16;
    p.qt = w.qt;
    p.dot = w.dot;
    p.k = (const bf16_t*)in.k;
    p.v = (const bf16_t*)in.v;
    p.text_kv = (const bf16_t*)in.text_kv;
    p.lse = w.lse;
    p.dsum = w.dsum;
    p.qranges = w.qranges;
    p.nqranges = w.nqranges;
    p.blocks = w.kblocks;
    p.dk = o.dk;
    p.dv = o.dv;
    p.dtext = o.dtext_kv;
    p.T = T;
    p.N = N;
    p.H = H;
    p.n_text = s.n_text;
    p.Lq = w.Lq;
    p.tau = tau;
    p.c = tau * 1.4426950408889634f;
#if VDN_DKV_WIDE
    const size_t sm = 2 * DkvWideSmem<D>::STAGE;
    (void)hipFuncSetAttribute((const void*)softmax_dkv_wide_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)sm);
    hipLaunchKernelGGL(softmax_dkv_wide_kernel<D>, dim3(w.nkblocks, H), dim3(kDkvWaves * 64), sm, st, p);
#else
    const size_t sm = 2 * DkvSmem<D>::STAGE;
    (void)hipFuncSetAttribute((const void*)softmax_dkv_mfma_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)sm);
    hipLaunchKernelGGL(softmax_dkv_mfma_kernel<D>, dim3(w.nkblocks, H), dim3(kWaves * 64), sm, st, p);
#endif
  }
  // dQ
  {
    DqParams p{};
    p.q = (const bf16_t*)in.q;
    p.dout = w.dos16;
    p.kp = b.kp;
    p.vp = w.vp;
    p.kt = w.kt;
    p.lse = w.lse;
    p.dsum = w.dsum;
    p.ranges = b.ranges;
    p.nranges = b.nranges;
    p.dq = o.dq;
    p.T = T;
    p.N = N;
    p.H = H;
    p.QT = (N + kDqBQ - 1) / kDqBQ;
    p.Ls = s.Ls;
    p.tau = tau;
    p.c = tau * 1.4426950408889634f;
    const size_t sm = 2 * DqSmem<D>::STAGE;
    (void)hipFuncSetAttribute((const void*)softmax_dq_mfma_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)sm);
    hipLaunchKernelGGL(softmax_dq_mfma_kernel<D>, dim3(p.QT * T * H), dim3(kDqWaves * 64), sm, st, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_softmax_backward_mfma(const Shape& s, const Inputs& in, const Buffers& b, const BwdBuffers& w,
                                        const BwdOutputs& o, hipStream_t st) {
  return s.d == 128 ? run_t<128>(s, in, b, w, o, st) : run_t<64>(s, in, b, w, o, st);
}

}  // namespace vdn
