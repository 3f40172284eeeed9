// Softmax-branch backward on CDNA4 matrix cores (bf16 operands, fp32 accumulate), d in {64, 128}.
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Local Softmax and
// Long-Range Linear Memory": o = P V with P = softmax(tau q K^T) over each query frame's key set.
// Its transpose, with P rebuilt from the forward's saved base-2 normaliser lse (P = 2^(c q.k - lse),
// c = tau log2 e) and Dq = rowsum(do * o):
//   dS = P (dP - Dq) tau,  dP = do V^T,   dq = dS K,   dK = dS^T q,   dV = P^T do.
// Two kernels, both on v_mfma_f32_16x16x32_bf16 with operand tiles staged in XOR-swizzled LDS by
// global_load_lds (two stages):
//   * softmax_dkv_mfma: one workgroup = 128 keys of one key slot (the global text and audio keys,
//     or one frame) and head, 16 keys per wave; it walks every 64-query tile of the query frames
//     that see the slot, then the tiles of the text and audio query rows when the backward includes
//     them (they see every key: "Video DeltaNet speeds MiniMax H3 video generation 14.5x",
//     summary).  Keys
//     stay in registers (K, V as B operands, both negated: the accumulators start at +lse and +D
//     read straight from LDS and hold lse - S and D - dP, whose exponential takes the sign as a
//     source modifier); per query tile it forms S = Q K^T and dP = dO V^T with the query rows
//     permuted so that a lane's values of two 16-row tiles are 8 consecutive queries, which makes
//     P and -dS directly the B operands of dV^T += dO^T P and dK^T -= Q^T dS (dO^T, Q^T tiles from
//     transposed copies).  Query rows past the end of their frame read an infinite lse, so their
//     P and dS are exactly zero without a select.
//   * softmax_dq_mfma: one workgroup = 256 queries of one frame (or of the text and audio query
//     rows, which walk every key and are dispatched first) and head, 32 per wave, walking the
//     frame's key ranges like the forward; S^T = K Q^T and dP^T = V dO^T with the key rows
//     permuted the same way, then dQ^T += K^T dS^T.  Queries past the end of the rows take an
//     infinite lse (zero P and dS); only a range's last, partial key tile masks keys (a
//     compile-time variant of the tile body, so full tiles carry no selects).
#include <type_traits>

#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

// the normaliser DMA'd for query rows past the end of their frame: exp2(-inf) = 0 exactly
__device__ float kInfRow = __builtin_inff();

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

constexpr int kWaves = 8;
constexpr int kVmcntZero = 0x0F70;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
// LDS swizzles (XOR on the 16-byte chunk index of a row).  gfx950 serves a 16-byte LDS read 16
// lanes per pass over 64 banks of 4 bytes, so the 16 rows one lane group reads must fall on 16
// distinct 16-byte slots of the 256-byte bank period.  Row-major tiles: a group reads rows
// {8a + b : a in 0..3, b in 0..3} + const of one chunk (rows of 2 D bytes); transposed tiles: 16
// consecutive rows of 128 bytes.
template <int D>
__device__ __forceinline__ int r_swz(int row) {
  return D == 128 ? (row & 3) | ((row >> 1) & 12) : ((row >> 1) & 1) | ((row >> 2) & 6);
}
__device__ __forceinline__ int t_swz(int row) { return (row >> 1) & 7; }
// row of a 16-row tile u (of a 32-row k-step pair) that lane l16 addresses: 8 (l16/4) + 4 (u%2) + l16%4
__device__ __forceinline__ int perm_row(int u, int l16) { return 32 * (u >> 1) + 8 * (l16 >> 2) + 4 * (u & 1) + (l16 & 3); }

// ---------------------------------------------------------------------------------------------
// Packing for the backward: transposed copies [H][D][ld] of token-major [rows][H][D] arrays, and
// head-major row copies [H][ld][D].  Pad columns/rows are zeroed once at allocation.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_t_kernel(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst,
                                                     int64_t rows, int H, int D, int64_t ld, int64_t col0) {
  __shared__ __attribute__((aligned(16))) bf16_t tile[64][64 + 8];
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int h = blockIdx.y, d0 = blockIdx.z * 64;
  if (r0 + 64 <= rows && ld % 8 == 0 && col0 % 8 == 0) {
    // a full tile with 16-byte aligned destination rows: 16-byte loads and stores
    for (int e = threadIdx.x; e < 64 * 8; e += 256) {
      const int r = e / 8, c8 = e % 8;
      *reinterpret_cast<u32x4*>(&tile[r][c8 * 8]) =
          *reinterpret_cast<const u32x4*>(src + ((r0 + r) * H + h) * D + d0 + c8 * 8);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 8; e += 256) {
      const int c = e / 8, r8 = e % 8;                 // output row d0 + c, input rows 8 r8 .. + 7
      bf16_t o[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = tile[8 * r8 + k][c];
      *reinterpret_cast<u32x4*>(dst + ((int64_t)h * D + d0 + c) * ld + col0 + r0 + 8 * r8) =
          *reinterpret_cast<const u32x4*>(o);
    }
    return;
  }
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

// one 16-byte chunk per thread: chunk e of src row (r, h) goes to dst row h ld + row0 + r
__global__ __launch_bounds__(256) void pack_rows_kernel(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst,
                                                        int64_t rows, int H, int D, int64_t ld, int64_t row0) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cpr = D / 8;
  if (e >= rows * H * cpr) return;
  const int c = (int)(e % cpr);
  const int64_t rh = e / cpr;
  const int h = (int)(rh % H);
  const int64_t r = rh / H;
  *reinterpret_cast<u32x4*>(dst + ((int64_t)h * ld + row0 + r) * D + c * 8) =
      *reinterpret_cast<const u32x4*>(src + (r * H + h) * D + c * 8);
}

// ---------------------------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------------------------
struct DkvParams {
  const bf16_t *q, *dout, *qt, *dot;    // q, do_s [TN][H][D]; their transposes [H][D][Lq] (context rows
                                        // from column TN)
  const bf16_t *cq, *cdout;             // context query rows and their do [n_cq][H][D] (n_cq > 0)
  const bf16_t *k, *v, *text_kv;        // [TN][H][D]; [2][n_glob][H][D]
  const float *lse, *dsum;              // [TN + n_cq][H]
  const int *qranges, *nqranges;        // per key slot: query-frame ranges
  const int4* work;                     // per workgroup: (key slot, first key of the slot, head, 0);
                                        // a negative slot: no work (padding of the XCD placement)
  float *dk, *dv, *dtext;               // fp32 outputs (accumulated)
  int T, N, H, n_glob, n_cq;            // n_glob global (text, audio) keys in slot 0; n_cq context rows
  int64_t Lq;
  float tau, c;
};

template <int D>
struct DkvSmem {
  static constexpr int ROW = 64 * D * 2;          // one 64-query row-major tile (Q or dO)
  static constexpr int STAGE = 4 * ROW + 512;     // Q, dO, Q^T, dO^T, then lse[64], dsum[64]
};

// KT 16-key tiles per wave (VDN_DKV_KT): with KT = 2 every Q, dO, Q^T and dO^T fragment a wave
// reads from LDS feeds two MFMAs, halving the LDS reads per MFMA of KT = 1; P and dS are formed
// and consumed one 32-query k-step at a time so that the accumulators of both key tiles, their K
// and V fragments and the k-step's operands fit the 256 registers of two waves per SIMD.
#ifndef VDN_DKV_KT
#define VDN_DKV_KT 2
#endif
constexpr int kDkvKT = VDN_DKV_KT;
constexpr int kDkvKeys = kWaves * 16 * kDkvKT;   // keys per workgroup

// CTX = false: the query tiles of the video frames that see the slot.  CTX = true: only the context
// query rows' tiles (they see every slot), a second pass that adds to the first one's dK, dV (a
// compile-time switch, so neither pass carries the other's selects)
template <int D, bool CTX>
__global__ __launch_bounds__(kWaves * 64, 1) void softmax_dkv_mfma_kernel(DkvParams P) {
  using SM = DkvSmem<D>;
  constexpr int KS = D / 32, DT = D / 16, KCH = D / 8, KT = kDkvKT;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int N = P.N, H = P.H;
  const int4 blk = P.work[blockIdx.x];
  if (blk.x < 0) return;
  const int slot = blk.x, h = blk.z;
  const int U = slot == 0 ? P.n_glob : N;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  bf16x8 kf[KT][KS], vf[KT][KS];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int key = blk.y + 16 * (KT * wave + kt) + l16;       // this lane's key of tile kt
    const int kc = key < U ? key : U - 1;
    const bf16_t* kbase = slot == 0 ? P.text_kv + ((int64_t)kc * H + h) * D
                                    : P.k + (((int64_t)(slot - 1) * N + kc) * H + h) * D;
    const bf16_t* vbase = slot == 0 ? P.text_kv + (((int64_t)P.n_glob + kc) * H + h) * D
                                    : P.v + (((int64_t)(slot - 1) * N + kc) * H + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[kt][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(kbase + ks * 32 + g * 8));
      // -V: sign bits flipped once here (the opaque copy keeps the compiler from redoing the flip
      // inside the tile loop)
      u32x4 vr = *reinterpret_cast<const u32x4*>(vbase + ks * 32 + g * 8) ^ 0x80008000u;
      asm volatile("" : "+v"(vr));
      vf[kt][ks] = as_bf16x8(vr);
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[kt][ks][e] = (__bf16)((float)kf[kt][ks][e] * -P.c);   // -scores in log2 units
    }
  }
  f32x4 dvt[KT][DT], dkt[KT][DT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      dvt[kt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dkt[kt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // query tiles: every 64-row tile of every frame in the slot's ranges, then the context rows
  // (pseudo-frame T: they see every key)
  // (the frame ranges are read once into scalar registers: read from the table inside the tile
  // walk, each tile's range lookup waited for a global load right before its tile copy)
  const int* qr = P.qranges + slot * 2 * kMaxRanges;
  const int nr = uniform(P.nqranges[slot]);
  const int tpf = (N + 63) / 64;
  int qs[kMaxRanges], ql[kMaxRanges];
  int nfr = 0;
#pragma unroll
  for (int r = 0; r < kMaxRanges; ++r) {
    qs[r] = r < nr ? uniform(qr[2 * r]) : 0;
    ql[r] = r < nr ? uniform(qr[2 * r + 1]) - qs[r] : 0;
    nfr += ql[r];
  }
  const int nvt = CTX ? 0 : uniform(nfr * tpf);
  const int ntiles = CTX ? (P.n_cq + 63) / 64 : nvt;
  auto tile_at = [&](int it, int& t, int& q0) {
    if (CTX && it >= nvt) {
      t = P.T;
      q0 = (it - nvt) * 64;
      return;
    }
    int fi = it / tpf;
    q0 = (it % tpf) * 64;
    t = 0;
#pragma unroll
    for (int r = 0; r < kMaxRanges; ++r) {
      if (fi < ql[r]) { t = qs[r] + fi; return; }
      fi -= ql[r];
    }
  };
  // DMA: Q and dO tiles [64][D] (row-major, rows clamped to the frame), Q^T and dO^T tiles [D][64]
  constexpr int R_ROWS_PER_KB = 1024 / (D * 2);
  constexpr int R_INSTR = SM::ROW / 1024 / kWaves;           // per wave, per row-major tile
  constexpr int T_INSTR = SM::ROW / 1024 / kWaves;           // per wave, per transposed tile
  // The normaliser and D-value arrays as values held in scalar registers: selected per wave in
  // the tile copy below, a select between the two parameter fields became a load from the
  // parameter block through a vector address, and its wait also completed the tile copies just
  // issued (so every tile's copy latency was exposed).
  const float* lse_p = P.lse;
  const float* dsum_p = P.dsum;
  asm volatile("" : "+s"(lse_p), "+s"(dsum_p));
  auto issue_tile = [&](int t, int q0, int stage) {
    unsigned char* base = smem + stage * SM::STAGE;
    // an opaque copy of the lane index: the per-lane DMA offsets are recomputed at each issue
    // instead of being hoisted out of the tile loop, where they cost registers the MFMA loop needs
    // (fewer spills; 2 % faster per backward call at 768p, same results)
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const bool cx = CTX && t == P.T;                           // the context rows
    const int rows = cx ? P.n_cq : N;
    const bf16_t* qsrc = cx ? P.cq : P.q + (int64_t)t * N * H * D;
    const bf16_t* osrc = cx ? P.cdout : P.dout + (int64_t)t * N * H * D;
#pragma unroll
    for (int i = 0; i < R_INSTR; ++i) {
      const int blkid = i * kWaves + wave;
      const int row = blkid * R_ROWS_PER_KB + lane / KCH;
      const int c = (lane % KCH) ^ r_swz<D>(row);
      const int qrow = min(q0 + row, rows - 1);
      const int64_t off = ((int64_t)qrow * H + h) * D + c * 8;
      __builtin_amdgcn_global_load_lds((gptr_t)(qsrc + off), (lptr_t)(base + blkid * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gptr_t)(osrc + off), (lptr_t)(base + SM::ROW + blkid * 1024), 16, 0, 0);
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
      const int64_t rr = ((int64_t)t * N + min(q0 + lane, rows - 1)) * H + h;
      const float* src = wave == 1 ? dsum_p + rr : q0 + lane < rows ? lse_p + rr : &kInfRow;
      __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)(base + 4 * SM::ROW + wave * 256), 4, 0, 0);
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
#pragma unroll
    for (int j = 0; j < 2; ++j) {                            // 32-query k-steps
      bf16x8 pj[KT], sj[KT];                                 // P and dS of this k-step, per key tile
#pragma unroll
      for (int u2 = 0; u2 < 2; ++u2) {
        const int u = 2 * j + u2;
        // accumulators start at lse and D of the lane's four query rows: they hold lse - S, D - dP
        f32x4 s[KT], dp[KT];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int qi = 32 * j + 8 * g + 4 * u2 + i;
          const float l = lse_s[qi], dd = dsum_s[qi];
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            s[kt][i] = l;
            dp[kt][i] = dd;
          }
        }
        const int row = perm_row(u, l16);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int ch = ks * 4 + g;
          const int boff = row * (D * 2) + ((ch ^ r_swz<D>(row)) * 16);
          const bf16x8 qa = as_bf16x8(*reinterpret_cast<const u32x4*>(qs + boff));
          const bf16x8 oa = as_bf16x8(*reinterpret_cast<const u32x4*>(os + boff));
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kf[kt][ks], s[kt], 0, 0, 0);
            dp[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa, vf[kt][ks], dp[kt], 0, 0, 0);
          }
        }
        // lane holds rows 4 g + i of tile u = queries 32 j + 8 g + 4 u2 + i, key l16 of tile kt
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            const float p = __builtin_amdgcn_exp2f(-s[kt][i]);
            const float ds = p * dp[kt][i];          // -dS / tau: -tau applied to dK at the end
            pj[kt][4 * u2 + i] = (__bf16)p;
            sj[kt][4 * u2 + i] = (__bf16)ds;
          }
        }
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int trow = dt * 16 + l16;
        const int ch = j * 4 + g;
        const int boff = trow * 128 + ((ch ^ t_swz(trow)) * 16);
        const bf16x8 ot = as_bf16x8(*reinterpret_cast<const u32x4*>(ots + boff));
        const bf16x8 qtv = as_bf16x8(*reinterpret_cast<const u32x4*>(qts + boff));
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          dvt[kt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ot, pj[kt], dvt[kt][dt], 0, 0, 0);
          dkt[kt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qtv, sj[kt], dkt[kt][dt], 0, 0, 0);
        }
      }
    }
  }
  // lane holds dV^T / dK^T rows d = 16 dt + 4 g + i of key l16 of tile kt
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int key = blk.y + 16 * (KT * wave + kt) + l16;
    if (key >= U) continue;
    float* dkp = slot == 0 ? P.dtext + ((int64_t)key * H + h) * D : P.dk + (((int64_t)(slot - 1) * N + key) * H + h) * D;
    float* dvp = slot == 0 ? P.dtext + (((int64_t)P.n_glob + key) * H + h) * D
                           : P.dv + (((int64_t)(slot - 1) * N + key) * H + h) * D;
    // every load first, then every store (interleaved, each load waited for the stores before it)
    f32x4 ka[DT], va[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      ka[dt] = *reinterpret_cast<const f32x4*>(dkp + dt * 16 + g * 4);
      va[dt] = *reinterpret_cast<const f32x4*>(dvp + dt * 16 + g * 4);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      *reinterpret_cast<f32x4*>(dkp + dt * 16 + g * 4) = ka[dt] - dkt[kt][dt] * tau;
      *reinterpret_cast<f32x4*>(dvp + dt * 16 + g * 4) = va[dt] + dvt[kt][dt];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------------------------
struct DqParams {
  const bf16_t *q, *dout;               // q, do_s [TN][H][D]
  const bf16_t *cq, *cdout;             // context query rows and their do [n_cq][H][D] (n_cq > 0)
  const bf16_t *kp, *vp, *kt;           // [H][Ls][D], [H][Ls][D], [H][D][Ls]
  const float *lse, *dsum;              // [TN + n_cq][H]
  const int *ranges, *nranges;          // key ranges of each query frame; row T: the context rows
  const int2* work;                     // per workgroup of the video rows: (query frame, query tile +
                                        // QT head); a negative frame: no work
  float *dq, *dcq;                      // fp32 [TN][H][D], [n_cq][H][D] (accumulated)
  int T, N, H, QT, n_cq, QTc;           // QTc query tiles of the context rows (0 without them)
  int ctx_split;                        // workgroups sharing one context query tile's key tiles
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

// CTX = false: one workgroup per (head, frame, query tile) of the video rows.  CTX = true: the
// context rows (pseudo-frame T, every key), each query tile's key tiles split over ctx_split
// workgroups that add their parts atomically; a launch of their own, before the video rows'.
template <int D, bool CTX>
__global__ __launch_bounds__(kDqWaves * 64, 1) void softmax_dq_mfma_kernel(DqParams P) {
  using SM = DqSmem<D>;
  constexpr int KS = D / 32, DT = D / 16, KCH = D / 8;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int w = blockIdx.x;
  int qt, t, h, part = 0;
  if constexpr (CTX) {
    qt = w % P.QTc;
    part = (w / P.QTc) % P.ctx_split;
    h = w / (P.QTc * P.ctx_split);
    t = P.T;
  } else {
    const int2 e = P.work[w];
    if (e.x < 0) return;
    t = e.x;
    qt = e.y % P.QT;
    h = e.y / P.QT;
  }
  constexpr bool cx = CTX;
  const int N = P.N, H = P.H;
  const int rows = cx ? P.n_cq : N;
  const bf16_t* qsrc = cx ? P.cq : P.q + (int64_t)t * N * H * D;
  const bf16_t* osrc = cx ? P.cdout : P.dout + (int64_t)t * N * H * D;
  const int64_t Ls = P.Ls;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int n_base = qt * kDqBQ + wave * 16 * kDqQT;
  bf16x8 qf[kDqQT][KS], of[kDqQT][KS];
  float lse[kDqQT], dsm[kDqQT];
  bool qv[kDqQT];
#pragma unroll
  for (int j = 0; j < kDqQT; ++j) {
    const int n = n_base + 16 * j + l16;
    qv[j] = n < rows;
    const int nc = min(n, rows - 1);
    const int64_t rr = ((int64_t)t * N + nc) * H + h;      // lse, D: context rows after the video rows
    const int64_t ro = ((int64_t)nc * H + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[j][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qsrc + ro + ks * 32 + g * 8));
      of[j][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(osrc + ro + ks * 32 + g * 8));
#if VDN_DQ_FOLD
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[j][ks][e] = (__bf16)((float)qf[j][ks][e] * P.c);
#endif
    }
    lse[j] = qv[j] ? P.lse[rr] : __builtin_inff();
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
  const int ntiles_all = nfull + npart;
  const int it0 = CTX ? ntiles_all * part / P.ctx_split : 0;
  const int it1 = CTX ? ntiles_all * (part + 1) / P.ctx_split : ntiles_all;
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
      const int c = (lane % KCH) ^ r_swz<D>(row);
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
  if (it1 > it0) {
    int key0, valid;
    tile_at(it0, key0, valid);
    issue_tile(key0, 0);
  }
  // the full key tiles come first in the walk, then each range's partial tile: two loops, the
  // second with the key mask compiled in
  auto step = [&](int it, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;       // keys valid..63 of the tile lie outside
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
    __syncthreads();
    if (it + 1 < it1) {
      int k1, v1;
      tile_at(it + 1, k1, v1);
      issue_tile(k1, (it + 1 - it0) & 1);
    }
    int key0, valid;
    tile_at(it, key0, valid);
    const unsigned char* ks_ = smem + ((it - it0) & 1) * SM::STAGE;
    const unsigned char* vs_ = ks_ + SM::TILE;
    const unsigned char* ts_ = ks_ + 2 * SM::TILE;
    {
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
            const int boff = row * (D * 2) + ((ch ^ r_swz<D>(row)) * 16);
            const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(ks_ + boff));
            const bf16x8 va = as_bf16x8(*reinterpret_cast<const u32x4*>(vs_ + boff));
#pragma unroll
            for (int j = 0; j < kDqQT; ++j) {
              s[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[j][ks], s[j], 0, 0, 0);
              dp[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, of[j][ks], dp[j], 0, 0, 0);
            }
          }
          // lane holds keys half*32 + 8 g + 4 u + i of query l16 (column tile j); a query past
          // the rows has lse = inf, so its P and dS are zero
#pragma unroll
          for (int j = 0; j < kDqQT; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#if VDN_DQ_FOLD
              float ds = __builtin_amdgcn_exp2f(s[j][i]) * dp[j][i];     // tau applied to dQ at the end
#else
              const float p = exp2f(s[j][i] * c - lse[j]);
              float ds = p * (dp[j][i] - dsm[j]) * tau;
#endif
              if constexpr (MASKED) {
                if (half * 32 + 8 * g + 4 * u + i >= valid) ds = 0.f;
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
  };
  const int split = min(max(nfull, it0), it1);
  for (int it = it0; it < split; ++it) step(it, std::false_type{});
  for (int it = split; it < it1; ++it) step(it, std::true_type{});
  // lane holds dQ^T rows d = 16 dt + 4 g + i of query l16 of tile j
#pragma unroll
  for (int j = 0; j < kDqQT; ++j) {
    if (!qv[j]) continue;
    if constexpr (CTX) {                        // parts of a context query tile: atomic adds
      float* dqp = P.dcq + (((int64_t)n_base + 16 * j + l16) * H + h) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          atomicAdd(dqp + dt * 16 + g * 4 + i, VDN_DQ_FOLD ? dqt[dt][j][i] * tau : dqt[dt][j][i]);
      continue;
    }
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
  const int n_cq = w.dctx_out ? s.n_ctx : 0;       // context query rows: columns TN.. of the transposes
  if (n_cq > 0) {
    pack_t_kernel<<<dim3((n_cq + 63) / 64, H, D / 64), 256, 0, st>>>((const bf16_t*)in.ctx_q, w.qt, n_cq, H, D, w.Lq,
                                                                     TN);
    pack_t_kernel<<<dim3((n_cq + 63) / 64, H, D / 64), 256, 0, st>>>((const bf16_t*)w.dctx_out, w.dot, n_cq, H, D,
                                                                     w.Lq, TN);
  }
  if (s.n_ctx > 0) {                               // the global (text, audio) keys
    pack_t_kernel<<<dim3((s.n_ctx + 63) / 64, H, D / 64), 256, 0, st>>>((const bf16_t*)in.text_kv, w.kt, s.n_ctx, H,
                                                                        D, s.Ls, 0);
    pack_rows_kernel<<<(unsigned)(((int64_t)s.n_ctx * H * (D / 8) + 255) / 256), 256, 0, st>>>(
        (const bf16_t*)in.text_kv + (int64_t)s.n_ctx * H * D, w.vp,
                                                       s.n_ctx, H, D, s.Ls, 0);
  }
  pack_t_kernel<<<dim3((int)((TN + 63) / 64), H, D / 64), 256, 0, st>>>((const bf16_t*)in.k, w.kt, TN, H, D, s.Ls,
                                                                       s.ctx_pad);
  pack_rows_kernel<<<(unsigned)((TN * H * (D / 8) + 255) / 256), 256, 0, st>>>((const bf16_t*)in.v, w.vp, TN, H, D, s.Ls,
                                                                               s.ctx_pad);
  // dK, dV
  {
    DkvParams p{};
    p.q = (const bf16_t*)in.q;
    p.dout = w.dos16;
    p.qt = w.qt;
    p.dot = w.dot;
    p.cq = (const bf16_t*)in.ctx_q;
    p.cdout = (const bf16_t*)w.dctx_out;
    p.k = (const bf16_t*)in.k;
    p.v = (const bf16_t*)in.v;
    p.text_kv = (const bf16_t*)in.text_kv;
    p.lse = w.lse;
    p.dsum = w.dsum;
    p.qranges = w.qranges;
    p.nqranges = w.nqranges;
    p.work = w.kwork;
    p.dk = o.dk;
    p.dv = o.dv;
    p.dtext = o.dtext_kv;
    p.T = T;
    p.N = N;
    p.H = H;
    p.n_glob = s.n_ctx;
    p.n_cq = n_cq;
    p.Lq = w.Lq;
    p.tau = tau;
    p.c = tau * 1.4426950408889634f;
    const size_t sm = 2 * DkvSmem<D>::STAGE;
    (void)hipFuncSetAttribute((const void*)softmax_dkv_mfma_kernel<D, false>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
    hipLaunchKernelGGL((softmax_dkv_mfma_kernel<D, false>), dim3(w.nkwork), dim3(kWaves * 64), sm, st, p);
    if (n_cq > 0) {                              // then the context rows' part, added on the same stream
      (void)hipFuncSetAttribute((const void*)softmax_dkv_mfma_kernel<D, true>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
      hipLaunchKernelGGL((softmax_dkv_mfma_kernel<D, true>), dim3(w.nkwork), dim3(kWaves * 64), sm, st, p);
    }
  }
  // dQ
  {
    DqParams p{};
    p.q = (const bf16_t*)in.q;
    p.dout = w.dos16;
    p.cq = (const bf16_t*)in.ctx_q;
    p.cdout = (const bf16_t*)w.dctx_out;
    p.kp = b.kp;
    p.vp = w.vp;
    p.kt = w.kt;
    p.lse = w.lse;
    p.dsum = w.dsum;
    p.ranges = b.ranges;
    p.nranges = b.nranges;
    p.work = w.qwork;
    p.dq = o.dq;
    p.dcq = o.dctx_q;
    p.T = T;
    p.N = N;
    p.H = H;
    p.QT = (N + kDqBQ - 1) / kDqBQ;
    p.n_cq = n_cq;
    p.QTc = (n_cq + kDqBQ - 1) / kDqBQ;
    // split each context query tile's key walk so that their own launch fills the GPU (two
    // workgroups per compute unit), each part at least an eighth of a frame's key walk
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                hipSuccess || cus <= 0)
      cus = 256;
    const int64_t ctx_tiles = ((int64_t)s.n_ctx + TN + 63) / 64, frame_tiles = (int64_t)(3 * s.C + 2) * N / 64 + 1;
    const int64_t fill = (2 * (int64_t)cus + (int64_t)p.QTc * H - 1) / std::max<int64_t>(1, (int64_t)p.QTc * H);
    p.ctx_split = n_cq > 0 ? (int)std::max<int64_t>(1, std::min<int64_t>({64, fill, ctx_tiles / frame_tiles * 8})) : 1;
    p.Ls = s.Ls;
    p.tau = tau;
    p.c = tau * 1.4426950408889634f;
    const size_t sm = 2 * DqSmem<D>::STAGE;
    if (n_cq > 0) {                              // the context rows first: their walks are the longest
      (void)hipFuncSetAttribute((const void*)softmax_dq_mfma_kernel<D, true>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
      hipLaunchKernelGGL((softmax_dq_mfma_kernel<D, true>), dim3(p.QTc * p.ctx_split * H), dim3(kDqWaves * 64), sm,
                         st, p);
    }
    (void)hipFuncSetAttribute((const void*)softmax_dq_mfma_kernel<D, false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)sm);
    hipLaunchKernelGGL((softmax_dq_mfma_kernel<D, false>), dim3(w.nqwork), dim3(kDqWaves * 64), sm, st, p);
  }
  return hipGetLastError();
}

}  // namespace

int softmax_dkv_block_keys() { return kDkvKeys; }
int softmax_dq_block_queries() { return kDqBQ; }

hipError_t launch_softmax_backward_mfma(const Shape& s, const Inputs& in, const Buffers& b, const BwdBuffers& w,
                                        const BwdOutputs& o, hipStream_t st) {
  return s.d == 128 ? run_t<128>(s, in, b, w, o, st) : run_t<64>(s, in, b, w, o, st);
}

}  // namespace vdn
