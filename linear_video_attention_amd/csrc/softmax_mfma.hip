// Block-sparse window softmax of the VDN layer on CDNA4 matrix cores (bf16 in, fp32 accumulate).
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Local Softmax and
// Long-Range Linear Memory": a video query in chunk c attends, with one softmax, to the global
// (text, audio) keys, the keys of chunks c-1, c, c+1 and the two boundary anchor frames (boundary
// query frames attend to every frame).  "Video DeltaNet speeds MiniMax H3 video generation 14.5x"
// (summary): the text and audio query rows attend to every key.  The key set of a row group is at
// most four contiguous ranges of the packed key space (built on the host).
//
// Work decomposition
//   * one workgroup = 384 queries of one frame and one head; 8 waves x 48 queries (three 16-query
//     column tiles), two waves per SIMD.  Every K or V^T fragment a wave reads from LDS feeds three
//     v_mfma_f32_16x16x32_bf16 (one per query tile), so a flop costs 2/3 of the LDS bytes of a
//     32-query wave on 32 x 32 tiles (measured 7 % faster than that layout, whose LDS reads ran
//     level with its MFMAs) while the registers (O^T 96, Q 48, S^T 24 per 32-key half) still fit
//     two waves per SIMD, whose interleaving hides each other's exponentials and LDS latency;
//   * key tiles of 64 keys are loaded straight from global memory into LDS (global_load_lds,
//     two stages by default: the next tile in flight; K as [key][d], V transposed as [d][key], both
//     XOR-swizzled so that every group of sixteen lanes of a 16-byte fragment read hits distinct
//     banks) and processed as two 32-key halves;
//   * S^T = K Q^T with keys as rows: the K fragment rows of 16-key tile t are the keys
//     8 (r / 4) + 4 t + (r % 4) of the half, so that a lane's four scores of tile 0 and four of
//     tile 1 are 8 consecutive keys -- exactly the B operand of O^T += V^T P^T, which is thus
//     taken straight from the score registers;
//   * exponent reference: softmax is invariant to the offset subtracted from the scores, and
//     |q.k| <= |q| max|k| bounds every score of the query, so p = 2^(s c - |q| kmax c) never
//     exceeds 1 and needs no running maximum or accumulator rescale.  Workgroups holding a row
//     whose bound |q| kmax c exceeds 4 log2 units (the limit of the query prescale below; 48 without
//     it, against underflow) flag themselves and a second launch of the same kernel with the
//     classic online maximum and unscaled queries redoes just those;
//   * workgroup order: context query rows (every key) first, then the boundary frames, then the
//     interior frames remapped so that consecutive query tiles -- which share their key window --
//     land on the same XCD (workgroups are dispatched round-robin over the 8 XCDs).
#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// Build parameters (defaults measured best at 768p; the alternatives are kept for measurement):
//   VDN_SOFTMAX_WAVES   waves per workgroup (8; 4 gives two 192-query workgroups per CU, ~4 % slower)
//   VDN_SOFTMAX_STAGES  LDS stages of the tile pipeline (2; 3 and 4 keep more tiles in flight,
//                       1-2 % slower since the key tiles mostly hit in L2 / Infinity Cache)
//   VDN_SOFTMAX_SCHED   1: order each half as K reads, score MFMAs | V reads, exponentials, P.V
//                       MFMAs (about 3 % faster than the compiler's own interleaving)
//   VDN_SOFTMAX_BK      keys per LDS tile (64; 128 halves the barriers but is 3 % slower)
//   VDN_SOFTMAX_DOT2SUM 1: the normaliser from the bf16-rounded weights by v_dot2c_f32_bf16 instead
//                       of fp32 adds (4 % slower: the sums wait for the conversions)
//   VDN_SOFTMAX_MMASUM  1: the normaliser on the matrix cores, one more MFMA per query tile and
//                       half with an all-ones A operand (sums the bf16-rounded weights); removes
//                       27 of the ~70 vector instructions of a half but is 2 % slower at 768p
//                       (6.80-6.82 against 6.64-6.71 ms): the matrix cores are the busier unit
//   VDN_SOFTMAX_QT, VDN_SOFTMAX_WG_PER_CU: query tiles per wave and the occupancy hint (3 and
//                       8 / waves; 4 waves x 4 or 5 tiles at one wave per SIMD, 404 / 492 registers,
//                       measured 27-33 % slower: the lone wave cannot hide its own exponentials)
//   VDN_SOFTMAX_PRESCALE 1: the first launch takes the queries as bf16(c q) (c = log2(e)/sqrt(d)) and
//                       starts each score accumulator at -mref, so a weight is exp2 of the
//                       accumulator with no multiply-add; the extra rounding of c q moves a score by
//                       at most 2^-9 |c q.k| <= 2^-9 mref, so rows whose bound mref exceeds 4 (log2
//                       units) are left to the second launch, which keeps the unscaled arithmetic
#ifndef VDN_SOFTMAX_WAVES
#define VDN_SOFTMAX_WAVES 8
#endif
#ifndef VDN_SOFTMAX_STAGES
#define VDN_SOFTMAX_STAGES 2
#endif
#ifndef VDN_SOFTMAX_SCHED
#define VDN_SOFTMAX_SCHED 1
#endif
#ifndef VDN_SOFTMAX_BK
#define VDN_SOFTMAX_BK 64
#endif
#ifndef VDN_SOFTMAX_DOT2SUM
#define VDN_SOFTMAX_DOT2SUM 0
#endif
#ifndef VDN_SOFTMAX_PRESCALE
#define VDN_SOFTMAX_PRESCALE 1
#endif
#ifndef VDN_SOFTMAX_MMASUM
#define VDN_SOFTMAX_MMASUM 0
#endif
constexpr int kBK = VDN_SOFTMAX_BK;  // keys per tile (64 or 128)
static_assert(kBK == 64 || kBK == 128, "key tile");
constexpr int kWaves = VDN_SOFTMAX_WAVES;       // waves per workgroup; 8 / kWaves workgroups per CU
#ifndef VDN_SOFTMAX_QT
#define VDN_SOFTMAX_QT 3
#endif
#ifndef VDN_SOFTMAX_WG_PER_CU
#define VDN_SOFTMAX_WG_PER_CU (8 / VDN_SOFTMAX_WAVES)
#endif
constexpr int kQT = VDN_SOFTMAX_QT; // 16-query column tiles per wave
constexpr int kQW = 16 * kQT;       // queries per wave
constexpr int kBQ = kWaves * kQW;   // queries per workgroup
constexpr int kStages = VDN_SOFTMAX_STAGES;     // LDS stages: up to kStages - 1 tiles in flight
static_assert(kStages >= 2 && kStages <= 4, "LDS stages");
constexpr float kMaxRef = VDN_SOFTMAX_PRESCALE ? 4.0f : 48.0f;   // log2 units; beyond it the fallback kernel runs
constexpr float kRescaleThreshold = 8.0f;   // fallback: log2 units of growth before a rescale
constexpr float kMasked = -1.0e30f;
constexpr int kVmcntZero = 0x0F70;          // s_waitcnt vmcnt(0), other counters untouched
// s_waitcnt immediate for vmcnt(n), n < 64 (low four bits in [3:0], high two in [15:14])
constexpr int vmcnt_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// LDS chunk swizzles (XOR on the 16-byte chunk index of a row).  gfx950 serves a 16-byte LDS read
// 16 lanes per pass over 64 banks of 4 bytes: lanes 16j .. 16j+15 read K rows
// {8a + b : a in 0..3, b in 0..3} + const of one chunk (rows of 2 D bytes) and 16 consecutive V^T
// rows of 128 bytes, and the swizzles put those 16 rows on 16 distinct 16-byte bank slots.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 3) | ((row >> 1) & 12) : ((row >> 1) & 1) | ((row >> 2) & 6);
}
__device__ __forceinline__ int v_swz(int row) { return (row >> 1) & 7; }

template <int D>
struct Smem {
  static constexpr int KCH = D / 8;                 // 16-byte chunks per K row
  static constexpr int K_BYTES = kBK * D * 2;
  static constexpr int V_BYTES = D * kBK * 2;
  static constexpr int STAGE = K_BYTES + V_BYTES;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

struct Params {
  const bf16_t* q;
  const bf16_t* qc;         // context (text, audio) query rows [n_ctx][H][D], or unused
  const bf16_t* kp;
  const bf16_t* vt;
  bf16_t* o_s;
  bf16_t* oc;               // their output [n_ctx][H][D]
  float* lse;               // [T*N + n_ctx][H]: log2 of each row's normaliser in scaled-score units, or nullptr
  const int* ranges;
  const int* nranges;
  const float* kmax;
  int* flags;
  int T, N, H, n_ctx;
  int64_t Ls;
  int QT, QTc, n_ctx_wg, n_bnd_wg, n_int_frames, first_int_frame, per_xcd, n_int_wg;
  float c_log2;
};

// FALLBACK = false: fixed exponent reference, writes its workgroup's flag (1 = redo).
// FALLBACK = true : online maximum; runs only the workgroups flagged by the first launch.
template <int D, bool FALLBACK>
__global__ __launch_bounds__(kWaves * 64, VDN_SOFTMAX_WG_PER_CU) void softmax_mfma_kernel(Params P) {
  using SM = Smem<D>;
  constexpr int KS = D / 32;          // k-steps of the QK^T contraction
  constexpr int DT = D / 16;          // 16-row d tiles of O^T
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int unsafe_any;

  const int w = blockIdx.x;
  if constexpr (FALLBACK) {
    if (P.flags[w] == 0) return;
  }
  // ---- workgroup -> (head, frame, query tile); context rows are pseudo-frame T ----
  int h, t, qt;
  if (w < P.n_ctx_wg) {
    qt = w % P.QTc;
    h = w / P.QTc;
    t = P.T;
  } else if (w - P.n_ctx_wg < P.n_bnd_wg) {
    const int wb = w - P.n_ctx_wg;
    qt = wb % P.QT;
    const int rest = wb / P.QT;
    const int nb = P.n_bnd_wg / (P.QT * P.H);
    const int bi = rest % nb;
    h = rest / nb;
    t = bi == 0 ? 0 : P.T - 1;
  } else {
    const int wp = w - P.n_ctx_wg - P.n_bnd_wg;
    const int L = (w & 7) * P.per_xcd + (wp >> 3);
    if (L >= P.n_int_wg) {
      if constexpr (!FALLBACK) {
        if (threadIdx.x == 0) P.flags[w] = 0;
      }
      return;
    }
    qt = L % P.QT;
    const int rest = L / P.QT;
    t = P.first_int_frame + rest % P.n_int_frames;
    h = rest / P.n_int_frames;
  }
  const int H = P.H;
  const int64_t Ls = P.Ls;
  const bool ctx = t == P.T;
  const int nrows = ctx ? P.n_ctx : P.N;
  const bf16_t* qsrc = ctx ? P.qc + (int64_t)h * D : P.q + ((int64_t)t * P.N * H + h) * D;
  bf16_t* odst = ctx ? P.oc + (int64_t)h * D : P.o_s + ((int64_t)t * P.N * H + h) * D;
  const float c_log2 = P.c_log2;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;

  // ---- Q fragments (B operand of S^T = K Q^T): query l16 of column tile j, d = 32 ks + 8 g .. +8 ----
  bf16x8 qf[kQT][KS];
  float qn2[kQT];
  const int n_base = qt * kBQ + wave * kQW;
#pragma unroll
  for (int j = 0; j < kQT; ++j) {
    qn2[j] = 0.f;
    const int n = n_base + 16 * j + l16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 val = {0, 0, 0, 0};
      if (n < nrows) val = *reinterpret_cast<const u32x4*>(qsrc + (int64_t)n * H * D + ks * 32 + g * 8);
      qf[j][ks] = as_bf16x8(val);
#pragma unroll
      for (int e = 0; e < 8; ++e) qn2[j] += (float)qf[j][ks][e] * (float)qf[j][ks][e];
    }
  }

  // ---- exponent reference (fixed path) or running maximum (fallback) ----
  float mref[kQT];
  {
    const float kmax = P.kmax[h];
    bool unsafe = false;
#pragma unroll
    for (int j = 0; j < kQT; ++j) {
      float s2 = qn2[j] + __shfl_xor(qn2[j], 16);
      s2 += __shfl_xor(s2, 32);
      mref[j] = sqrtf(s2) * kmax * c_log2;
      unsafe |= !(mref[j] <= kMaxRef);
    }
    if constexpr (!FALLBACK && VDN_SOFTMAX_PRESCALE) {
#pragma unroll
      for (int j = 0; j < kQT; ++j)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) qf[j][ks][e] = (__bf16)((float)qf[j][ks][e] * c_log2);
    }
    if constexpr (!FALLBACK) {
      if (tid == 0) unsafe_any = 0;
      __syncthreads();
      if (__builtin_amdgcn_ballot_w64(unsafe) && lane == 0) atomicOr(&unsafe_any, 1);
      __syncthreads();
      const int bad = unsafe_any;
      if (tid == 0) P.flags[w] = bad;
      if (bad) return;
    } else {
#pragma unroll
      for (int j = 0; j < kQT; ++j) mref[j] = -INFINITY;
    }
  }

  // ---- key tiles: full 64-key tiles of every range first, then each range's partial last tile ----
  const int* rg = P.ranges + t * 2 * kMaxRanges;
  const int nr = uniform(P.nranges[t]);
  const int rs0 = uniform(rg[0]), rl0 = uniform(rg[1]) - rs0;
  const int rs1 = nr > 1 ? uniform(rg[2]) : 0, rl1 = nr > 1 ? uniform(rg[3]) - rs1 : 0;
  const int rs2 = nr > 2 ? uniform(rg[4]) : 0, rl2 = nr > 2 ? uniform(rg[5]) - rs2 : 0;
  const int rs3 = nr > 3 ? uniform(rg[6]) : 0, rl3 = nr > 3 ? uniform(rg[7]) - rs3 : 0;
  const int nf0 = rl0 / kBK, nf1 = rl1 / kBK, nf2 = rl2 / kBK, nf3 = rl3 / kBK;
  const int nfull = nf0 + nf1 + nf2 + nf3;
  const int pp0 = (rl0 % kBK) != 0, pp1 = (rl1 % kBK) != 0, pp2 = (rl2 % kBK) != 0, pp3 = (rl3 % kBK) != 0;
  const int ntiles = nfull + pp0 + pp1 + pp2 + pp3;
  auto tile_at = [&](int it, int& key0, int& valid) {
    if (it < nfull) {
      valid = kBK;
      if (it < nf0) { key0 = rs0 + it * kBK; return; }
      it -= nf0;
      if (it < nf1) { key0 = rs1 + it * kBK; return; }
      it -= nf1;
      if (it < nf2) { key0 = rs2 + it * kBK; return; }
      it -= nf2;
      key0 = rs3 + it * kBK;
      return;
    }
    it -= nfull;                              // it-th range that has a partial tile
    if (pp0 && it-- == 0) { key0 = rs0 + nf0 * kBK; valid = rl0 - nf0 * kBK; return; }
    if (pp1 && it-- == 0) { key0 = rs1 + nf1 * kBK; valid = rl1 - nf1 * kBK; return; }
    if (pp2 && it-- == 0) { key0 = rs2 + nf2 * kBK; valid = rl2 - nf2 * kBK; return; }
    key0 = rs3 + nf3 * kBK;
    valid = rl3 - nf3 * kBK;
  };

  const unsigned char* kh = reinterpret_cast<const unsigned char*>(P.kp + (int64_t)h * Ls * D);
  const unsigned char* vh = reinterpret_cast<const unsigned char*>(P.vt + (int64_t)h * D * Ls);

  // Direct global -> LDS tile loads: one instruction of a wave fills 1 KB of LDS, lane l writing
  // bytes [16 l, 16 l + 16), so each lane fetches the global chunk whose swizzled LDS position is
  // its own.  The packed key space ends with a zero tile, so no load leaves the buffer.
  constexpr int K_INSTR = SM::K_BYTES / 1024 / kWaves;     // per wave
  constexpr int V_INSTR = SM::V_BYTES / 1024 / kWaves;
  constexpr int K_ROWS_PER_KB = 1024 / (D * 2);
  constexpr int kVmcntTile = vmcnt_wait(K_INSTR + V_INSTR);          // loads of one tile
  constexpr int kVmcntTile2 = vmcnt_wait(2 * (K_INSTR + V_INSTR));   // ... of two tiles
  static_assert(2 * (K_INSTR + V_INSTR) < 64, "vmcnt field");
  uint32_t koff[K_INSTR], voff[V_INSTR];
#pragma unroll
  for (int i = 0; i < K_INSTR; ++i) {
    const int row = (i * kWaves + wave) * K_ROWS_PER_KB + lane / SM::KCH;
    const int c = (lane % SM::KCH) ^ k_swz<D>(row);
    koff[i] = (uint32_t)(row * D + c * 8) * 2u;
  }
#pragma unroll
  for (int i = 0; i < V_INSTR; ++i) {
    constexpr int VCH = kBK / 8;                        // 16-byte chunks per V^T row
    const int row = (i * kWaves + wave) * (64 / VCH) + lane / VCH;
    const int c = (lane % VCH) ^ v_swz(row);
    voff[i] = (uint32_t)((int64_t)row * Ls + c * 8) * 2u;
  }
  auto issue_tile = [&](int key0, int stage) {
    unsigned char* kb = smem + stage * SM::STAGE;
    unsigned char* vb = kb + SM::K_BYTES;
    const unsigned char* kt0 = kh + (int64_t)key0 * D * 2;
    const unsigned char* vt0 = vh + (int64_t)key0 * 2;
#pragma unroll
    for (int i = 0; i < K_INSTR; ++i)
      __builtin_amdgcn_global_load_lds((gptr_t)(kt0 + koff[i]), (lptr_t)(kb + (i * kWaves + wave) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < V_INSTR; ++i)
      __builtin_amdgcn_global_load_lds((gptr_t)(vt0 + voff[i]), (lptr_t)(vb + (i * kWaves + wave) * 1024), 16, 0, 0);
  };

  f32x4 oacc[DT][kQT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int j = 0; j < kQT; ++j) oacc[dt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float lsum[kQT];
#pragma unroll
  for (int j = 0; j < kQT; ++j) lsum[j] = 0.f;
#if VDN_SOFTMAX_MMASUM
  f32x4 lacc[kQT];
#pragma unroll
  for (int j = 0; j < kQT; ++j) lacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x8 ones8 = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                        (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
#endif

  // K row read by this lane for 16-key tile u of a half (see header): key 8 (l16 / 4) + 4 u + l16 % 4
  const int krow0 = 8 * (l16 >> 2) + (l16 & 3);

  // S^T of one 32-key half: two 16-key row tiles x kQT query tiles.  All K fragments of the half
  // are read before the first MFMA so the LDS latency is paid once per half.
  auto scores = [&](const unsigned char* kb, int half, f32x4 (&sacc)[2][kQT]) {
    bf16x8 kf[2][KS];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int row = half * 32 + krow0 + 4 * u;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = ks * 4 + g;
        kf[u][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(kb + row * (D * 2) + ((c ^ k_swz<D>(row)) * 16)));
      }
    }
    constexpr bool kPre = !FALLBACK && VDN_SOFTMAX_PRESCALE;   // accumulators start at -mref
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < kQT; ++j)
        sacc[u][j] = kPre ? f32x4{-mref[j], -mref[j], -mref[j], -mref[j]} : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < kQT; ++j)
          sacc[u][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[u][ks], qf[j][ks], sacc[u][j], 0, 0, 0);
#if VDN_SOFTMAX_SCHED
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * KS, 0);         // the K fragment reads
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * KS * kQT, 0);   // then the score MFMAs
#endif
  };
  // lane's score i of row tile u is key half*32 + 8 g + 4 u + i
  auto mask = [&](int half, int valid, f32x4 (&sacc)[2][kQT]) {
    // an opaque copy of g: with it the compiler cannot prove the key offset below 64, so the
    // caller's "valid < kBK" test stays a real branch that full tiles skip (else it becomes an
    // unconditional select on every score of every tile)
    int gl = g;
    asm volatile("" : "+v"(gl));
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (half * 32 + 8 * gl + 4 * u + i >= valid) {
#pragma unroll
          for (int j = 0; j < kQT; ++j) sacc[u][j][i] = kMasked;
        }
      }
  };
  // running maximum with lazy rescale (fallback kernel only); a query's 32 scores of the half are
  // spread over the four lane groups g
  auto online_max = [&](f32x4 (&sacc)[2][kQT]) {
    float mxc[kQT];
    bool need = false;
#pragma unroll
    for (int j = 0; j < kQT; ++j) {
      float mx = sacc[0][j][0];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[u][j][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      mxc[j] = mx * c_log2;
      need |= mxc[j] > mref[j] + kRescaleThreshold;
    }
    if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
      for (int j = 0; j < kQT; ++j) {
        const float mnew = fmaxf(mref[j], mxc[j]);
        const float alpha = exp2f(mref[j] - mnew);
        mref[j] = mnew;
        lsum[j] *= alpha;
#if VDN_SOFTMAX_MMASUM
        lacc[j] *= alpha;
#endif
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt][j] *= alpha;
      }
    }
  };
  // P^T fragment of query tile j: keys 8 g .. 8 g + 7 of the half (row tile 0 then row tile 1)
  auto probs = [&](const f32x4 (&sacc)[2][kQT], bf16x8 (&pf)[kQT]) {
#pragma unroll
    for (int j = 0; j < kQT; ++j) {
      float ls = 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // raw v_exp_f32: results below 2^-126 flush to zero, harmless since the largest term of
          // every query is >= 2^-96 (fixed reference) or 1 (online maximum)
          const float p = (!FALLBACK && VDN_SOFTMAX_PRESCALE) ? __builtin_amdgcn_exp2f(sacc[u][j][i])
                                                              : __builtin_amdgcn_exp2f(fmaf(sacc[u][j][i], c_log2, -mref[j]));
#if !VDN_SOFTMAX_DOT2SUM && !VDN_SOFTMAX_MMASUM
          ls += p;
#endif
          pf[j][4 * u + i] = (__bf16)p;
        }
#if VDN_SOFTMAX_DOT2SUM
      // the normaliser from the rounded weights, two per v_dot2c_f32_bf16
      const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int e = 0; e < 4; ++e) ls = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[j][2 * e], pf[j][2 * e + 1]}, one2, ls, false);
#endif
#if !VDN_SOFTMAX_MMASUM
      lsum[j] += ls;
#endif
    }
  };
  auto accumulate = [&](const unsigned char* vb, int half, const bf16x8 (&pf)[kQT]) {
    bf16x8 vf[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int vrow = dt * 16 + l16;
      const int c = half * 4 + g;
      vf[dt] = as_bf16x8(*reinterpret_cast<const u32x4*>(vb + vrow * (kBK * 2) + ((c ^ v_swz(vrow)) * 16)));
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < kQT; ++j)
        oacc[dt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pf[j], oacc[dt][j], 0, 0, 0);
#if VDN_SOFTMAX_MMASUM
    // every row of the product is the query's sum of the half's 32 rounded weights
#pragma unroll
    for (int j = 0; j < kQT; ++j) lacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pf[j], lacc[j], 0, 0, 0);
#endif
#if VDN_SOFTMAX_SCHED
    __builtin_amdgcn_sched_group_barrier(0x100, DT, 0);        // V fragment reads first,
    __builtin_amdgcn_sched_group_barrier(0x002, 256, 0);       // then the probabilities (VALU),
    __builtin_amdgcn_sched_group_barrier(0x008, (DT + VDN_SOFTMAX_MMASUM) * kQT, 0);  // then the MFMAs
#endif
  };

  // Tiles are loaded kStages - 1 ahead of the one being computed; iteration it waits for tile it,
  // synchronises (after which the stage of tile it-1 is free in every wave), refills that stage
  // and computes tile it as two 32-key halves.
  auto wait_younger = [&](int younger) {          // wait until at most `younger` tiles are in flight
    if (younger >= 2) __builtin_amdgcn_s_waitcnt(kVmcntTile2);
    else if (younger == 1) __builtin_amdgcn_s_waitcnt(kVmcntTile);
    else __builtin_amdgcn_s_waitcnt(kVmcntZero);
  };
  for (int i = 0; i < kStages - 1 && i < ntiles; ++i) {
    int key0, valid;
    tile_at(i, key0, valid);
    issue_tile(key0, i);
  }
  for (int it = 0; it < ntiles; ++it) {
    wait_younger(min(ntiles - 1, it + kStages - 2) - it);    // tile it landed
    __syncthreads();
    if (it + kStages - 1 < ntiles) {
      int nkey0, nvalid;
      tile_at(it + kStages - 1, nkey0, nvalid);
      issue_tile(nkey0, (it + kStages - 1) % kStages);
    }
    int key0, valid;
    tile_at(it, key0, valid);
    const unsigned char* kb = smem + (it % kStages) * SM::STAGE;
    const unsigned char* vb = kb + SM::K_BYTES;
#pragma unroll 1
    for (int hp = 0; hp < kBK / 64; ++hp) {     // 64 keys per pass, as two 32-key halves
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int half = 2 * hp + hh;
        f32x4 sacc[2][kQT];
        bf16x8 pf[kQT];
        scores(kb, half, sacc);
        if (valid < kBK) mask(half, valid, sacc);
        if constexpr (FALLBACK) online_max(sacc);
        probs(sacc, pf);
        accumulate(vb, half, pf);
      }
    }
  }

  // ---- normalise and store (bf16): lane holds d rows 16 dt + 4 g + i of query l16 of tile j ----
#pragma unroll
  for (int j = 0; j < kQT; ++j) {
#if VDN_SOFTMAX_MMASUM
    const float tot = lacc[j][0];
#else
    float tot = lsum[j] + __shfl_xor(lsum[j], 16);
    tot += __shfl_xor(tot, 32);
#endif
    const float inv = 1.0f / tot;
    const int n = n_base + 16 * j + l16;
    // video rows at t N + n, context rows (t = T) after them
    if (P.lse && n < nrows && g == 0) P.lse[((int64_t)t * P.N + n) * H + h] = mref[j] + __log2f(tot);
    if (n < nrows) {
      bf16_t* op = odst + (int64_t)n * H * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        __bf16 b4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) b4[i] = (__bf16)(oacc[dt][j][i] * inv);
        *reinterpret_cast<uint2*>(op + dt * 16 + g * 4) = __builtin_bit_cast(uint2, b4);
      }
    }
  }
}

template <int D>
void launch_t(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st, hipEvent_t after_first) {
  Params P{};
  P.q = (const bf16_t*)in.q;
  P.qc = (const bf16_t*)in.ctx_q;
  P.kp = b.kp;
  P.vt = b.vt;
  P.o_s = (bf16_t*)b.os;
  P.oc = (bf16_t*)in.ctx_out;
  P.lse = b.lse;
  P.ranges = b.ranges;
  P.nranges = b.nranges;
  P.kmax = b.kmax;
  P.flags = b.flags;
  P.T = s.T;
  P.N = s.N;
  P.H = s.H;
  P.n_ctx = s.n_ctx;
  P.Ls = s.Ls;
  P.QT = (s.N + kBQ - 1) / kBQ;
  P.QTc = (s.n_ctx + kBQ - 1) / kBQ;
  P.n_ctx_wg = in.ctx_out ? P.QTc * s.H : 0;
  const bool two_bnd = s.anchors && s.T > 1;
  const int nb = s.anchors ? (two_bnd ? 2 : 1) : 0;
  P.n_int_frames = s.T - nb;
  P.first_int_frame = s.anchors ? 1 : 0;
  P.n_bnd_wg = nb * P.QT * s.H;
  P.n_int_wg = P.n_int_frames * P.QT * s.H;
  P.per_xcd = (P.n_int_wg + 7) / 8;
  P.c_log2 = 1.4426950408889634f / sqrtf((float)D);
  const int grid = softmax_grid(s, in.ctx_out != nullptr);
  const size_t smem = kStages * Smem<D>::STAGE;
  (void)hipFuncSetAttribute((const void*)softmax_mfma_kernel<D, false>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  (void)hipFuncSetAttribute((const void*)softmax_mfma_kernel<D, true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  hipLaunchKernelGGL((softmax_mfma_kernel<D, false>), dim3(grid), dim3(kWaves * 64), smem, st, P);
  if (after_first) (void)hipEventRecord(after_first, st);
  hipLaunchKernelGGL((softmax_mfma_kernel<D, true>), dim3(grid), dim3(kWaves * 64), smem, st, P);
}

}  // namespace

int softmax_grid(const Shape& s, bool with_ctx) {
  const int QT = (s.N + kBQ - 1) / kBQ;
  const int nb = s.anchors ? (s.T > 1 ? 2 : 1) : 0;
  const int n_ctx_wg = with_ctx ? (s.n_ctx + kBQ - 1) / kBQ * s.H : 0;
  const int n_bnd_wg = nb * QT * s.H;
  const int n_int_wg = (s.T - nb) * QT * s.H;
  return n_ctx_wg + n_bnd_wg + 8 * ((n_int_wg + 7) / 8);
}

hipError_t launch_softmax_mfma(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st,
                               hipEvent_t after_first) {
  if (s.d == 128) launch_t<128>(s, in, b, st, after_first);
  else launch_t<64>(s, in, b, st, after_first);
  return hipGetLastError();
}

}  // namespace vdn
