// Block-sparse window softmax of the VDN layer on CDNA4 matrix cores (bf16 in, fp32 accumulate).
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Local Softmax and
// Long-Range Linear Memory": a video query in chunk c attends, with one softmax, to the text keys,
// the keys of chunks c-1, c, c+1 and the two boundary anchor frames (boundary query frames attend
// to every frame).  The key set of a query frame is at most four contiguous ranges of the packed
// key space (built on the host), so the kernel is a flash-style attention over a range list.
//
// Work decomposition
//   * one workgroup = 256 queries of one frame and one head; 8 waves x 32 queries, two waves per
//     SIMD so one wave's exponentials overlap the other's MFMAs (measured faster on gfx950 than
//     4 waves x 64 queries at one wave per SIMD, which halves the LDS reads per MFMA but leaves
//     every LDS and MFMA latency exposed);
//   * key tiles of 64 keys are loaded straight from global memory into LDS (global_load_lds, four
//     stages: up to three tiles in flight; K as [key][d], V transposed as [d][key], both
//     XOR-swizzled so the 16-byte fragment reads are bank-conflict free) and processed as two
//     32-key halves;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys as rows, queries as columns) so that each
//     lane ends up holding 16 consecutive keys of one query -- the row permutation used when the
//     K fragments are read makes those keys contiguous;  O^T += V^T P^T with the same instruction,
//     P taken straight from the S^T registers (no LDS round trip);
//   * exponent reference: softmax is invariant to the offset subtracted from the scores, and
//     |q.k| <= |q| max|k| bounds every score of the query, so p = 2^(s c - |q| kmax c) never
//     exceeds 1 and needs no running maximum and no rescaling of the accumulator (kmax = largest
//     key norm of the head, from the packing pass).  When that bound is so loose that the largest
//     term could underflow (|q| kmax c > 48 in log2 units -- far outside unit-normalised inputs)
//     the workgroup flags itself and a second launch of the same kernel with the classic online
//     maximum (running max, rescale of the accumulator) redoes just those workgroups;
//   * workgroup order: the long boundary-frame workgroups first (longest job first), then the
//     interior ones remapped so that consecutive query tiles -- which share their key window --
//     land on the same XCD (workgroups are dispatched round-robin over the 8 XCDs).
#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

constexpr int kBK = 64;        // keys per tile
#ifndef VDN_SOFTMAX_BQ
#define VDN_SOFTMAX_BQ 256
#endif
#ifndef VDN_SOFTMAX_SIMPLE
#define VDN_SOFTMAX_SIMPLE 0
#endif
constexpr int kBQ = VDN_SOFTMAX_BQ;   // queries per workgroup
#ifndef VDN_SOFTMAX_STAGES
#define VDN_SOFTMAX_STAGES 4
#endif
constexpr bool kSimpleLoop = VDN_SOFTMAX_SIMPLE != 0;
constexpr int kPipeStages = VDN_SOFTMAX_STAGES;     // LDS stages of the pipelined loop (3 or 4)
constexpr int kStages = kSimpleLoop ? 2 : kPipeStages;
static_assert(kPipeStages == 3 || kPipeStages == 4, "pipeline stages");
// Wave shape: QSUB 32-query column tiles per wave, kBQ / (32 QSUB) waves per workgroup.
#ifndef VDN_SOFTMAX_QSUB
#define VDN_SOFTMAX_QSUB 1
#endif
constexpr int kQSub = VDN_SOFTMAX_QSUB;
constexpr int kWaves = kBQ / (32 * kQSub);
constexpr int kQW = 32 * kQSub;        // queries per wave
constexpr float kMaxRef = 48.0f;            // log2 units; beyond it the fallback kernel runs
constexpr float kRescaleThreshold = 8.0f;   // fallback: log2 units of growth before a rescale
constexpr float kMasked = -1.0e30f;
constexpr int kVmcntZero = 0x0F70;          // s_waitcnt vmcnt(0), other counters untouched

// LDS chunk swizzles (16-byte chunks).  K rows are read 16 rows per 16 lanes in the order
// {0-3,16-19,4-7,20-23} (+8 for the next 16 lanes); V^T rows 16 consecutive rows per 16 lanes.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  const int r = row & 31;
  if constexpr (D == 128) return (r & 7) | ((r >> 1) & 8);
  else return ((r >> 1) & 3) | ((r >> 2) & 4);
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
__global__ __launch_bounds__(kWaves * 64, 8 / kWaves) void softmax_mfma_kernel(Params P) {
  using SM = Smem<D>;
  constexpr int KS = D / 16;          // k-steps of the QK^T contraction
  constexpr int DT = D / 32;          // 32-row d tiles of O^T
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int unsafe_any;

  const int w = blockIdx.x;
  if constexpr (FALLBACK) {
    if (P.flags[w] == 0) return;
  }
  // ---- workgroup -> (head, frame, query tile); the context rows (every key) come first as
  // pseudo-frame T, then the boundary frames, then the interior frames ----
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
  // this workgroup's query rows: nrows rows of stride H*D from qsrc, results to odst
  const bool ctx = t == P.T;
  const int nrows = ctx ? P.n_ctx : P.N;
  const bf16_t* qsrc = ctx ? P.qc + (int64_t)h * D : P.q + ((int64_t)t * P.N * H + h) * D;
  bf16_t* odst = ctx ? P.oc + (int64_t)h * D : P.o_s + ((int64_t)t * P.N * H + h) * D;
  const float c_log2 = P.c_log2;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hl = lane >> 5;

  // ---- Q fragments (B operand of S^T = K Q^T): query = l32 (+32 qs), d = ks*16 + hl*8 .. +8 ----
  bf16x8 qf[kQSub][KS];
  float qn2[kQSub];
#pragma unroll
  for (int qs = 0; qs < kQSub; ++qs) qn2[qs] = 0.f;
  const int n_base = qt * kBQ + wave * kQW;
#pragma unroll
  for (int qs = 0; qs < kQSub; ++qs) {
    const int n = n_base + qs * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 val = {0, 0, 0, 0};
      if (n < nrows) val = *reinterpret_cast<const u32x4*>(qsrc + (int64_t)n * H * D + ks * 16 + hl * 8);
      qf[qs][ks] = as_bf16x8(val);
#pragma unroll
      for (int e = 0; e < 8; ++e) qn2[qs] += (float)qf[qs][ks][e] * (float)qf[qs][ks][e];
    }
  }

  // ---- exponent reference (fixed path) or running maximum (fallback) ----
  float mref[kQSub];
  {
    const float kmax = P.kmax[h];
    bool unsafe = false;
#pragma unroll
    for (int qs = 0; qs < kQSub; ++qs) {
      const float qn = sqrtf(qn2[qs] + __shfl_xor(qn2[qs], 32));
      mref[qs] = qn * kmax * c_log2;
      unsafe |= !(mref[qs] <= kMaxRef);
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
      for (int qs = 0; qs < kQSub; ++qs) mref[qs] = -INFINITY;
    }
  }

  // ---- key tiles (all workgroup-uniform scalars).  Full 64-key tiles of every range come first,
  // then the partial last tile of each range whose length is not a multiple of 64: the main loop
  // is then straight-line code and only the short second loop masks keys. ----
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

  // Direct global -> LDS tile loads (global_load_lds_dwordx4): one instruction of a wave fills 1 KB
  // of LDS, lane l writing bytes [16 l, 16 l + 16).  Each lane therefore fetches the global chunk
  // whose swizzled LDS position is its own: a workgroup-uniform tile base plus a fixed 32-bit lane
  // offset.  The packed key space ends with a zero tile, so no load leaves the buffer.
  constexpr int K_INSTR = SM::K_BYTES / 1024 / kWaves;     // per wave
  constexpr int V_INSTR = SM::V_BYTES / 1024 / kWaves;
  constexpr int K_ROWS_PER_KB = 1024 / (D * 2);
  static_assert(K_INSTR + V_INSTR < 16, "vmcnt field");
  constexpr int kVmcntTile = 0x0F70 | (K_INSTR + V_INSTR);   // s_waitcnt vmcnt(loads of one tile)
  constexpr int kVmcntTile2 = 0x0F70 | (2 * (K_INSTR + V_INSTR));   // ... of two tiles
  static_assert(2 * (K_INSTR + V_INSTR) < 16, "vmcnt field");
  uint32_t koff[K_INSTR], voff[V_INSTR];
#pragma unroll
  for (int i = 0; i < K_INSTR; ++i) {
    const int row = (i * kWaves + wave) * K_ROWS_PER_KB + lane / SM::KCH;
    const int c = (lane % SM::KCH) ^ k_swz<D>(row);
    koff[i] = (uint32_t)(row * D + c * 8) * 2u;
  }
#pragma unroll
  for (int i = 0; i < V_INSTR; ++i) {
    const int row = (i * kWaves + wave) * 8 + lane / 8;
    const int c = (lane % 8) ^ v_swz(row);
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

  f32x16 oacc[kQSub][DT];
#pragma unroll
  for (int qs = 0; qs < kQSub; ++qs)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[qs][dt][i] = 0.f;
  float lsum[kQSub];
#pragma unroll
  for (int qs = 0; qs < kQSub; ++qs) lsum[qs] = 0.f;

  // row of the K tile that this lane feeds as MFMA row l32 (see header): key 16*h + 4*a + b
  const int krow = ((l32 >> 2) & 1) * 16 + (l32 >> 3) * 4 + (l32 & 3);

  // S^T for one 32-key half: 2 query subtiles.  All K fragments of the half are read before the
  // first MFMA so the LDS latency is paid once per half, not once per fragment.
  auto scores = [&](const unsigned char* kb, int kt, f32x16 (&sacc)[kQSub]) {
    const int row = kt * 32 + krow;
    bf16x8 kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = ks * 2 + hl;
      kf[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(kb + row * (D * 2) + ((c ^ k_swz<D>(row)) * 16)));
    }
#pragma unroll
    for (int qs = 0; qs < kQSub; ++qs)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[qs][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int qs = 0; qs < kQSub; ++qs)
        sacc[qs] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[qs][ks], sacc[qs], 0, 0, 0);
  };
  auto mask = [&](int kt, int valid, f32x16 (&sacc)[kQSub]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kl = kt * 32 + hl * 16 + i;
      if (kl >= valid) {
#pragma unroll
        for (int qs = 0; qs < kQSub; ++qs) sacc[qs][i] = kMasked;
      }
    }
  };
  // running maximum with lazy rescale (fallback kernel only)
  auto online_max = [&](f32x16 (&sacc)[kQSub]) {
    float mxc[kQSub];
    bool need = false;
#pragma unroll
    for (int qs = 0; qs < kQSub; ++qs) {
      float mx = sacc[qs][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[qs][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      mxc[qs] = mx * c_log2;
      need |= mxc[qs] > mref[qs] + kRescaleThreshold;
    }
    if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
      for (int qs = 0; qs < kQSub; ++qs) {
        const float mnew = fmaxf(mref[qs], mxc[qs]);
        const float alpha = exp2f(mref[qs] - mnew);
        mref[qs] = mnew;
        lsum[qs] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[qs][dt][i] *= alpha;
      }
    }
  };
  auto probs = [&](const f32x16 (&sacc)[kQSub], bf16x8 (&pf)[kQSub][2]) {
#pragma unroll
    for (int qs = 0; qs < kQSub; ++qs) {
      float ls = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // raw v_exp_f32: results below 2^-126 flush to zero, harmless since the largest term of
        // every query is >= 2^-96 (fixed reference) or 1 (online maximum)
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[qs][i], c_log2, -mref[qs]));
        ls += p;
        pf[qs][i >> 3][i & 7] = (__bf16)p;
      }
      lsum[qs] += ls;
    }
  };
  auto accumulate = [&](const unsigned char* vb, int kt, const bf16x8 (&pf)[kQSub][2]) {
    bf16x8 vf[DT][2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int vrow = dt * 32 + l32;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int c = kt * 4 + hl * 2 + s;
        vf[dt][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(vb + vrow * (kBK * 2) + ((c ^ v_swz(vrow)) * 16)));
      }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int qs = 0; qs < kQSub; ++qs)
          oacc[qs][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[dt][s], pf[qs][s], oacc[qs][dt], 0, 0, 0);
  };

  auto next_tile = [&](int it) {
    if (it + 1 < ntiles) {
      int nkey0, nvalid;
      tile_at(it + 1, nkey0, nvalid);
      issue_tile(nkey0, (it + 1) & 1);
    }
  };

  if constexpr (!FALLBACK && !kSimpleLoop) {
    // Software-pipelined over tiles with kPipeStages LDS stages: iteration i computes the scores of
    // tile i+1 (MFMA) while it turns the scores of tile i into probabilities (VALU), then
    // accumulates P.V of tile i.  The two streams are independent inside the iteration, so one
    // wave keeps the matrix pipe and the vector ALU busy at the same time.  Full tiles come before
    // partial ones (tile_at), so masking is a uniform branch outside the overlapped block.
    // Tiles are loaded kPipeStages - 1 ahead of the one whose scores are computed.
    constexpr int S = kPipeStages;
    auto wait_younger = [&](int younger) {          // wait until at most `younger` tiles are in flight
      if (younger >= 2) __builtin_amdgcn_s_waitcnt(kVmcntTile2);
      else if (younger == 1) __builtin_amdgcn_s_waitcnt(kVmcntTile);
      else __builtin_amdgcn_s_waitcnt(kVmcntZero);
    };
    f32x16 sc0[kQSub], sc1[kQSub];          // scores of the tile being finished
    for (int i = 0; i < S - 1 && i < ntiles; ++i) {
      int key0, valid;
      tile_at(i, key0, valid);
      issue_tile(key0, i);
    }
    wait_younger(min(ntiles, S - 1) - 1);           // tile 0 landed
    __syncthreads();
    scores(smem, 0, sc0);
    scores(smem, 1, sc1);
    for (int it = 0; it + 1 < ntiles; ++it) {
      wait_younger(min(ntiles - 1, it + S - 2) - (it + 1));   // tile it+1 landed
      __syncthreads();                              // ... for every wave; stage (it-1)%S is free
      if (it + S - 1 < ntiles) {
        int nkey0, nvalid;
        tile_at(it + S - 1, nkey0, nvalid);
        issue_tile(nkey0, (it + S - 1) % S);
      }
      int key0, valid;
      tile_at(it, key0, valid);
      if (valid < kBK) {
        mask(0, valid, sc0);
        mask(1, valid, sc1);
      }
      const unsigned char* kn = smem + ((it + 1) % S) * SM::STAGE;
      const unsigned char* vb = smem + (it % S) * SM::STAGE + SM::K_BYTES;
      f32x16 sn0[kQSub], sn1[kQSub];
      bf16x8 p0[kQSub][2], p1[kQSub][2];
      scores(kn, 0, sn0);
      probs(sc0, p0);
      scores(kn, 1, sn1);
      probs(sc1, p1);
      accumulate(vb, 0, p0);
      accumulate(vb, 1, p1);
#pragma unroll
      for (int qs = 0; qs < kQSub; ++qs) {
        sc0[qs] = sn0[qs];
        sc1[qs] = sn1[qs];
      }
    }
    {
      const int it = ntiles - 1;
      int key0, valid;
      tile_at(it, key0, valid);
      if (valid < kBK) {
        mask(0, valid, sc0);
        mask(1, valid, sc1);
      }
      const unsigned char* vb = smem + (it % S) * SM::STAGE + SM::K_BYTES;
      bf16x8 p0[kQSub][2], p1[kQSub][2];
      probs(sc0, p0);
      probs(sc1, p1);
      accumulate(vb, 0, p0);
      accumulate(vb, 1, p1);
    }
  } else {
    {
      int key0, valid;
      tile_at(0, key0, valid);
      issue_tile(key0, 0);
    }
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
      next_tile(it);
      int key0, valid;
      tile_at(it, key0, valid);
      const unsigned char* kb = smem + (it & 1) * SM::STAGE;
      const unsigned char* vb = kb + SM::K_BYTES;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x16 sacc[kQSub];
        bf16x8 pf[kQSub][2];
        scores(kb, kt, sacc);
        if (valid < kBK) mask(kt, valid, sacc);
        if constexpr (FALLBACK) online_max(sacc);
        probs(sacc, pf);
        accumulate(vb, kt, pf);
      }
      __builtin_amdgcn_s_waitcnt(kVmcntZero);
      __syncthreads();
    }
  }

  // ---- normalise and store o_s (bf16) ----
#pragma unroll
  for (int qs = 0; qs < kQSub; ++qs) {
    const float tot = lsum[qs] + __shfl_xor(lsum[qs], 32);
    const float inv = 1.0f / tot;
    const int n = n_base + qs * 32 + l32;
    if (n < nrows) {
      bf16_t* op = odst + (int64_t)n * H * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          __bf16 b4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) b4[e] = (__bf16)(oacc[qs][dt][g * 4 + e] * inv);
          *reinterpret_cast<uint2*>(op + dt * 32 + g * 8 + hl * 4) = __builtin_bit_cast(uint2, b4);
        }
    }
  }
}

template <int D>
void launch_t(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  Params P{};
  P.q = (const bf16_t*)in.q;
  P.qc = (const bf16_t*)in.ctx_q;
  P.kp = b.kp;
  P.vt = b.vt;
  P.o_s = (bf16_t*)b.os;
  P.oc = (bf16_t*)in.ctx_out;
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
  (void)hipFuncSetAttribute((const void*)softmax_mfma_kernel<D, false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)smem);
  (void)hipFuncSetAttribute((const void*)softmax_mfma_kernel<D, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)smem);
  hipLaunchKernelGGL((softmax_mfma_kernel<D, false>), dim3(grid), dim3(kWaves * 64), smem, st, P);
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

hipError_t launch_softmax_mfma(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  if (s.d == 128) launch_t<128>(s, in, b, st);
  else launch_t<64>(s, in, b, st);
  return hipGetLastError();
}

}  // namespace vdn
