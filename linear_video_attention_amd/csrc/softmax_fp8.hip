// FP8 (E4M3) variant of the block-sparse window softmax on CDNA4 matrix cores, d = 128.
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Local Softmax and
// Long-Range Linear Memory": one softmax per video query over the global (text, audio) keys, the
// keys of chunks c-1 .. c+1 and the boundary anchors (every frame for boundary query frames); the
// pages run their production kernels with FP8 (section "Adapting the Pretrained H3 backbone") but
// do not fix its roundings.  The roundings made here, each a deterministic step:
//   * operands: K8 = e4m3(s_k k), V8 = e4m3(s_v v) (power-of-two scales per head, packed by
//     prep_fp8.hip), Q8 = e4m3(s_q c q) with c = log2(e)/sqrt(d) and s_q = 2^(8 - e) from the
//     largest |c q_i| of the query;
//   * scores x = <Q8, K8> / (s_q s_k), already in log2 units, on v_mfma_scale_f32_16x16x128_f8f6f4
//     (the E8M0 block scales divide by s_k and s_q; fp32 accumulate, started at 8 - m);
//   * weights P8 = e4m3(2^(8 + x - m)) with the offset m = c |q| kmax when that bound is <= 4
//     (then the largest weight of every row is >= 1, far above E4M3's underflow), else the row's
//     exact maximum max x (a second launch of this kernel, for the workgroups that hold such rows,
//     first scans the row's scores for it); a weight is exp2 of the accumulator;
//   * o = sum P8 V8 / (s_v sum P8): the normaliser sums the rounded weights, on the matrix cores
//     (a constant all-ones A operand next to the V^T tiles), and o_s is stored in bf16.
//
// Work decomposition (as the bf16 kernel, with 128-key tiles: one k-step of the P.V product):
//   * one workgroup = 256 queries of one frame and head, 8 waves x 32 queries (two 16-query
//     tiles), two waves per SIMD;
//   * K [128 keys][128 B] and V^T [128 channels][128 B] tiles go global -> LDS by
//     global_load_lds (16-byte chunks XOR-swizzled so each 8-lane group of a fragment read hits
//     distinct banks), two stages;
//   * S^T = K Q^T with key rows permuted: 16-key tile u of the 128-key tile, fragment row r, is key
//     32 (r / 4) + 4 u + r % 4, so the four scores a lane gets from tile u are keys 32 g + 4 u + i
//     (g = lane / 16): over u = 0..7 a lane holds 32 consecutive keys of its query, exactly its
//     32 bytes of the P^T operand of O^T += V^T P^T.  A and B operands of one MFMA place the same
//     contraction index at the same (lane group, byte), whatever the hardware's own k order.
#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

constexpr int D = 128;
constexpr int kBK = 128;            // keys per tile
constexpr int kWaves = 8;
// Build parameters (defaults measured best at 768p; the alternatives are kept for measurement):
//   VDN_FP8_QT   16-query tiles per wave (2; 3 exceeds the register budget of two waves per SIMD)
//   VDN_FP8_UG   16-key score tiles formed per step before their weights (1, 2, 4)
#ifndef VDN_FP8_QT
#define VDN_FP8_QT 2
#endif
#ifndef VDN_FP8_UG
#define VDN_FP8_UG 2
#endif
constexpr int kQT = VDN_FP8_QT;     // 16-query tiles per wave
constexpr int kUG = VDN_FP8_UG;
constexpr int kQW = 16 * kQT;
constexpr int kBQ = kWaves * kQW;   // queries per workgroup
#ifndef VDN_FP8_STAGES
#define VDN_FP8_STAGES 2
#endif
constexpr int kStages = VDN_FP8_STAGES;   // LDS stages (2; 3 keeps two tiles in flight, 2 % slower)
static_assert(kStages == 2 || kStages == 3, "stages");
constexpr int K_BYTES = kBK * D;    // 16 KB
constexpr int V_BYTES = D * kBK;    // 16 KB
constexpr int STAGE = K_BYTES + V_BYTES;
constexpr float kBoundLimit = 4.0f; // log2 units: larger bounds take the row maximum as offset
constexpr float kShift = 8.0f;      // weights are rounded as 2^8 p
constexpr float kMasked = -1.0e30f;
constexpr int kVmcntZero = 0x0F70;
constexpr uint32_t kOnes = 0x38383838u;   // four E4M3 ones

// LDS swizzles (XOR on the 16-byte chunk index of a 128-byte row): a 16-byte LDS read is served
// 16 lanes per pass over 64 banks of 4 bytes, and the 16 rows one lane group reads -- K rows
// {32 a + b : a in 0..3, b in 0..3} + const, V^T rows 16 consecutive -- fall on 16 distinct
// 16-byte slots of the 256-byte bank period
__device__ __forceinline__ int k_swz(int row) { return ((row >> 1) & 1) | ((row >> 4) & 6); }
__device__ __forceinline__ int v_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float pow2_scale(float m) {
  if (!(m > 0.f)) return 1.f;
  int e;
  (void)frexpf(m, &e);
  return ldexpf(1.f, 8 - e);
}

__device__ __forceinline__ f32x4 mfma8(const i32x8& a, const i32x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// scores of the c-scaled query in log2 units: (K8 . Q8) 2^(ea - 127) 2^(eb - 127) + c0
__device__ __forceinline__ f32x4 mfma8_scaled(const i32x8& a, const i32x8& b, const f32x4& c0, int ea, int eb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c0, 0, 0, 0, ea, 0, eb);
}

__device__ __forceinline__ i32x8 join(u32x4 lo, u32x4 hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Walks a query frame's key ranges (at most four, in order) 128 keys at a time.
struct TileCursor {
  int s0, e0, s1, e1, s2, e2, s3, e3;   // [start, end) of each range; unused ranges are empty
  int r, key;                           // current range and the next tile's first key
  __device__ __forceinline__ int end_of(int i) const { return i == 0 ? e0 : i == 1 ? e1 : i == 2 ? e2 : e3; }
  __device__ __forceinline__ int start_of(int i) const { return i == 0 ? s0 : i == 1 ? s1 : i == 2 ? s2 : s3; }
  // the next tile: its first key and its number of keys (<= 128); only called while tiles remain
  __device__ __forceinline__ void pop(int& key0, int& valid) {
    while (key >= end_of(r)) {            // skip to the next range that has keys
      ++r;
      key = start_of(r);
    }
    key0 = key;
    valid = min(kBK, end_of(r) - key);
    key += kBK;
  }
};

// K and V^T tiles of 128 keys from global memory straight into one LDS stage: per wave K_INSTR + V_INSTR
// instructions of 1 KB each (lane offsets koff, voff precomputed with the swizzle)
constexpr int K_INSTR = K_BYTES / 1024 / kWaves;   // 2
constexpr int V_INSTR = V_BYTES / 1024 / kWaves;   // 2
__device__ __forceinline__ void issue_tile(const uint8_t* kh, const uint8_t* vh, const uint32_t (&koff)[K_INSTR],
                                           const uint32_t (&voff)[V_INSTR], unsigned char* kb, int key0, int wave) {
  unsigned char* vb = kb + K_BYTES;
  const uint8_t* kt0 = kh + (int64_t)key0 * D;
  const uint8_t* vt0 = vh + key0;
#pragma unroll
  for (int i = 0; i < K_INSTR; ++i)
    __builtin_amdgcn_global_load_lds((gptr_t)(kt0 + koff[i]), (lptr_t)(kb + (i * kWaves + wave) * 1024), 16, 0, 0);
#pragma unroll
  for (int i = 0; i < V_INSTR; ++i)
    __builtin_amdgcn_global_load_lds((gptr_t)(vt0 + voff[i]), (lptr_t)(vb + (i * kWaves + wave) * 1024), 16, 0, 0);
}

struct Params {
  const bf16_t* q;
  const bf16_t* qc;
  const uint8_t* k8;
  const uint8_t* v8;
  bf16_t* o_s;
  bf16_t* oc;
  const int* ranges;
  const int* nranges;
  const float* kmax;
  const float* scale;       // [H][2]: s_k, s_v
  int* flags;
  int T, N, H, n_ctx;
  int64_t Ls8;
  int QT, QTc, n_ctx_wg, n_bnd_wg, n_int_frames, first_int_frame, per_xcd, n_int_wg;
  float c_log2;
};

// FALLBACK = false: bound offset for every row; a workgroup holding a row whose bound exceeds the
// limit flags itself and returns.  FALLBACK = true: runs the flagged workgroups only; rows over the
// limit take their exact row maximum (first pass over the key tiles), the others the bound.
template <bool FALLBACK>
__global__ __launch_bounds__(kWaves * 64, 1) void softmax_fp8_kernel(Params P) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int unsafe_any;
  const int w = blockIdx.x;
  if constexpr (FALLBACK) {
    if (P.flags[w] == 0) return;
  }
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
  const int64_t Ls8 = P.Ls8;
  const bool ctx = t == P.T;
  const int nrows = ctx ? P.n_ctx : P.N;
  const bf16_t* qsrc = ctx ? P.qc + (int64_t)h * D : P.q + ((int64_t)t * P.N * H + h) * D;
  bf16_t* odst = ctx ? P.oc + (int64_t)h * D : P.o_s + ((int64_t)t * P.N * H + h) * D;
  const float sk = P.scale[2 * h], sv = P.scale[2 * h + 1];
  const int ekey = 127 - ilogbf(sk);              // E8M0 exponent dividing the scores by s_k
  const float kmax = P.kmax[h];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;

  // ---- Q8 fragments: query l16 of tile j, channels 32 g .. 32 g + 31 ----
  i32x8 qf[kQT];
  int escale[kQT];               // per query: E8M0 exponent dividing the scores by s_q
  float moff[kQT];               // per query: exponent offset minus the shift
  bool over[kQT];                // the query's bound exceeds the limit
  const int n_base = qt * kBQ + wave * kQW;
  bool unsafe = false;
#pragma unroll
  for (int j = 0; j < kQT; ++j) {
    const int n = n_base + 16 * j + l16;
    float x[32];
    u32x4 raw[4] = {};
    if (n < nrows) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        raw[c] = *reinterpret_cast<const u32x4*>(qsrc + (int64_t)n * H * D + 32 * g + 8 * c);
    }
    float amax = 0.f, ss = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * c + 2 * e] = __uint_as_float(raw[c][e] << 16);
        x[8 * c + 2 * e + 1] = __uint_as_float(raw[c][e] & 0xFFFF0000u);
      }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      ss += x[i] * x[i];
      x[i] *= P.c_log2;                          // the query enters as c q
      amax = fmaxf(amax, fabsf(x[i]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const float sq = pow2_scale(amax);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int wv = __builtin_amdgcn_cvt_pk_fp8_f32(sq * x[4 * i], sq * x[4 * i + 1], 0, false);
      wv = __builtin_amdgcn_cvt_pk_fp8_f32(sq * x[4 * i + 2], sq * x[4 * i + 3], wv, true);
      qf[j][i] = wv;
    }
    escale[j] = 127 - ilogbf(sq);
    const float bound = sqrtf(ss) * kmax * P.c_log2;
    over[j] = !(bound <= kBoundLimit);
    unsafe |= over[j];
    moff[j] = bound - kShift;
  }
  if constexpr (!FALLBACK) {
    if (tid == 0) unsafe_any = 0;
    __syncthreads();
    if (__builtin_amdgcn_ballot_w64(unsafe) && lane == 0) atomicOr(&unsafe_any, 1);
    __syncthreads();
    const int bad = unsafe_any;
    if (tid == 0) P.flags[w] = bad;
    if (bad) return;
  }

  // ---- key tiles: the ranges in order, 128 keys at a time (a range's last tile may be partial) ----
  const int* rg = P.ranges + t * 2 * kMaxRanges;
  const int nr = uniform(P.nranges[t]);
  TileCursor cur;
  cur.s0 = uniform(rg[0]);
  cur.e0 = uniform(rg[1]);
  cur.s1 = nr > 1 ? uniform(rg[2]) : 0;
  cur.e1 = nr > 1 ? uniform(rg[3]) : 0;
  cur.s2 = nr > 2 ? uniform(rg[4]) : 0;
  cur.e2 = nr > 2 ? uniform(rg[5]) : 0;
  cur.s3 = nr > 3 ? uniform(rg[6]) : 0;
  cur.e3 = nr > 3 ? uniform(rg[7]) : 0;
  cur.r = 0;
  cur.key = cur.s0;
  const int ntiles = (cur.e0 - cur.s0 + kBK - 1) / kBK + (cur.e1 - cur.s1 + kBK - 1) / kBK +
                     (cur.e2 - cur.s2 + kBK - 1) / kBK + (cur.e3 - cur.s3 + kBK - 1) / kBK;

  const uint8_t* kh = P.k8 + (int64_t)h * Ls8 * D;
  const uint8_t* vh = P.v8 + (int64_t)h * D * Ls8;
  // one global_load_lds of a wave fills 1 KB = 8 rows of 128 B; lane l writes row 8 i' + l / 8,
  // chunk position l % 8, and fetches the global chunk whose swizzled position that is
  uint32_t koff[K_INSTR], voff[V_INSTR];
#pragma unroll
  for (int i = 0; i < K_INSTR; ++i) {
    const int row = (i * kWaves + wave) * 8 + lane / 8;
    koff[i] = (uint32_t)(row * D + ((lane % 8) ^ k_swz(row)) * 16);
  }
#pragma unroll
  for (int i = 0; i < V_INSTR; ++i) {
    const int row = (i * kWaves + wave) * 8 + lane / 8;
    voff[i] = (uint32_t)((int64_t)row * Ls8 + ((lane % 8) ^ v_swz(row)) * 16);
  }
  // K fragment of 16-key tile u: row 32 (l16 / 4) + 4 u + l16 % 4, channels 32 g .. 32 g + 31
  const int krow0 = 32 * (l16 >> 2) + (l16 & 3);
  auto kfrag = [&](const unsigned char* kb, int u) __attribute__((always_inline)) {
    const int row = krow0 + 4 * u;
    const unsigned char* base = kb + row * D;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + (((2 * g) ^ k_swz(row)) * 16));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + (((2 * g + 1) ^ k_swz(row)) * 16));
    return join(lo, hi);
  };
  // V^T fragment of channel tile dt: row 16 dt + l16, keys 32 g .. 32 g + 31 of the tile
  auto vfrag = [&](const unsigned char* vb, int dt) __attribute__((always_inline)) {
    const int row = 16 * dt + l16;
    const unsigned char* base = vb + row * kBK;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + (((2 * g) ^ v_swz(row)) * 16));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + (((2 * g + 1) ^ v_swz(row)) * 16));
    return join(lo, hi);
  };

  // Tile pipeline: tiles are loaded kStages - 1 ahead of the one being computed.  At the top of an
  // iteration a wave waits until only the younger tiles' loads are in flight; after the barrier
  // the stage of tile it - 1 is free in every wave and takes tile it + kStages - 1.  va / vb hold
  // the key counts of the tiles in flight (oldest first).
  constexpr int kVmcntOneTile = 0x0F70 | (K_INSTR + V_INSTR);
#define VDN_FP8_FIRST_TILE(cursor, va, vb)                                                   \
  {                                                                                          \
    int key0_;                                                                               \
    if (ntiles > 0) {                                                                        \
      cursor.pop(key0_, va);                                                                 \
      issue_tile(kh, vh, koff, voff, smem, key0_, wave);                                     \
    }                                                                                        \
    if (kStages == 3 && ntiles > 1) {                                                        \
      cursor.pop(key0_, vb);                                                                 \
      issue_tile(kh, vh, koff, voff, smem + STAGE, key0_, wave);                             \
    }                                                                                        \
  }
#define VDN_FP8_NEXT_TILE(it, cursor, valid, va, vb, kb)                                     \
  {                                                                                          \
    if (kStages == 3 && it + 1 < ntiles) __builtin_amdgcn_s_waitcnt(kVmcntOneTile);          \
    else __builtin_amdgcn_s_waitcnt(kVmcntZero);                                             \
    __syncthreads();                                                                         \
    valid = va;                                                                              \
    if (kStages == 3) va = vb;                                                               \
    if (it + kStages - 1 < ntiles) {                                                         \
      int key0_;                                                                             \
      cursor.pop(key0_, kStages == 3 ? vb : va);                                             \
      issue_tile(kh, vh, koff, voff, smem + ((it + kStages - 1) % kStages) * STAGE, key0_, wave); \
    }                                                                                        \
    kb = smem + (it % kStages) * STAGE;                                                      \
  }

  if constexpr (FALLBACK) {
    // rows over the limit: offset = c max x, from a first pass over the scores
    float mx[kQT];
#pragma unroll
    for (int j = 0; j < kQT; ++j) mx[j] = kMasked;
    TileCursor c1 = cur;
    int valid, va = 0, vb = 0;
    const unsigned char* kb;
    VDN_FP8_FIRST_TILE(c1, va, vb)
    for (int it = 0; it < ntiles; ++it) {
      VDN_FP8_NEXT_TILE(it, c1, valid, va, vb, kb)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const i32x8 kf = kfrag(kb, u);
#pragma unroll
        for (int j = 0; j < kQT; ++j) {
          const f32x4 s = mfma8_scaled(kf, qf[j], f32x4{0.f, 0.f, 0.f, 0.f}, ekey, escale[j]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (32 * g + 4 * u + i < valid) mx[j] = fmaxf(mx[j], s[i]);
        }
      }
    }
    __syncthreads();            // every wave is done with the stages before they are reused
#pragma unroll
    for (int j = 0; j < kQT; ++j) {
      float m = fmaxf(mx[j], __shfl_xor(mx[j], 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      if (over[j]) moff[j] = m - kShift;
    }
  }

  f32x4 oacc[D / 16][kQT], lacc[kQT];
#pragma unroll
  for (int j = 0; j < kQT; ++j) {
    lacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) oacc[dt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const i32x8 ones = {(int)kOnes, (int)kOnes, (int)kOnes, (int)kOnes, (int)kOnes, (int)kOnes, (int)kOnes, (int)kOnes};

  int valid, va = 0, vb = 0;
  const unsigned char* kb;
  VDN_FP8_FIRST_TILE(cur, va, vb)
  for (int it = 0; it < ntiles; ++it) {
    VDN_FP8_NEXT_TILE(it, cur, valid, va, vb, kb)
    const unsigned char* vb = kb + K_BYTES;
    i32x8 pf[kQT];
    // scores and weights, kUG 16-key tiles at a time
#pragma unroll
    for (int up = 0; up < 8 / kUG; ++up) {
      i32x8 kf[kUG];
#pragma unroll
      for (int uu = 0; uu < kUG; ++uu) kf[uu] = kfrag(kb, kUG * up + uu);
      f32x4 s[kUG][kQT];
#pragma unroll
      for (int uu = 0; uu < kUG; ++uu)
#pragma unroll
        for (int j = 0; j < kQT; ++j)
          s[uu][j] = mfma8_scaled(kf[uu], qf[j], f32x4{-moff[j], -moff[j], -moff[j], -moff[j]}, ekey, escale[j]);
#pragma unroll
      for (int uu = 0; uu < kUG; ++uu) {
        const int u = kUG * up + uu;
        if (valid < kBK) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (32 * g + 4 * u + i >= valid)
#pragma unroll
              for (int j = 0; j < kQT; ++j) s[uu][j][i] = kMasked;
        }
#pragma unroll
        for (int j = 0; j < kQT; ++j) {
          float p[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(s[uu][j][i]);
          int wv = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
          wv = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wv, true);
          pf[j][u] = wv;
        }
      }
    }
    // O^T += V^T P^T and the normaliser (ones row) on the matrix cores
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const i32x8 vf = vfrag(vb, dt);
#pragma unroll
      for (int j = 0; j < kQT; ++j) oacc[dt][j] = mfma8(vf, pf[j], oacc[dt][j]);
    }
#pragma unroll
    for (int j = 0; j < kQT; ++j) lacc[j] = mfma8(ones, pf[j], lacc[j]);
  }

  // ---- normalise and store (bf16): lane holds channels 16 dt + 4 g + i of query l16 of tile j ----
#pragma unroll
  for (int j = 0; j < kQT; ++j) {
    const int n = n_base + 16 * j + l16;
    if (n >= nrows) continue;
    const float inv = 1.0f / (lacc[j][0] * sv);
    bf16_t* op = odst + (int64_t)n * H * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      __bf16 b4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) b4[i] = (__bf16)(oacc[dt][j][i] * inv);
      *reinterpret_cast<uint2*>(op + dt * 16 + g * 4) = __builtin_bit_cast(uint2, b4);
    }
  }
}

}  // namespace

int softmax_fp8_grid(const Shape& s, bool with_ctx) {
  const int QT = (s.N + kBQ - 1) / kBQ;
  const int nb = s.anchors ? (s.T > 1 ? 2 : 1) : 0;
  const int n_ctx_wg = with_ctx ? (s.n_ctx + kBQ - 1) / kBQ * s.H : 0;
  const int n_bnd_wg = nb * QT * s.H;
  const int n_int_wg = (s.T - nb) * QT * s.H;
  return n_ctx_wg + n_bnd_wg + 8 * ((n_int_wg + 7) / 8);
}

hipError_t launch_softmax_fp8(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st,
                              hipEvent_t after_first) {
  if (s.d != D) return hipErrorInvalidValue;
  Params P{};
  P.q = (const bf16_t*)in.q;
  P.qc = (const bf16_t*)in.ctx_q;
  P.k8 = b.k8;
  P.v8 = b.v8;
  P.o_s = (bf16_t*)b.os;
  P.oc = (bf16_t*)in.ctx_out;
  P.ranges = b.ranges;
  P.nranges = b.nranges;
  P.kmax = b.kmax;
  P.scale = b.scale8;
  P.flags = b.flags;
  P.T = s.T;
  P.N = s.N;
  P.H = s.H;
  P.n_ctx = s.n_ctx;
  P.Ls8 = s.Ls8;
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
  const int grid = softmax_fp8_grid(s, in.ctx_out != nullptr);
  const size_t smem = kStages * STAGE;
  (void)hipFuncSetAttribute((const void*)softmax_fp8_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  (void)hipFuncSetAttribute((const void*)softmax_fp8_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  hipLaunchKernelGGL(softmax_fp8_kernel<false>, dim3(grid), dim3(kWaves * 64), smem, st, P);
  if (after_first) (void)hipEventRecord(after_first, st);
  hipLaunchKernelGGL(softmax_fp8_kernel<true>, dim3(grid), dim3(kWaves * 64), smem, st, P);
  return hipGetLastError();
}

}  // namespace vdn
