// Block-sparse window softmax of the VDN layer on CDNA4 matrix cores (bf16 in, fp32 accumulate).
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Local Softmax and
// Long-Range Linear Memory": a video query in chunk c attends, with one softmax, to the text keys,
// the keys of chunks c-1, c, c+1 and the two boundary anchor frames (boundary query frames attend
// to every frame).  The key set of a query frame is at most four contiguous ranges of the packed
// key space (built on the host), so the kernel is a flash-style attention over a range list.
//
// Work decomposition
//   * one workgroup = 256 queries of one frame and one head; 4 waves x 64 queries;
//   * key tiles of 64 keys are loaded straight from global memory into LDS (global_load_lds,
//     double buffered; K as [key][d], V transposed as [d][key], both XOR-swizzled so the 16-byte
//     fragment reads are bank-conflict free) and processed as two 32-key halves;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys as rows, queries as columns) so that each
//     lane ends up holding 16 consecutive keys of one query -- the row permutation used when the
//     K fragments are read makes those keys contiguous;  O^T += V^T P^T with the same instruction,
//     P taken straight from the S^T registers (no LDS round trip);
//   * online softmax in base 2 with a lazy rescale: the running reference max only moves when a
//     tile's max exceeds it by more than 8 (a factor 256), so the O rescale (128 values per lane)
//     is skipped for almost every tile; exactness is unaffected since the final division uses the
//     same reference;
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

constexpr int kBK = 64;        // keys per tile
constexpr int kWaves = 4;
constexpr int kQW = 64;        // queries per wave
constexpr int kBQ = kWaves * kQW;
constexpr float kRescaleThreshold = 8.0f;   // log2 units
constexpr float kMasked = -1.0e30f;

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

typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;
constexpr int kVmcntZero = 0x0F70;   // s_waitcnt vmcnt(0), other counters untouched

template <int D>
__global__ __launch_bounds__(256, 1) void softmax_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kp, const bf16_t* __restrict__ vt,
    bf16_t* __restrict__ o_s, const int* __restrict__ ranges, const int* __restrict__ nranges, int T, int N, int H,
    int64_t Lk, int QT, int n_bnd_wg, int n_int_frames, int first_int_frame, int per_xcd, int n_int_wg,
    float c_log2) {
  using SM = Smem<D>;
  constexpr int KS = D / 16;          // k-steps of the QK^T contraction
  constexpr int DT = D / 32;          // 32-row d tiles of O^T
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  // ---- workgroup -> (head, frame, query tile) ----
  const int w = blockIdx.x;
  int h, t, qt;
  if (w < n_bnd_wg) {
    qt = w % QT;
    const int rest = w / QT;
    const int nb = n_bnd_wg / (QT * H);
    const int bi = rest % nb;
    h = rest / nb;
    t = bi == 0 ? 0 : T - 1;
  } else {
    const int wp = w - n_bnd_wg;
    const int x = w & 7;
    const int L = x * per_xcd + (wp >> 3);
    if (L >= n_int_wg) return;
    qt = L % QT;
    const int rest = L / QT;
    t = first_int_frame + rest % n_int_frames;
    h = rest / n_int_frames;
  }

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hl = lane >> 5;

  // ---- Q fragments (B operand of S^T = K Q^T): query = l32 (+32 qs), d = ks*16 + hl*8 .. +8 ----
  bf16x8 qf[2][KS];
  const int n_base = qt * kBQ + wave * kQW;
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int n = n_base + qs * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 val = {0, 0, 0, 0};
      if (n < N) val = *reinterpret_cast<const u32x4*>(q + (((int64_t)t * N + n) * H + h) * D + ks * 16 + hl * 8);
      qf[qs][ks] = as_bf16x8(val);
    }
  }

  // ---- key tiles: flatten the range list ----
  const int nr = nranges[t];
  int rs[kMaxRanges], re[kMaxRanges], rtiles[kMaxRanges];
  int ntiles = 0;
#pragma unroll
  for (int r = 0; r < kMaxRanges; ++r) {
    rs[r] = r < nr ? ranges[t * 2 * kMaxRanges + 2 * r] : 0;
    re[r] = r < nr ? ranges[t * 2 * kMaxRanges + 2 * r + 1] : 0;
    rtiles[r] = r < nr ? (re[r] - rs[r] + kBK - 1) / kBK : 0;
    ntiles += rtiles[r];
  }
  auto tile_at = [&](int it, int& key0, int& valid) {
    int r = 0;
#pragma unroll
    for (int rr = 0; rr < kMaxRanges - 1; ++rr)
      if (r == rr && it >= rtiles[rr]) { it -= rtiles[rr]; r = rr + 1; }
    int s0 = rs[0], e0 = re[0];
#pragma unroll
    for (int rr = 1; rr < kMaxRanges; ++rr)
      if (r == rr) { s0 = rs[rr]; e0 = re[rr]; }
    key0 = s0 + it * kBK;
    valid = min(kBK, e0 - key0);
  };

  const bf16_t* kh = kp + (int64_t)h * Lk * D;
  const bf16_t* vh = vt + (int64_t)h * D * Lk;

  // Direct global -> LDS tile loads (global_load_lds_dwordx4): one instruction of a wave fills 1 KB
  // of LDS, lane l writing bytes [16 l, 16 l + 16).  Each lane therefore fetches the global chunk
  // whose swizzled LDS position is its own.  Keys past the key space are clamped to its last
  // chunk (finite data; such keys are masked).
  constexpr int K_INSTR = Smem<D>::K_BYTES / 1024 / kWaves;     // per wave
  constexpr int V_INSTR = Smem<D>::V_BYTES / 1024 / kWaves;
  constexpr int K_ROWS_PER_KB = 1024 / (D * 2);
  auto issue_tile = [&](int key0, int stage) {
    unsigned char* kb = smem + stage * SM::STAGE;
    unsigned char* vb = kb + SM::K_BYTES;
#pragma unroll
    for (int i = 0; i < K_INSTR; ++i) {
      const int blk = i * kWaves + wave;
      const int row = blk * K_ROWS_PER_KB + lane / SM::KCH;
      const int c = (lane % SM::KCH) ^ k_swz<D>(row);
      int64_t j = key0 + row;
      j = j < Lk ? j : Lk - 1;
      __builtin_amdgcn_global_load_lds((gptr_t)(kh + j * D + c * 8), (lptr_t)(kb + blk * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < V_INSTR; ++i) {
      const int blk = i * kWaves + wave;
      const int row = blk * 8 + lane / 8;
      const int c = (lane % 8) ^ v_swz(row);
      int64_t j = key0 + c * 8;
      j = j + 8 <= Lk ? j : Lk - 8;
      __builtin_amdgcn_global_load_lds((gptr_t)(vh + (int64_t)row * Lk + j), (lptr_t)(vb + blk * 1024), 16, 0, 0);
    }
  };

  f32x16 oacc[2][DT];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[qs][dt][i] = 0.f;
  float mref[2] = {-INFINITY, -INFINITY};
  float lsum[2] = {0.f, 0.f};

  // row of the K tile that this lane feeds as MFMA row l32 (see header): key 16*h + 4*a + b
  const int krow = ((l32 >> 2) & 1) * 16 + (l32 >> 3) * 4 + (l32 & 3);

  {
    int key0, valid;
    tile_at(0, key0, valid);
    issue_tile(key0, 0);
  }
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int stage = it & 1;
    int key0, valid;
    tile_at(it, key0, valid);
    if (it + 1 < ntiles) {
      int nkey0, nvalid;
      tile_at(it + 1, nkey0, nvalid);
      issue_tile(nkey0, stage ^ 1);
    }
    const unsigned char* kb = smem + stage * SM::STAGE;
    const unsigned char* vb = kb + SM::K_BYTES;

#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {       // two 32-key halves of the tile
      // ---- S^T = K Q^T for 32 keys x 64 queries ----
      f32x16 sacc[2];
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[qs][i] = 0.f;
      const int row = kt * 32 + krow;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = ks * 2 + hl;
        const bf16x8 kf = as_bf16x8(*reinterpret_cast<const u32x4*>(kb + row * (D * 2) + ((c ^ k_swz<D>(row)) * 16)));
#pragma unroll
        for (int qs = 0; qs < 2; ++qs)
          sacc[qs] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qs][ks], sacc[qs], 0, 0, 0);
      }
      // ---- mask the tail of a partial tile ----
      if (valid < kBK) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kl = kt * 32 + hl * 16 + i;
          if (kl >= valid) { sacc[0][i] = kMasked; sacc[1][i] = kMasked; }
        }
      }
      // ---- online softmax: this lane holds 16 keys of 2 queries; the other 16 are in lane ^ 32 ----
      float mxc[2];
      bool need = false;
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        float mx = sacc[qs][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[qs][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        mxc[qs] = mx * c_log2;
        need |= mxc[qs] > mref[qs] + kRescaleThreshold;
      }
      if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
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
      bf16x8 pf[2][2];     // [qs][k-step]
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        float ls = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = exp2f(fmaf(sacc[qs][i], c_log2, -mref[qs]));
          ls += p;
          pf[qs][i >> 3][i & 7] = (__bf16)p;
        }
        lsum[qs] += ls;
      }
      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int vrow = dt * 32 + l32;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int c = kt * 4 + hl * 2 + s;
          const bf16x8 vf = as_bf16x8(*reinterpret_cast<const u32x4*>(vb + vrow * (kBK * 2) + ((c ^ v_swz(vrow)) * 16)));
#pragma unroll
          for (int qs = 0; qs < 2; ++qs)
            oacc[qs][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qs][s], oacc[qs][dt], 0, 0, 0);
        }
      }
    }

    __builtin_amdgcn_s_waitcnt(kVmcntZero);
    __syncthreads();
  }

  // ---- normalise and store o_s (bf16) ----
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const float tot = lsum[qs] + __shfl_xor(lsum[qs], 32);
    const float inv = 1.0f / tot;
    const int n = n_base + qs * 32 + l32;
    if (n < N) {
      bf16_t* op = o_s + (((int64_t)t * N + n) * H + h) * D;
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
  const int QT = (s.N + kBQ - 1) / kBQ;
  const bool two_bnd = s.anchors && s.T > 1;
  const int nb = s.anchors ? (two_bnd ? 2 : 1) : 0;
  const int n_int_frames = s.T - nb;
  const int first_int = s.anchors ? 1 : 0;
  const int n_bnd_wg = nb * QT * s.H;
  const int n_int_wg = n_int_frames * QT * s.H;
  const int per_xcd = (n_int_wg + 7) / 8;
  const int grid = n_bnd_wg + 8 * per_xcd;
  const size_t smem = 2 * Smem<D>::STAGE;
  const float c_log2 = 1.4426950408889634f / sqrtf((float)D);
  hipLaunchKernelGGL(softmax_mfma_kernel<D>, dim3(grid), dim3(256), smem, st, (const bf16_t*)in.q, b.kp, b.vt,
                     (bf16_t*)b.os, b.ranges, b.nranges, s.T, s.N, s.H, s.Lk, QT, n_bnd_wg, n_int_frames, first_int,
                     per_xcd, n_int_wg, c_log2);
}

}  // namespace

hipError_t launch_softmax_mfma(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st) {
  if (s.d == 128) {
    (void)hipFuncSetAttribute((const void*)softmax_mfma_kernel<128>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              2 * Smem<128>::STAGE);
    launch_t<128>(s, in, b, st);
  } else {
    (void)hipFuncSetAttribute((const void*)softmax_mfma_kernel<64>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              2 * Smem<64>::STAGE);
    launch_t<64>(s, in, b, st);
  }
  return hipGetLastError();
}

}  // namespace vdn
