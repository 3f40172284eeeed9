// Merge backward on CDNA4 matrix cores (bf16 plans, d in {64, 128}).
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Gating the Softmax and
// Linear Branch Outputs": out = (g_s * o_s) Wp0 + (g_l * r) Wp1 with g = sigmoid(q Wg) and
// r = RMSNorm(o_l), o_l = S q (section "Video Delta Attention: A Frame-Wise Solution").  Per
// (token, head) row the transpose needs eight d x d matrix-vector products:
//   o_l = S q,  a_s = Wg0^T q,  a_l = Wg1^T q,  dx_s = Wp0 dout,  dx_l = Wp1 dout,
//   dq  = Wg0 dz_s + Wg1 dz_l + S^T do_l,
// with, elementwise, do_s = g_s dx_s, dz_s = dx_s o_s g_s (1 - g_s), dr = g_l dx_l,
// dz_l = dx_l r g_l (1 - g_l), do_l = (dr - r mean(r dr)) / rms, and D = rowsum(do_s o_s).
//
// Layout: one workgroup = 128 rows (tokens) of one frame and head, 8 waves x 16 tokens.  Every
// product is computed channels x tokens on v_mfma_f32_16x16x32_bf16 with the d x d matrix as the
// A operand, read from LDS, and the token vectors as the B operand held in registers.  The rows of
// every matrix image are permuted so that output channel tile 2 ks + u, row 4 g + i is channel
// 32 ks + 8 g + 4 u + i: a lane's accumulators then hold exactly the eight consecutive channels
// per k-step that the next product's B operand needs, so results feed the following products
// straight from registers.  The matrix images (weights once, the chunk states per slot and head)
// are written by a small kernel in that row order, XOR-swizzled by 16-byte chunk, and copied into
// LDS with global_load_lds, four images at a time.
//
// The same machinery serves the token gradients of the linear branch (section "Video Delta
// Attention: A Frame-Wise Solution"): per written token, with G = dA + dA^T and dB of its frame (or of
// the text, at beta / 2), dk += beta (G k + dB^T v), dv += beta dB k, dbeta += k^T dA k + v^T dB k,
// i.e. three d x d products per row with the images G, dB^T and dB.
//
// Precision: q, dout, o_s and the weights are bf16 inputs, exact as MFMA operands.  The fp32
// operands (the state S, dz_s, dz_l, do_l) enter as bf16 hi + lo pairs, so every product is exact
// to about 2^-16 relative; sums accumulate in fp32.
#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

constexpr int kWaves = 8;
constexpr int kTok = 16 * kWaves;           // tokens per workgroup
constexpr int kVmcntZero = 0x0F70;          // s_waitcnt vmcnt(0), other counters untouched
constexpr int kWeightImages = 6;            // Wg0^T, Wg1^T, Wp0, Wp1, Wg0, Wg1
constexpr int kStateImages = 4;             // S hi, S lo, S^T hi, S^T lo per (slot, head)

// image row p holds matrix row perm(p) (see the header)
__device__ __forceinline__ int perm_row(int p) {
  const int ct = p >> 4, r = p & 15;
  return 32 * (ct >> 1) + 8 * (r >> 2) + 4 * (ct & 1) + (r & 3);
}
// byte offset of 16-byte chunk c of image row p
template <int D>
__device__ __forceinline__ int img_off(int p, int c) {
  return p * (D * 2) + ((c ^ (p & 7)) * 16);
}

__device__ __forceinline__ uint16_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// Images: blockIdx.x < 6 the weights, then 4 per (slot, head) of the states S = S_fwd + S_rev.
template <int D>
__global__ __launch_bounds__(256) void merge_images_kernel(const bf16_t* __restrict__ gate_w,
                                                           const bf16_t* __restrict__ proj_w,
                                                           const float* __restrict__ states, int H, int Nc,
                                                           uint16_t* __restrict__ img) {
  constexpr int64_t DD = (int64_t)D * D;
  const int m = blockIdx.x;
  unsigned char* dst = reinterpret_cast<unsigned char*>(img + (int64_t)m * DD);
  const float *sf = nullptr, *sr = nullptr;
  int kind = 0;
  if (m >= kWeightImages) {
    const int idx = (m - kWeightImages) / kStateImages;   // slot * H + head
    kind = (m - kWeightImages) % kStateImages;
    const int slot = idx / H, h = idx % H;
    sf = states + ((int64_t)slot * H + h) * DD;
    sr = states + ((int64_t)(Nc + 1 + slot) * H + h) * DD;
  }
  for (int e = threadIdx.x; e < D * (D / 8); e += 256) {
    const int p = e / (D / 8), c = e % (D / 8);
    const int j = perm_row(p);
    uint16_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = 8 * c + i;
      if (m < kWeightImages) {
        // A(j, k) of each weight product (gate_w, proj_w are [2][in][out])
        int64_t src;
        const bf16_t* w;
        switch (m) {
          case 0: w = gate_w; src = (int64_t)k * D + j; break;        // Wg0^T
          case 1: w = gate_w + DD; src = (int64_t)k * D + j; break;   // Wg1^T
          case 2: w = proj_w; src = (int64_t)j * D + k; break;        // Wp0
          case 3: w = proj_w + DD; src = (int64_t)j * D + k; break;   // Wp1
          case 4: w = gate_w; src = (int64_t)j * D + k; break;        // Wg0
          default: w = gate_w + DD; src = (int64_t)j * D + k; break;  // Wg1
        }
        v[i] = w[src];
      } else {
        const int64_t src = kind < 2 ? (int64_t)j * D + k : (int64_t)k * D + j;   // S or S^T
        const float x = sf[src] + sr[src];
        const uint16_t hi = bf16_bits(x);
        v[i] = (kind & 1) ? bf16_bits(x - to_f32(hi)) : hi;
      }
    }
    *reinterpret_cast<uint4*>(dst + img_off<D>(p, c)) = *reinterpret_cast<const uint4*>(v);
  }
}

// Copy one image into LDS buffer `buf` (every wave issues its share).
template <int D>
__device__ __forceinline__ void dma_image(const unsigned char* src, unsigned char* smem, int buf, int wave, int lane) {
  constexpr int kBytes = D * D * 2;
#pragma unroll
  for (int i = 0; i < kBytes / (kWaves * 1024); ++i) {
    const int off = (i * kWaves + wave) * 1024;
    __builtin_amdgcn_global_load_lds((gptr_t)(src + off + lane * 16), (lptr_t)(smem + buf * kBytes + off), 16, 0, 0);
  }
}

// acc[ct] += A(image in LDS buffer buf) B, B given per k-step as the lane's eight channels
template <int D>
__device__ __forceinline__ void product(const unsigned char* smem, int buf, const bf16x8 (&b)[D / 32],
                                        f32x4 (&acc)[D / 16], int l16, int g) {
  const unsigned char* a = smem + buf * (D * D * 2);
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct) {
      const int p = 16 * ct + l16;
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(a + img_off<D>(p, 4 * ks + g));
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b[ks], acc[ct], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);   // at most one k-step of A fragments in registers
  }
}

template <int D>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[D / 16]) {
#pragma unroll
  for (int ct = 0; ct < D / 16; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// the lane's value e (0..7) of k-step ks: channel 32 ks + 8 g + e
template <int D>
__device__ __forceinline__ float at(const f32x4 (&acc)[D / 16], int ks, int e) {
  return acc[2 * ks + (e >> 2)][e & 3];
}

// fp32 values (as accumulators) -> bf16 hi and lo B operands
template <int D>
__device__ __forceinline__ void split(const f32x4 (&x)[D / 16], bf16x8 (&hi)[D / 32], bf16x8 (&lo)[D / 32]) {
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = at<D>(x, ks, e);
      const __bf16 h = (__bf16)v;
      hi[ks][e] = h;
      lo[ks][e] = (__bf16)(v - (float)h);
    }
}

// store the lane's 8 channels of each k-step (two 16-byte stores)
template <int D>
__device__ __forceinline__ void store_vec(float* __restrict__ dst, const f32x4 (&x)[D / 16], int g) {
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    *reinterpret_cast<f32x4*>(dst + 32 * ks + 8 * g) = x[2 * ks];
    *reinterpret_cast<f32x4*>(dst + 32 * ks + 8 * g + 4) = x[2 * ks + 1];
  }
}

template <int D>
__global__ __launch_bounds__(kWaves * 64) void merge_bwd_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ o_s, const bf16_t* __restrict__ dout,
    const uint16_t* __restrict__ img, float* __restrict__ dq, bf16_t* __restrict__ dos16, float* __restrict__ do_l,
    float* __restrict__ x_s, float* __restrict__ x_l, float* __restrict__ dz_s, float* __restrict__ dz_l,
    float* __restrict__ dsum, int T, int N, int C, int Nc, int H, int anchors) {
  constexpr int KS = D / 32, CT = D / 16;
  constexpr int64_t DD = (int64_t)D * D;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];   // four images
  const int t = blockIdx.y, h = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
  const int n = blockIdx.x * kTok + wave * 16 + l16;
  const bool ok = n < N;
  const int64_t row = ((int64_t)t * N + (ok ? n : 0)) * H + h;   // (token, head) row
  const bool bnd = anchors && (t == 0 || t == T - 1);
  const int slot = bnd ? Nc : t / C;
  const unsigned char* wimg = reinterpret_cast<const unsigned char*>(img);
  const unsigned char* simg = reinterpret_cast<const unsigned char*>(img + (kWeightImages + kStateImages * ((int64_t)slot * H + h)) * DD);
  constexpr int IMG = D * D * 2;

  // buffers: [Wg0^T, Wp0, S hi, S lo], then [Wg1^T, Wp1, Wg0, Wg1], then [S^T hi, S^T lo]
  dma_image<D>(wimg, smem, 0, wave, lane);
  dma_image<D>(wimg + 2 * IMG, smem, 1, wave, lane);
  dma_image<D>(simg, smem, 2, wave, lane);
  dma_image<D>(simg + IMG, smem, 3, wave, lane);
  bf16x8 qf[KS], df[KS], of[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int64_t e = row * D + 32 * ks + 8 * g;
    const bf16x8 z = {};
    qf[ks] = ok ? *reinterpret_cast<const bf16x8*>(q + e) : z;
    df[ks] = ok ? *reinterpret_cast<const bf16x8*>(dout + e) : z;
    of[ks] = ok ? *reinterpret_cast<const bf16x8*>(o_s + e) : z;
  }
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  __syncthreads();
  // softmax half: g_s = sigmoid(Wg0^T q), dx_s = Wp0 dout; do_s = g_s dx_s, x_s = g_s o_s,
  // dz_s = dx_s o_s g_s (1 - g_s) (stored at once; dz_s is kept for dq), D = rowsum(do_s o_s)
  f32x4 zs[CT];
  float dsm = 0.f;
  {
    f32x4 ga[CT], dx[CT];
    zero_acc<D>(ga);
    zero_acc<D>(dx);
    product<D>(smem, 0, qf, ga, l16, g);
    product<D>(smem, 1, df, dx, l16, g);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ct = 2 * ks + (e >> 2), i = e & 3;
        const float os = (float)of[ks][e], s_ = sigmoidf_(ga[ct][i]), x_ = dx[ct][i];
        const float dos = x_ * s_;
        dsm += dos * os;
        zs[ct][i] = x_ * os * s_ * (1.f - s_);
        dx[ct][i] = dos;
        ga[ct][i] = s_ * os;
      }
    if (ok) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {             // do_s in bf16 (the softmax transpose's operand)
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)at<D>(dx, ks, e);
        *reinterpret_cast<bf16x8*>(dos16 + row * D + 32 * ks + 8 * g) = v;
      }
      store_vec<D>(x_s + row * D, ga, g);
      store_vec<D>(dz_s + row * D, zs, g);
    }
  }
  dsm += __shfl_xor(dsm, 16);
  dsm += __shfl_xor(dsm, 32);
  if (ok && g == 0) dsum[row] = dsm;
  // o_l = S q and its RMS over the token's d channels (the four lanes l16 + 16 g hold a token)
  f32x4 r[CT];
  zero_acc<D>(r);
  product<D>(smem, 2, qf, r, l16, g);
  product<D>(smem, 3, qf, r, l16, g);
  float ss = 0.f;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) ss += r[ct][i] * r[ct][i];
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  const float rho = sqrtf(ss / D + 1e-6f);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) r[ct][i] = r[ct][i] / rho;
  __syncthreads();                                    // every wave is done with buffers 0-3
  dma_image<D>(wimg + IMG, smem, 0, wave, lane);      // Wg1^T
  dma_image<D>(wimg + 3 * IMG, smem, 1, wave, lane);  // Wp1
  dma_image<D>(wimg + 4 * IMG, smem, 2, wave, lane);  // Wg0
  dma_image<D>(wimg + 5 * IMG, smem, 3, wave, lane);  // Wg1
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  __syncthreads();
  // linear half: g_l = sigmoid(Wg1^T q), dx_l = Wp1 dout; dr = g_l dx_l, x_l = g_l r,
  // dz_l = dx_l r g_l (1 - g_l); do_l = (dr - r mean(r dr)) / rho
  f32x4 zl[CT], dl[CT];
  {
    f32x4 ga[CT];
    zero_acc<D>(ga);
    zero_acc<D>(dl);
    product<D>(smem, 0, qf, ga, l16, g);
    product<D>(smem, 1, df, dl, l16, g);
    float rdr = 0.f;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float l_ = sigmoidf_(ga[ct][i]), rv = r[ct][i], x_ = dl[ct][i];
        const float dr = x_ * l_;
        rdr += rv * dr;
        zl[ct][i] = x_ * rv * l_ * (1.f - l_);
        dl[ct][i] = dr;
        ga[ct][i] = l_ * rv;
      }
    if (ok) {
      store_vec<D>(x_l + row * D, ga, g);
      store_vec<D>(dz_l + row * D, zl, g);
    }
    rdr += __shfl_xor(rdr, 16);
    rdr += __shfl_xor(rdr, 32);
    rdr /= D;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) dl[ct][i] = (dl[ct][i] - r[ct][i] * rdr) / rho;
  }
  if (ok) store_vec<D>(do_l + row * D, dl, g);
  // dq = Wg0 dz_s + Wg1 dz_l + S^T do_l
  f32x4 acc[CT];
  zero_acc<D>(acc);
  {
    bf16x8 hi[KS], lo[KS];
    split<D>(zs, hi, lo);
    product<D>(smem, 2, hi, acc, l16, g);
    product<D>(smem, 2, lo, acc, l16, g);
    split<D>(zl, hi, lo);
    product<D>(smem, 3, hi, acc, l16, g);
    product<D>(smem, 3, lo, acc, l16, g);
  }
  __syncthreads();                                    // every wave is done with buffers 0-1
  dma_image<D>(simg + 2 * IMG, smem, 0, wave, lane);  // S^T hi
  dma_image<D>(simg + 3 * IMG, smem, 1, wave, lane);  // S^T lo
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  __syncthreads();
  {
    bf16x8 hi[KS], lo[KS];
    split<D>(dl, hi, lo);
    product<D>(smem, 0, hi, acc, l16, g);
    product<D>(smem, 0, lo, acc, l16, g);
    product<D>(smem, 1, hi, acc, l16, g);
  }
  if (ok) store_vec<D>(dq + row * D, acc, g);
}

// Token-gradient images: per (slot, head) six images, G hi, G lo, dB^T hi, dB^T lo, dB hi, dB lo
// (G = dA + dA^T is symmetric).  Boundary frames are never written and get no images.
constexpr int kTokImages = 6;

template <int D>
__global__ __launch_bounds__(256) void token_images_kernel(const float* __restrict__ gsym, const float* __restrict__ gdb,
                                                           int T, int H, int anchors, uint16_t* __restrict__ img) {
  constexpr int64_t DD = (int64_t)D * D;
  const int m = blockIdx.x % kTokImages, idx = blockIdx.x / kTokImages;   // idx = slot * H + head
  const int slot = idx / H;
  if (slot > 0 && anchors && (slot - 1 == 0 || slot - 1 == T - 1)) return;
  const float* src = (m < 2 ? gsym : gdb) + (int64_t)idx * DD;
  unsigned char* dst = reinterpret_cast<unsigned char*>(img + (int64_t)blockIdx.x * DD);
  for (int e = threadIdx.x; e < D * (D / 8); e += 256) {
    const int p = e / (D / 8), c = e % (D / 8);
    const int j = perm_row(p);
    uint16_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = 8 * c + i;
      const float x = (m == 2 || m == 3) ? src[(int64_t)k * D + j] : src[(int64_t)j * D + k];   // dB^T or G, dB
      const uint16_t hi = bf16_bits(x);
      v[i] = (m & 1) ? bf16_bits(x - to_f32(hi)) : hi;
    }
    *reinterpret_cast<uint4*>(dst + img_off<D>(p, c)) = *reinterpret_cast<const uint4*>(v);
  }
}

// one workgroup = 128 tokens of one slot (0: text, f + 1: frame f) and head, 8 waves x 16 tokens
template <int D>
__global__ __launch_bounds__(kWaves * 64) void token_grads_mfma_kernel(
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const float* __restrict__ beta,
    const bf16_t* __restrict__ text_kv, const uint16_t* __restrict__ img, int T, int N, int H, int n_text,
    int n_ctx, int anchors, float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dbeta,
    float* __restrict__ dtext_kv) {
  constexpr int KS = D / 32, CT = D / 16;
  constexpr int64_t DD = (int64_t)D * D;
  constexpr int IMG = D * D * 2;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];   // four images
  const int slot = blockIdx.y, h = blockIdx.z;
  if (slot > 0 && anchors && (slot - 1 == 0 || slot - 1 == T - 1)) return;
  const int U = slot == 0 ? n_text : N;
  if ((int)blockIdx.x * kTok >= U) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
  const int u = blockIdx.x * kTok + wave * 16 + l16;
  const bool ok = u < U;
  const float wscale = slot == 0 ? 0.5f : 1.0f;
  const int64_t tok0 = slot == 0 ? 0 : (int64_t)(slot - 1) * N;
  const bf16_t* kb = slot == 0 ? text_kv : k;
  const bf16_t* vb = slot == 0 ? text_kv + (int64_t)n_ctx * H * D : v;   // V half of [2][n_ctx][H][d]
  float* dkb = slot == 0 ? dtext_kv : dk;
  float* dvb = slot == 0 ? dtext_kv + (int64_t)n_ctx * H * D : dv;
  const int64_t brow0 = slot == 0 ? 0 : n_text + tok0;
  const int64_t off = ((tok0 + (ok ? u : 0)) * H + h) * D;
  const unsigned char* timg = reinterpret_cast<const unsigned char*>(img + (int64_t)kTokImages * ((int64_t)slot * H + h) * DD);

  dma_image<D>(timg, smem, 0, wave, lane);            // G hi
  dma_image<D>(timg + IMG, smem, 1, wave, lane);      // G lo
  dma_image<D>(timg + 2 * IMG, smem, 2, wave, lane);  // dB^T hi
  dma_image<D>(timg + 3 * IMG, smem, 3, wave, lane);  // dB^T lo
  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 z = {};
    kf[ks] = ok ? *reinterpret_cast<const bf16x8*>(kb + off + 32 * ks + 8 * g) : z;
    vf[ks] = ok ? *reinterpret_cast<const bf16x8*>(vb + off + 32 * ks + 8 * g) : z;
  }
  const float wr = ok ? wscale * beta[(brow0 + u) * H + h] : 0.f;
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  __syncthreads();
  f32x4 g1[CT], g2[CT];
  zero_acc<D>(g1);
  zero_acc<D>(g2);
  product<D>(smem, 0, kf, g1, l16, g);                // G k
  product<D>(smem, 1, kf, g1, l16, g);
  product<D>(smem, 2, vf, g2, l16, g);                // dB^T v
  product<D>(smem, 3, vf, g2, l16, g);
  __syncthreads();                                    // every wave is done with buffers 0-3
  dma_image<D>(timg + 4 * IMG, smem, 0, wave, lane);  // dB hi
  dma_image<D>(timg + 5 * IMG, smem, 1, wave, lane);  // dB lo
  // dk += beta (G k + dB^T v); the k^T dA k part of dbeta is k . (G k) / 2
  float part = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ct = 2 * ks + (e >> 2), i = e & 3;
      part += 0.5f * (float)kf[ks][e] * g1[ct][i];
      g1[ct][i] = wr * (g1[ct][i] + g2[ct][i]);
    }
  if (ok) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        f32x4* p = reinterpret_cast<f32x4*>(dkb + off + 32 * ks + 8 * g + 4 * hlf);
        *p += g1[2 * ks + hlf];
      }
  }
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  __syncthreads();
  f32x4 gv[CT];
  zero_acc<D>(gv);
  product<D>(smem, 0, kf, gv, l16, g);                // dB k
  product<D>(smem, 1, kf, gv, l16, g);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ct = 2 * ks + (e >> 2), i = e & 3;
      part += (float)vf[ks][e] * gv[ct][i];
      gv[ct][i] *= wr;
    }
  if (ok) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        f32x4* p = reinterpret_cast<f32x4*>(dvb + off + 32 * ks + 8 * g + 4 * hlf);
        *p += gv[2 * ks + hlf];
      }
  }
  part += __shfl_xor(part, 16);
  part += __shfl_xor(part, 32);
  if (ok && g == 0) dbeta[(brow0 + u) * H + h] += wscale * part;
}

template <int D>
hipError_t launch_tok_t(const Shape& s, const Inputs& in, const BwdBuffers& w, const BwdOutputs& o, hipStream_t st) {
  token_images_kernel<D><<<kTokImages * (s.T + 1) * s.H, 256, 0, st>>>(w.gsym, w.gdb, s.T, s.H, s.anchors, w.mimg);
  constexpr size_t sm = (size_t)4 * D * D * 2;
  (void)hipFuncSetAttribute((const void*)token_grads_mfma_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)sm);
  const int U = s.N > s.n_text ? s.N : s.n_text;
  token_grads_mfma_kernel<D><<<dim3((U + kTok - 1) / kTok, s.T + 1, s.H), kWaves * 64, sm, st>>>(
      (const bf16_t*)in.k, (const bf16_t*)in.v, in.beta, (const bf16_t*)in.text_kv, w.mimg, s.T, s.N, s.H, s.n_text,
      s.n_ctx, s.anchors, o.dk, o.dv, o.dbeta, o.dtext_kv);
  return hipGetLastError();
}

template <int D>
hipError_t launch_t(const Shape& s, const Inputs& in, const Buffers& b, const BwdBuffers& w, const BwdOutputs& o,
                    hipStream_t st) {
  const int nimg = kWeightImages + kStateImages * (s.Nc + 1) * s.H;
  merge_images_kernel<D><<<nimg, 256, 0, st>>>((const bf16_t*)in.gate_w, (const bf16_t*)in.proj_w, b.states, s.H,
                                               s.Nc, w.mimg);
  constexpr size_t sm = (size_t)4 * D * D * 2;
  (void)hipFuncSetAttribute((const void*)merge_bwd_mfma_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  merge_bwd_mfma_kernel<D><<<dim3((s.N + kTok - 1) / kTok, s.T, s.H), kWaves * 64, sm, st>>>(
      (const bf16_t*)in.q, (const bf16_t*)b.os, (const bf16_t*)w.dout, w.mimg, o.dq, w.dos16, w.do_l, w.x_s, w.x_l,
      w.dz_s, w.dz_l, w.dsum, s.T, s.N, s.C, s.Nc, s.H, s.anchors);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_token_grads_mfma(const Shape& s, const Inputs& in, const BwdBuffers& w, const BwdOutputs& o,
                                   hipStream_t st) {
  if (s.d == 128) return launch_tok_t<128>(s, in, w, o, st);
  if (s.d == 64) return launch_tok_t<64>(s, in, w, o, st);
  return hipErrorInvalidValue;
}

hipError_t launch_merge_bwd_mfma(const Shape& s, const Inputs& in, const Buffers& b, const BwdBuffers& w,
                                 const BwdOutputs& o, hipStream_t st) {
  if (s.d == 128) return launch_t<128>(s, in, b, w, o, st);
  if (s.d == 64) return launch_t<64>(s, in, b, w, o, st);
  return hipErrorInvalidValue;
}

}  // namespace vdn
