// X^T Y sums of the backward on CDNA4 matrix cores (bf16 plans, d in {64, 128}).
//
// "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Gating the Softmax and
// Linear Branch Outputs": the gradients of the gate and projection weights are sums over every
// (token, head) row of outer products, dW = sum_rows x^T y, and the readout of the linear branch
// (section "Video Delta Attention: A Frame-Wise Solution") needs the same sum over the rows of each
// chunk, sum do_l q^T.  Each block sums the rows of one share of a row segment into a d x d partial
// (the reduce kernel of the generic path then adds the shares in order).
//
// Per 64-row tile the block stages X and Y in LDS, row-major with the 16-byte chunks of row r
// XOR-swizzled by 4 (r % 4) (d = 128) or 4 ((r / 2) % 2) (d = 64); the MFMA operands, eight
// consecutive rows of one column per lane, come from ds_read_b64_tr_b16 transposed reads (lane j of
// each 16-lane group gets the four values at column j of the 4 x 16 block its group addresses).
// v_mfma_f32_32x32x16_bf16, four waves, wave w owning output rows [32 MT (w % 2), +32 MT) and
// columns [32 NT (w / 2), +32 NT), MT = NT = d / 64.  An fp32 operand enters as bf16 hi + lo parts
// (three products: hi hi, hi lo, lo hi), so the sums keep about 2^-16 relative accuracy; bf16
// operands are exact.  The next tile's rows are loaded into registers while the current one is
// multiplied.
#include <type_traits>

#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 lds_bf16x4;

constexpr int kTU = 64;          // rows per tile
constexpr int kThreads = 256;

template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return 4 * (r & 3);
  else return 4 * ((r >> 1) & 1);
}

__device__ __forceinline__ bf16x4 tr_read(const unsigned char* p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                        (__attribute__((address_space(3))) lds_bf16x4*)(p)));
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// eight consecutive elements of one row, as loaded from global memory
template <typename T>
struct Chunk;
template <>
struct Chunk<bf16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void put(unsigned char* hi, unsigned char*) const { *reinterpret_cast<uint4*>(hi) = v; }
};
template <>
struct Chunk<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void put(unsigned char* hi, unsigned char* lo) const {
    const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    bf16x8 h, l;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const __bf16 t = (__bf16)x[i];
      h[i] = t;
      l[i] = (__bf16)(x[i] - (float)t);
    }
    *reinterpret_cast<bf16x8*>(hi) = h;
    *reinterpret_cast<bf16x8*>(lo) = l;
  }
};

template <int D, typename TX, typename TY>
__global__ __launch_bounds__(kThreads) void xty_mfma_kernel(const TX* __restrict__ x, const TY* __restrict__ y,
                                                            const Segment* __restrict__ segs, int H, int splits,
                                                            float* __restrict__ partial) {
  constexpr bool XF = std::is_same<TX, float>::value, YF = std::is_same<TY, float>::value;
  constexpr int ROW = 2 * D, TILE = kTU * ROW, CH = D / 8;
  constexpr int PER = kTU * CH / kThreads;         // chunks per thread per array and tile
  constexpr int MT = D / 64, NT = D / 64;
  // LDS: X hi, Y hi, then X lo and / or Y lo
  __shared__ __attribute__((aligned(16))) unsigned char smem[(2 + XF + YF) * TILE];
  unsigned char* xh = smem;
  unsigned char* yh = smem + TILE;
  unsigned char* xl = smem + 2 * TILE;
  unsigned char* yl = smem + (2 + XF) * TILE;

  const Segment sg = segs[blockIdx.x];
  const int split = blockIdx.y;
  const int heads = sg.head < 0 ? H : 1;
  const int64_t total = (int64_t)sg.nrows * heads;            // (row, head) pairs of the segment
  const int64_t per = (total + splits - 1) / splits;
  const int64_t p0 = (int64_t)split * per, p1 = min(total, p0 + per);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  Chunk<TX> cx[PER];
  Chunk<TY> cy[PER];
  auto load = [&](int64_t base) {
#pragma unroll
    for (int s = 0; s < PER; ++s) {
      const int e = tid + s * kThreads, r = e / CH, c = e % CH;
      const int64_t p = base + r;
      if (p < p1) {
        const int64_t row = sg.row0 + p / heads;
        const int hh = sg.head < 0 ? (int)(p % heads) : sg.head;
        const int64_t off = (row * H + hh) * D + c * 8;
        cx[s].load(x + off);
        cy[s].load(y + off);
      } else {
        cx[s].zero();
        cy[s].zero();
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int s = 0; s < PER; ++s) {
      const int e = tid + s * kThreads, r = e / CH, c = e % CH;
      const int o = r * ROW + ((c ^ swz<D>(r)) << 4);
      cx[s].put(xh + o, xl + o);
      cy[s].put(yh + o, yl + o);
    }
  };

  // transposed-read lane offsets: lane (g = lane / 16, i = lane % 16) addresses row
  // 8 (g / 2) + (i / 4) (+ 4 for the second read) and column 16 (g % 2) + 4 (i % 4) of a
  // 16-row x 32-column fragment block
  const int g = lane >> 4, li = lane & 15;
  const int tr_row = 8 * (g >> 1) + (li >> 2);
  const int tr_col = 16 * (g & 1) + 4 * (li & 3);
  auto tr_off = [&](int c0) {
    const int c = c0 + tr_col;
    return tr_row * ROW + (((c >> 3) ^ swz<D>(tr_row)) << 4) + (c & 7) * 2;
  };
  const int xg = wave & 1, yg = wave >> 1;
  int xoff[MT], yoff[NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xoff[mt] = tr_off((xg * MT + mt) * 32);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) yoff[nt] = tr_off((yg * NT + nt) * 32);

  f32x16 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.f;

  if (p0 < p1) load(p0);
  for (int64_t base = p0; base < p1; base += kTU) {
    __syncthreads();                       // the previous tile has been consumed
    stash();
    __syncthreads();
    if (base + kTU < p1) load(base + kTU);
#pragma unroll
    for (int ks = 0; ks < kTU / 16; ++ks) {
      const int kb = ks * 16 * ROW;
      bf16x8 yf[NT][1 + YF];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        yf[nt][0] = cat(tr_read(yh + kb + yoff[nt]), tr_read(yh + kb + yoff[nt] + 4 * ROW));
        if constexpr (YF) yf[nt][YF] = cat(tr_read(yl + kb + yoff[nt]), tr_read(yl + kb + yoff[nt] + 4 * ROW));
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 xf = cat(tr_read(xh + kb + xoff[mt]), tr_read(xh + kb + xoff[mt] + 4 * ROW));
        bf16x8 xlf;
        if constexpr (XF) xlf = cat(tr_read(xl + kb + xoff[mt]), tr_read(xl + kb + xoff[mt] + 4 * ROW));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf, yf[nt][0], acc[mt][nt], 0, 0, 0);
          if constexpr (YF) acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf, yf[nt][YF], acc[mt][nt], 0, 0, 0);
          if constexpr (XF) acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xlf, yf[nt][0], acc[mt][nt], 0, 0, 0);
        }
      }
    }
  }

  // acc[mt][nt][r]: row 32 (xg MT + mt) + 8 (r / 4) + 4 (lane / 32) + r % 4, column
  // 32 (yg NT + nt) + lane % 32
  float* out = partial + ((int64_t)blockIdx.x * splits + split) * D * D;
  const int l32 = lane & 31, hl = lane >> 5;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = (xg * MT + mt) * 32 + 8 * (r / 4) + 4 * hl + (r % 4);
        const int j = (yg * NT + nt) * 32 + l32;
        out[(int64_t)i * D + j] = acc[mt][nt][r];
      }
}

template <int D, typename TX, typename TY>
hipError_t launch_t(const TX* x, const TY* y, const Segment* segs, int nseg, int splits, int H, float* partial,
                    hipStream_t st) {
  xty_mfma_kernel<D, TX, TY><<<dim3(nseg, splits), kThreads, 0, st>>>(x, y, segs, H, splits, partial);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_xty_mfma(int d, const void* x, bool x_f32, const void* y, bool y_f32, const Segment* segs, int nseg,
                           int splits, int H, float* partial, hipStream_t st) {
  if (x_f32 == y_f32) return hipErrorInvalidValue;   // one operand fp32, the other bf16
  if (d == 128) {
    if (x_f32) return launch_t<128>((const float*)x, (const bf16_t*)y, segs, nseg, splits, H, partial, st);
    return launch_t<128>((const bf16_t*)x, (const float*)y, segs, nseg, splits, H, partial, st);
  }
  if (d == 64) {
    if (x_f32) return launch_t<64>((const float*)x, (const bf16_t*)y, segs, nseg, splits, H, partial, st);
    return launch_t<64>((const bf16_t*)x, (const float*)y, segs, nseg, splits, H, partial, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace vdn
