// Allocation-free layer forward: the stages of vdn_forward on a workspace held in one static device
// array, for callers that cannot allocate device memory (code under HIP graph capture, serving
// loops that must not call hipMalloc).  The library calls no allocating routine here: no
// hipMalloc, no hipFree, no plan.
//
// The array is the same on every call on one GPU and keeps the previous call's contents, so each
// call first rebuilds what a plan sets up once at creation: the key-range table of the softmax
// branch (from the frame rules of "Video DeltaNet: Near-Lossless Hybrid Attention for Video
// Models", section "Local Softmax and Long-Range Linear Memory") and the tile of zero keys past the
// end of the packed keys and values.  Every other workspace byte a stage reads was written by an
// earlier stage of the same call.  Calls that overlap on one GPU (two streams, two threads) share
// the array and race.
#include <mutex>

#include "dev_common.h"
#include "vdn_internal.h"

namespace vdn {
namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;   // per GPU, held until the process ends
constexpr int kMaxDevices = 64;

// The workspace.  In host code this name is a host-side stand-in, not a device address: kernels
// and copies take the address hipGetSymbolAddress returns for the current device.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
char* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device with that device current.
hipError_t scratch_address(int dev, char** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// Block 0: the key-range table ([T+1][2 kMaxRanges] bounds, unused entries zero, then [T+1]
// counts; row T: the context query rows).  Blocks 1..H (packed-K/V plans only): zero the 128 keys
// [Lk, Ls) of head blockIdx.x - 1 in Kp [H][Ls][d] and in Vt [H][d][Ls].
__global__ __launch_bounds__(256) void noalloc_setup_kernel(Shape s, int* __restrict__ ranges, bf16_t* __restrict__ kp,
                                                            bf16_t* __restrict__ vt) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0) {
    int* counts = ranges + (size_t)(s.T + 1) * 2 * kMaxRanges;
    for (int t = tid; t <= s.T; t += blockDim.x) {
      int64_t r[2 * kMaxRanges];
      const int n = key_ranges(s, t, r, kMaxRanges);
      for (int i = 0; i < 2 * kMaxRanges; ++i) ranges[(size_t)t * 2 * kMaxRanges + i] = i < 2 * n ? (int)r[i] : 0;
      counts[t] = n;
    }
    return;
  }
  const int h = blockIdx.x - 1;
  const int64_t tail = s.Ls - s.Lk;                       // 128 keys
  bf16_t* kt = kp + ((int64_t)h * s.Ls + s.Lk) * s.d;      // contiguous tail * d elements
  for (int64_t e = tid; e < tail * s.d; e += blockDim.x) kt[e] = 0;
  for (int64_t e = tid; e < tail * s.d; e += blockDim.x) {
    const int64_t row = e / tail, j = e % tail;           // feature row, key
    vt[((int64_t)h * s.d + row) * s.Ls + s.Lk + j] = 0;
  }
}

}  // namespace
}  // namespace vdn

extern "C" vdn_status vdn_forward_noalloc(int T, int N, int C, int n_text, int H, int d, int anchors, vdn_dtype dtype,
                                          const void* q, const void* k, const void* v, const float* beta,
                                          const void* text_kv, const void* gate_w, const void* proj_w, void* out,
                                          void* stream) {
  using namespace vdn;
  const vdn_status chk = check_plan_args(T, N, C, n_text, 0, H, d, anchors, dtype, 0u);
  if (chk != VDN_OK) return chk;
  const Shape s = make_shape(T, N, C, n_text, 0, H, d, anchors, dtype);
  const Kinds kinds = choose_kinds(s);
  const Layout lay = make_layout(s, kinds);
  if (lay.total > kScratchBytes) return VDN_ERR_TOO_LARGE;
  const Inputs in{q, k, v, beta, text_kv, gate_w, proj_w, out, nullptr, nullptr, nullptr};
  const vdn_status achk = check_forward_args(s, in);
  if (achk != VDN_OK) return achk;
  int dev = -1;
  char* base = nullptr;
  if (hipGetDevice(&dev) != hipSuccess || scratch_address(dev, &base) != hipSuccess) {
    (void)hipGetLastError();
    return VDN_ERR_HIP;
  }
  const Buffers b = make_buffers(base, lay, kinds, s);
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  noalloc_setup_kernel<<<1 + (kinds.softmax_mfma ? H : 0), 256, 0, st>>>(
      s, reinterpret_cast<int*>(base + lay.ranges), b.kp, b.vt);
  if (hipGetLastError() != hipSuccess ||
      enqueue_forward(s, kinds, b, in, st, nullptr, nullptr, nullptr, nullptr) != hipSuccess) {
    (void)hipGetLastError();
    return VDN_ERR_HIP;
  }
  return VDN_OK;
}
