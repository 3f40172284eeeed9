// C ABI of the VDN layer forward: argument validation, plan ownership, stream fork/join and stage
// timing.  The kernels themselves live in the .hip files; see include/vdn.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "vdn_internal.h"

namespace vdn {

Buffers make_buffers(char* ws, const Layout& lay, const Kinds& kinds, const Shape& s) {
  Buffers b{};
  b.os = ws + lay.os;
  b.kp = kinds.softmax_mfma ? reinterpret_cast<uint16_t*>(ws + lay.kp) : nullptr;
  b.vt = kinds.softmax_mfma ? reinterpret_cast<uint16_t*>(ws + lay.vt) : nullptr;
  b.minv = reinterpret_cast<float*>(ws + lay.minv);
  b.bw = reinterpret_cast<float*>(ws + lay.bw);
  b.mhl = kinds.scan_mfma ? reinterpret_cast<uint16_t*>(ws + lay.mhl) : nullptr;
  b.cw = kinds.scan_mfma ? reinterpret_cast<float*>(ws + lay.cw) : nullptr;
  b.pp = kinds.scan_mfma ? reinterpret_cast<uint16_t*>(ws + lay.pp) : nullptr;
  b.qq = kinds.scan_mfma ? reinterpret_cast<float*>(ws + lay.qq) : nullptr;
  b.states = reinterpret_cast<float*>(ws + lay.states);
  b.wt = kinds.epilogue_mfma ? reinterpret_cast<uint16_t*>(ws + lay.wt) : nullptr;
  b.wt8 = kinds.epilogue_mx ? reinterpret_cast<uint8_t*>(ws + lay.wt8) : nullptr;
  b.wsc8 = kinds.epilogue_mx ? reinterpret_cast<uint8_t*>(ws + lay.wsc8) : nullptr;
  const bool packed = kinds.softmax_mfma || kinds.softmax_fp8;
  b.kmax_part = kinds.softmax_mfma ? reinterpret_cast<float*>(ws + lay.kmax_part) : nullptr;
  b.kmax = packed ? reinterpret_cast<float*>(ws + lay.kmax) : nullptr;
  b.flags = packed ? reinterpret_cast<int*>(ws + lay.flags) : nullptr;
  b.k8 = kinds.softmax_fp8 ? reinterpret_cast<uint8_t*>(ws + lay.k8) : nullptr;
  b.v8 = kinds.softmax_fp8 ? reinterpret_cast<uint8_t*>(ws + lay.v8) : nullptr;
  b.part8 = kinds.softmax_fp8 ? reinterpret_cast<float*>(ws + lay.part8) : nullptr;
  b.scale8 = kinds.softmax_fp8 ? reinterpret_cast<float*>(ws + lay.scale8) : nullptr;
  b.lse = kinds.softmax_fp8 ? nullptr : reinterpret_cast<float*>(ws + lay.lse);
  b.ranges = reinterpret_cast<const int*>(ws + lay.ranges);
  b.nranges = b.ranges + (size_t)(s.T + 1) * 2 * kMaxRanges;
  return b;
}

Shape make_shape(int T, int N, int C, int n_text, int n_audio, int H, int d, int anchors, vdn_dtype dt) {
  Shape s{};
  s.T = T; s.N = N; s.C = C; s.n_text = n_text; s.H = H; s.d = d; s.anchors = anchors; s.dtype = dt;
  s.n_audio = n_audio;
  s.n_ctx = n_text + n_audio;
  s.Nc = (T + C - 1) / C;
  s.ctx_pad = (int)round_up(s.n_ctx, kTextPad);
  s.Lk = (int64_t)s.ctx_pad + (int64_t)T * N;
  s.Ls = s.Lk + 128;
  s.Ls8 = s.Lk + 128;
  return s;
}

bool shape_ok(int T, int N, int C, int n_text, int H, int d, int anchors) {
  return T > 0 && N > 0 && C > 0 && n_text >= 0 && H > 0 && d > 0 && (anchors == 0 || anchors == 1);
}

vdn_status check_plan_args(int T, int N, int C, int n_text, int n_audio, int H, int d, int anchors,
                           vdn_dtype dtype, unsigned flags) {
  if (!shape_ok(T, N, C, n_text, H, d, anchors) || n_audio < 0) return VDN_ERR_INVALID_ARG;
  const int64_t n_ctx = (int64_t)n_text + n_audio;
  if (dtype != VDN_F32 && dtype != VDN_BF16) return VDN_ERR_UNSUPPORTED;
  if (d != 16 && d != 32 && d != 64 && d != 128) return VDN_ERR_UNSUPPORTED;
  // keep every index well inside 63 bits and grid dimensions inside their limits
  const int64_t tokens = (int64_t)T * N;
  if (tokens > (int64_t(1) << 31) || tokens * H * d > (int64_t(1) << 40) || n_ctx * H * d > (int64_t(1) << 40))
    return VDN_ERR_UNSUPPORTED;
  if (flags & ~(unsigned)(VDN_FLAG_GENERIC_KERNELS | VDN_FLAG_SERIAL | VDN_FLAG_OVERLAP | VDN_FLAG_FP8_SOFTMAX |
                          VDN_FLAG_FP8_EPILOGUE))
    return VDN_ERR_INVALID_ARG;
  // MXFP8 epilogue: bf16, d = 128 (one readout wave per 32-channel block), matrix-core kernels
  if ((flags & VDN_FLAG_FP8_EPILOGUE) && (flags & VDN_FLAG_GENERIC_KERNELS)) return VDN_ERR_INVALID_ARG;
  if ((flags & VDN_FLAG_FP8_EPILOGUE) && (dtype != VDN_BF16 || d != 128)) return VDN_ERR_UNSUPPORTED;
  if ((flags & VDN_FLAG_SERIAL) && (flags & VDN_FLAG_OVERLAP)) return VDN_ERR_INVALID_ARG;
  const bool fp8 = (flags & VDN_FLAG_FP8_SOFTMAX) != 0;
  if (fp8 && (flags & VDN_FLAG_GENERIC_KERNELS)) return VDN_ERR_INVALID_ARG;
  // FP8 softmax: bf16 inputs, d = 128, key tiles 16-key aligned, 32-bit lane offsets into V8
  if (fp8 && (dtype != VDN_BF16 || d != 128 || N % 16 != 0 ||
              (int64_t)d * (round_up(n_ctx, kTextPad) + tokens + 128) >= (int64_t(1) << 31)))
    return VDN_ERR_UNSUPPORTED;
  if (round_up(n_ctx, kTextPad) + tokens > INT32_MAX) return VDN_ERR_UNSUPPORTED;
  return VDN_OK;
}

namespace {

bool is_aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

bool spans_overlap(const Span& x, const Span& y) {
  if (!x.p || !y.p || x.n == 0 || y.n == 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(x.p), b = reinterpret_cast<uintptr_t>(y.p);
  return a < b + y.n && b < a + x.n;
}

vdn_status check_forward_args(const Shape& s, const Inputs& in) {
  if (!in.q || !in.k || !in.v || !in.beta || !in.gate_w || !in.proj_w || !in.out) return VDN_ERR_INVALID_ARG;
  if (s.n_ctx > 0 && !in.text_kv) return VDN_ERR_INVALID_ARG;
  if (!in.ctx_q != !in.ctx_out) return VDN_ERR_INVALID_ARG;          // context rows: both or neither
  const void* ptrs[] = {in.q, in.k, in.v, in.beta, in.gate_w, in.proj_w, in.out};
  for (const void* ptr : ptrs) if (!is_aligned16(ptr)) return VDN_ERR_INVALID_ARG;
  const void* opt[] = {in.text_kv, in.alpha, in.ctx_q, in.ctx_out};
  for (const void* ptr : opt) if (ptr && !is_aligned16(ptr)) return VDN_ERR_INVALID_ARG;
  // the outputs' bytes are disjoint from every input's and from each other's
  const size_t elt = s.dtype == VDN_BF16 ? 2 : 4;
  const size_t tok = (size_t)s.T * s.N * s.H * s.d * elt;
  const size_t ctx = (size_t)s.n_ctx * s.H * s.d * elt;
  const size_t dd2 = (size_t)2 * s.d * s.d * elt;
  const Span ins[] = {{in.q, tok},
                      {in.k, tok},
                      {in.v, tok},
                      {in.beta, ((size_t)s.n_text + (size_t)s.T * s.N) * s.H * 4},
                      {s.n_ctx > 0 ? in.text_kv : nullptr, 2 * ctx},
                      {in.gate_w, dd2},
                      {in.proj_w, dd2},
                      {in.alpha, (size_t)s.T * s.H * s.d * 4},
                      {in.ctx_q, ctx}};
  const Span outs[] = {{in.out, tok}, {in.ctx_out, ctx}};
  for (const Span& o : outs)
    for (const Span& i : ins)
      if (spans_overlap(o, i)) return VDN_ERR_INVALID_ARG;
  if (spans_overlap(outs[0], outs[1])) return VDN_ERR_INVALID_ARG;
  return VDN_OK;
}

hipError_t enqueue_forward(const Shape& s, const Kinds& kinds, const Buffers& b, const Inputs& in, hipStream_t main,
                           hipStream_t side, hipEvent_t ev_fork, hipEvent_t ev_join, hipEvent_t* ev) {
  auto mark = [&](int stage, int end, hipStream_t st) {
    if (ev) (void)hipEventRecord(ev[stage * 2 + end], st);
  };
  hipError_t e = hipSuccess;
#define VDN_TRY(x) do { if ((e = (x)) != hipSuccess) return e; } while (0)
  mark(VDN_STAGE_TOTAL, 0, main);
  // linear branch: on the caller's stream, or for overlapped plans on the side stream, forked from
  // the caller's stream
  hipStream_t lin = side ? side : main;
  if (side) {
    VDN_TRY(hipEventRecord(ev_fork, main));
    VDN_TRY(hipStreamWaitEvent(side, ev_fork, 0));
  }
  mark(VDN_STAGE_VDA_STATS, 0, lin);
  VDN_TRY(launch_vda_stats(s, in, b, kinds.stats_mfma, lin));
  mark(VDN_STAGE_VDA_STATS, 1, lin);
  mark(VDN_STAGE_VDA_SCAN, 0, lin);
  VDN_TRY(launch_vda_scan(s, in, b, kinds.scan_mfma, lin));
  mark(VDN_STAGE_VDA_SCAN, 1, lin);
  if (side) VDN_TRY(hipEventRecord(ev_join, side));
  // softmax branch on the caller's stream
  mark(VDN_STAGE_PREP, 0, main);
  if (kinds.softmax_mfma) VDN_TRY(launch_prep_kv(s, in, b, main));
  if (kinds.softmax_fp8) VDN_TRY(launch_prep_fp8(s, in, b, main));
  if (kinds.epilogue_mx) VDN_TRY(launch_prep_weights_mx(s, in, b, main));
  else if (kinds.epilogue_mfma) VDN_TRY(launch_prep_weights(s, in, b, main));
  mark(VDN_STAGE_PREP, 1, main);
  mark(VDN_STAGE_SOFTMAX, 0, main);
  mark(VDN_STAGE_SOFTMAX_FIRST, 0, main);
  hipEvent_t first_end = ev ? ev[VDN_STAGE_SOFTMAX_FIRST * 2 + 1] : nullptr;
  if (kinds.softmax_fp8) {
    VDN_TRY(launch_softmax_fp8(s, in, b, main, first_end));
  } else if (kinds.softmax_mfma) {
    VDN_TRY(launch_softmax_mfma(s, in, b, main, first_end));
  } else {
    VDN_TRY(launch_softmax_simt(s, in, b, main));
    mark(VDN_STAGE_SOFTMAX_FIRST, 1, main);
  }
  mark(VDN_STAGE_SOFTMAX, 1, main);
  // join, then readout + gates + projections
  if (side) VDN_TRY(hipStreamWaitEvent(main, ev_join, 0));
  mark(VDN_STAGE_EPILOGUE, 0, main);
  if (kinds.epilogue_mfma) VDN_TRY(launch_epilogue_mfma(s, in, b, kinds.epilogue_mx, main));
  else VDN_TRY(launch_epilogue(s, in, b, false, main));
  mark(VDN_STAGE_EPILOGUE, 1, main);
  mark(VDN_STAGE_TOTAL, 1, main);
#undef VDN_TRY
  return hipSuccess;
}

}  // namespace vdn

struct vdn_plan {
  vdn::Shape s;
  vdn::Layout lay;
  vdn::Kinds kinds;
  int device = -1;
  char* ws = nullptr;
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  // stage timing (mutable: recording events does not change the plan's meaning)
  bool overlap = false;                          // linear branch on the side stream
  // the most recent call was a successful forward (its intermediates are in the workspace), with or
  // without the decay gate
  mutable bool fwd_valid = false, fwd_alpha = false;
  mutable int prof_max = 0, prof_count = 0;
  mutable std::vector<hipEvent_t> prof_events;   // [prof_max][VDN_NUM_STAGES][2]
  // backward workspace and tables, allocated by the first vdn_backward call
  char* bws = nullptr;
  vdn::BwdBuffers bw{};
  // FP8 plans: the bf16 plan of the same shape whose backward theirs runs (created on first use)
  vdn_plan* exact = nullptr;
};

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

vdn::Buffers buffers_of(const vdn_plan* p) { return vdn::make_buffers(p->ws, p->lay, p->kinds, p->s); }

void free_plan(vdn_plan* p) {
  if (!p) return;
  if (p->device >= 0) (void)hipSetDevice(p->device);
  for (hipEvent_t e : p->prof_events) if (e) (void)hipEventDestroy(e);
  if (p->ev_fork) (void)hipEventDestroy(p->ev_fork);
  if (p->ev_join) (void)hipEventDestroy(p->ev_join);
  if (p->side) (void)hipStreamDestroy(p->side);
  if (p->ws) (void)hipFree(p->ws);
  if (p->bws) (void)hipFree(p->bws);
  if (p->exact) free_plan(p->exact);
  delete p;
}

}  // namespace

extern "C" {

const char* vdn_status_str(vdn_status s) {
  switch (s) {
    case VDN_OK: return "ok";
    case VDN_ERR_INVALID_ARG: return "invalid argument";
    case VDN_ERR_UNSUPPORTED: return "unsupported configuration";
    case VDN_ERR_OUT_OF_MEMORY: return "out of device memory";
    case VDN_ERR_HIP: return "HIP runtime error";
    case VDN_ERR_TOO_LARGE: return "workspace exceeds the static scratch of vdn_forward_noalloc";
  }
  return "unknown status";
}

int vdn_key_ranges(int T, int N, int C, int n_text, int anchors, int t, int64_t* ranges, int max_ranges) {
  if (!vdn::shape_ok(T, N, C, n_text, 1, 1, anchors) || t < 0 || t >= T || (max_ranges > 0 && !ranges) || max_ranges < 0)
    return -1;
  vdn::Shape s = vdn::make_shape(T, N, C, n_text, 0, 1, 1, anchors, VDN_F32);
  return vdn::key_ranges(s, t, ranges, max_ranges);
}

int vdn_scan_frames(int T, int C, int anchors, int t, int dir, int* frames, int max_frames) {
  if (!vdn::shape_ok(T, 1, C, 0, 1, 1, anchors) || t < 0 || t >= T || (dir != 0 && dir != 1) ||
      (max_frames > 0 && !frames) || max_frames < 0)
    return -1;
  vdn::Shape s = vdn::make_shape(T, 1, C, 0, 0, 1, 1, anchors, VDN_F32);
  return vdn::scan_frames(s, t, dir, frames, max_frames);
}

vdn_status vdn_plan_create(int T, int N, int C, int n_text, int H, int d, int anchors, vdn_dtype dtype,
                           vdn_plan** plan_out) {
  return vdn_plan_create_ex(T, N, C, n_text, H, d, anchors, dtype, 0u, plan_out);
}

vdn_status vdn_plan_create_ex(int T, int N, int C, int n_text, int H, int d, int anchors, vdn_dtype dtype,
                              unsigned flags, vdn_plan** plan_out) {
  return vdn_plan_create_joint(T, N, C, n_text, 0, H, d, anchors, dtype, flags, plan_out);
}

vdn_status vdn_plan_create_joint(int T, int N, int C, int n_text, int n_audio, int H, int d, int anchors,
                                 vdn_dtype dtype, unsigned flags, vdn_plan** plan_out) {
  if (!plan_out) return VDN_ERR_INVALID_ARG;
  *plan_out = nullptr;
  const vdn_status chk = vdn::check_plan_args(T, N, C, n_text, n_audio, H, d, anchors, dtype, flags);
  if (chk != VDN_OK) return chk;
  const bool fp8 = (flags & VDN_FLAG_FP8_SOFTMAX) != 0;

  vdn_plan* p = new (std::nothrow) vdn_plan();
  if (!p) return VDN_ERR_OUT_OF_MEMORY;
  p->s = vdn::make_shape(T, N, C, n_text, n_audio, H, d, anchors, dtype);
  p->kinds = (flags & VDN_FLAG_GENERIC_KERNELS) ? vdn::Kinds{} : vdn::choose_kinds(p->s);
  if (fp8) {
    p->kinds.softmax_mfma = false;
    p->kinds.softmax_fp8 = true;
  }
  if (flags & VDN_FLAG_FP8_EPILOGUE) {
    p->kinds.epilogue_mfma = true;
    p->kinds.epilogue_mx = true;
  }
  p->overlap = (flags & VDN_FLAG_OVERLAP) != 0;
  p->lay = vdn::make_layout(p->s, p->kinds);
  if (hipGetDevice(&p->device) != hipSuccess) { free_plan(p); return VDN_ERR_HIP; }
  if (hipMalloc(&p->ws, p->lay.total) != hipSuccess) {
    (void)hipGetLastError();
    p->ws = nullptr;
    free_plan(p);
    return VDN_ERR_OUT_OF_MEMORY;
  }
  // key-range table: one row per query frame, then one for the context (text and audio) rows
  std::vector<int> tab((size_t)(T + 1) * (2 * vdn::kMaxRanges + 1), 0);
  for (int t = 0; t <= T; ++t) {
    int64_t r[2 * vdn::kMaxRanges];
    int n = vdn::key_ranges(p->s, t, r, vdn::kMaxRanges);
    for (int i = 0; i < 2 * n; ++i) tab[(size_t)t * 2 * vdn::kMaxRanges + i] = (int)r[i];
    tab[(size_t)(T + 1) * 2 * vdn::kMaxRanges + t] = n;
  }
  // the packed K/V padding tile must hold finite values (zero); the packing pass never writes it
  if ((p->kinds.softmax_mfma &&
       (hipMemset(p->ws + p->lay.kp, 0, (size_t)p->s.H * p->s.Ls * d * 2) != hipSuccess ||
        hipMemset(p->ws + p->lay.vt, 0, (size_t)p->s.H * p->s.Ls * d * 2) != hipSuccess)) ||
      (p->kinds.softmax_fp8 &&
       (hipMemset(p->ws + p->lay.k8, 0, (size_t)p->s.H * p->s.Ls8 * d) != hipSuccess ||
        hipMemset(p->ws + p->lay.v8, 0, (size_t)p->s.H * p->s.Ls8 * d) != hipSuccess)) ||
      hipMemcpy(p->ws + p->lay.ranges, tab.data(), tab.size() * sizeof(int), hipMemcpyHostToDevice) != hipSuccess ||
      (p->overlap && (hipStreamCreateWithFlags(&p->side, hipStreamNonBlocking) != hipSuccess ||
                      hipEventCreateWithFlags(&p->ev_fork, hipEventDisableTiming) != hipSuccess ||
                      hipEventCreateWithFlags(&p->ev_join, hipEventDisableTiming) != hipSuccess))) {
    free_plan(p);
    return VDN_ERR_HIP;
  }
  *plan_out = p;
  return VDN_OK;
}

void vdn_plan_destroy(vdn_plan* plan) { free_plan(plan); }

size_t vdn_plan_workspace_bytes(const vdn_plan* plan) { return plan ? plan->lay.total : 0; }

vdn_status vdn_plan_kernel_kind(const vdn_plan* plan, int stage, int* kind) {
  if (!plan || !kind) return VDN_ERR_INVALID_ARG;
  switch (stage) {
    case VDN_STAGE_SOFTMAX:
    case VDN_STAGE_SOFTMAX_FIRST: *kind = plan->kinds.softmax_fp8 ? 2 : plan->kinds.softmax_mfma; break;
    case VDN_STAGE_PREP: *kind = plan->kinds.softmax_mfma || plan->kinds.softmax_fp8 || plan->kinds.epilogue_mfma; break;
    case VDN_STAGE_VDA_STATS: *kind = plan->kinds.stats_mfma; break;
    case VDN_STAGE_VDA_SCAN: *kind = plan->kinds.scan_mfma; break;
    case VDN_STAGE_EPILOGUE: *kind = plan->kinds.epilogue_mx ? 2 : plan->kinds.epilogue_mfma; break;
    default: return VDN_ERR_INVALID_ARG;
  }
  return VDN_OK;
}

namespace {

vdn_status forward_impl(const vdn_plan* plan, const void* q, const void* k, const void* v, const float* beta,
                        const void* ctx_q, const void* text_kv, const float* alpha, const void* gate_w,
                        const void* proj_w, void* out, void* ctx_out, void* stream) {
  if (!plan) return VDN_ERR_INVALID_ARG;
  if (!ctx_q != !ctx_out) return VDN_ERR_INVALID_ARG;          // context rows: both or neither
  if (plan->s.n_ctx == 0) ctx_q = ctx_out = nullptr;
  const vdn::Inputs in{q, k, v, beta, text_kv, gate_w, proj_w, out, alpha, ctx_q, ctx_out};
  const vdn_status chk = vdn::check_forward_args(plan->s, in);
  if (chk != VDN_OK) return chk;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return VDN_ERR_HIP;
  if (dev != plan->device) return VDN_ERR_INVALID_ARG;

  hipEvent_t* ev = nullptr;
  if (plan->prof_count < plan->prof_max) {
    ev = &plan->prof_events[(size_t)plan->prof_count * VDN_NUM_STAGES * 2];
    ++plan->prof_count;
  }
  plan->fwd_valid = false;                       // until every stage is enqueued
  if (vdn::enqueue_forward(plan->s, plan->kinds, buffers_of(plan), in, reinterpret_cast<hipStream_t>(stream),
                           plan->overlap ? plan->side : nullptr, plan->ev_fork, plan->ev_join, ev) != hipSuccess) {
    (void)hipGetLastError();
    return VDN_ERR_HIP;
  }
  plan->fwd_valid = true;
  plan->fwd_alpha = alpha != nullptr;
  return VDN_OK;
}

}  // namespace

vdn_status vdn_forward(const vdn_plan* plan, const void* q, const void* k, const void* v, const float* beta,
                       const void* text_kv, const void* gate_w, const void* proj_w, void* out, void* stream) {
  return forward_impl(plan, q, k, v, beta, nullptr, text_kv, nullptr, gate_w, proj_w, out, nullptr, stream);
}

vdn_status vdn_forward_decay(const vdn_plan* plan, const void* q, const void* k, const void* v, const float* beta,
                             const void* text_kv, const float* alpha, const void* gate_w, const void* proj_w,
                             void* out, void* stream) {
  if (!alpha) return VDN_ERR_INVALID_ARG;
  return forward_impl(plan, q, k, v, beta, nullptr, text_kv, alpha, gate_w, proj_w, out, nullptr, stream);
}

vdn_status vdn_forward_joint(const vdn_plan* plan, const void* q, const void* k, const void* v, const float* beta,
                             const void* ctx_q, const void* ctx_kv, const float* alpha, const void* gate_w,
                             const void* proj_w, void* out, void* ctx_out, void* stream) {
  return forward_impl(plan, q, k, v, beta, ctx_q, ctx_kv, alpha, gate_w, proj_w, out, ctx_out, stream);
}

namespace {

// Backward workspace: buffers and host-built tables (scan order, readout slots, query ranges per
// key slot, row segments), allocated once per plan.
vdn_status ensure_backward(vdn_plan* p) {
  if (p->bws) return VDN_OK;
  const vdn::Shape& s = p->s;
  const int T = s.T, N = s.N, H = s.H, d = s.d, Nc = s.Nc, C = s.C;
  const int64_t rows = (int64_t)T * N * H;
  const int64_t dd = (int64_t)d * d;
  // scan order and readout slots
  std::vector<int> order;
  for (int f = 0; f < T; ++f)
    if (!vdn::is_boundary(s, f)) order.push_back(f);
  const int nslots = Nc + 2;
  std::vector<int> mslot(2 * nslots, 0);
  for (int c = 0; c < Nc; ++c) {
    int mf = 0, mr = 0;
    for (int f : order) {
      if (f / C <= c - 2) ++mf;
      if (f / C >= c + 2) ++mr;
    }
    mslot[c] = mf;
    mslot[nslots + c] = mr;
  }
  // query-frame ranges for each key slot (0 = the global text and audio keys: every frame; 1 + f =
  // frame f); the context query rows, when a backward includes them, see every slot
  std::vector<int> qr((size_t)(T + 1) * 2 * vdn::kMaxRanges, 0), nqr(T + 1, 0);
  for (int slot = 0; slot <= T; ++slot) {
    int n = 0, start = -1;
    for (int t = 0; t <= T; ++t) {
      bool sees = false;
      if (t < T) {
        if (slot == 0) sees = true;
        else {
          const int f = slot - 1;
          int64_t r[2 * vdn::kMaxRanges];
          const int nr = vdn::key_ranges(s, t, r, vdn::kMaxRanges);
          const int64_t key = (int64_t)s.ctx_pad + (int64_t)f * N;
          for (int i = 0; i < nr; ++i) sees |= (r[2 * i] <= key && key < r[2 * i + 1]);
        }
      }
      if (sees && start < 0) start = t;
      if (!sees && start >= 0) {
        if (n >= vdn::kMaxRanges) return VDN_ERR_UNSUPPORTED;
        qr[(size_t)slot * 2 * vdn::kMaxRanges + 2 * n] = start;
        qr[(size_t)slot * 2 * vdn::kMaxRanges + 2 * n + 1] = t;
        ++n;
        start = -1;
      }
    }
    nqr[slot] = n;
  }
  // row segments: all rows of all heads; each chunk's non-boundary frames and each boundary
  // frame, per head
  std::vector<vdn::Segment> seg_all{{0, T * N, -1}}, seg_read;
  for (int c = 0; c < nslots; ++c)
    for (int h = 0; h < H; ++h) {
      int f0 = 0, f1 = 0;
      if (c < Nc) {
        f0 = c * C;
        f1 = std::min(T, (c + 1) * C);
        while (f0 < f1 && vdn::is_boundary(s, f0)) ++f0;
        while (f1 > f0 && vdn::is_boundary(s, f1 - 1)) --f1;
      } else if (s.anchors) {
        f0 = c == Nc ? 0 : T - 1;
        f1 = f0 + 1;
        if (c == Nc + 1 && T == 1) f1 = f0;          // a single frame is one boundary frame
      }
      seg_read.push_back({(int64_t)f0 * N, (f1 - f0) * N, h});
    }
  // Workgroup tables of the MFMA softmax transposes.  Workgroups are dispatched round-robin over
  // the 8 XCDs, so entry w runs on XCD w % 8.  A group of workgroups that stream the same operand
  // tiles (the key blocks of one slot and head; the query tiles of one frame and head) is placed on
  // one XCD, whose L2 then serves them all; groups go in decreasing work (the slots every query
  // frame sees, the frames that see every key: their walks are the longest and start with the
  // launch), each to the XCD with the least work so far.
  auto xcd_table = [](const auto& groups, const std::vector<int64_t>& work, auto noop) {
    using E = decltype(noop);
    constexpr int kXcds = 8;
    std::vector<std::vector<E>> q(kXcds);
    std::vector<int64_t> load(kXcds, 0);
    for (size_t g = 0; g < groups.size(); ++g) {
      const int x = (int)(std::min_element(load.begin(), load.end()) - load.begin());
      load[x] += work[g];
      q[x].insert(q[x].end(), groups[g].begin(), groups[g].end());
    }
    size_t rounds = 0;
    for (const auto& v : q) rounds = std::max(rounds, v.size());
    std::vector<E> table(rounds * kXcds, noop);
    for (int x = 0; x < kXcds; ++x)
      for (size_t r = 0; r < q[x].size(); ++r) table[r * kXcds + x] = q[x][r];
    return table;
  };
  // dK/dV: blocks of bkeys keys of one slot; the global keys and the boundary frames first
  const int bkeys = vdn::softmax_dkv_block_keys();
  std::vector<std::vector<int4>> kgroups;
  std::vector<int64_t> kgwork;
  auto add_slot = [&](int slot) {
    const int U = slot == 0 ? s.n_ctx : N;
    int64_t frames = 0;
    for (int r = 0; r < nqr[slot]; ++r)
      frames += qr[(size_t)slot * 2 * vdn::kMaxRanges + 2 * r + 1] - qr[(size_t)slot * 2 * vdn::kMaxRanges + 2 * r];
    for (int h = 0; h < H; ++h) {
      std::vector<int4> g;
      for (int k0 = 0; k0 < U; k0 += bkeys) g.push_back(make_int4(slot, k0, h, 0));
      kgwork.push_back((int64_t)g.size() * frames);
      kgroups.push_back(std::move(g));
    }
  };
  if (s.n_ctx > 0) add_slot(0);
  for (int f = 0; f < T; ++f)
    if (vdn::is_boundary(s, f)) add_slot(1 + f);
  for (int f = 0; f < T; ++f)
    if (!vdn::is_boundary(s, f)) add_slot(1 + f);
  const std::vector<int4> kwork = xcd_table(kgroups, kgwork, make_int4(-1, 0, 0, 0));
  // dQ: the query tiles of one frame and head; frames by decreasing key count
  const int QT = (N + vdn::softmax_dq_block_queries() - 1) / vdn::softmax_dq_block_queries();
  std::vector<int> qframes(T);
  std::vector<int64_t> nkeys(T, 0);
  for (int t = 0; t < T; ++t) {
    qframes[t] = t;
    int64_t r[2 * vdn::kMaxRanges];
    const int nr = vdn::key_ranges(s, t, r, vdn::kMaxRanges);
    for (int i = 0; i < nr; ++i) nkeys[t] += r[2 * i + 1] - r[2 * i];
  }
  std::stable_sort(qframes.begin(), qframes.end(), [&](int a, int b) { return nkeys[a] > nkeys[b]; });
  std::vector<std::vector<int2>> qgroups;
  std::vector<int64_t> qgwork;
  for (int t : qframes)
    for (int h = 0; h < H; ++h) {
      std::vector<int2> g;
      for (int qt = 0; qt < QT; ++qt) g.push_back(make_int2(t, qt + QT * h));
      qgwork.push_back((int64_t)QT * nkeys[t]);
      qgroups.push_back(std::move(g));
    }
  const std::vector<int2> qwork = xcd_table(qgroups, qgwork, make_int2(-1, 0));
  const bool mfma_bwd = p->kinds.softmax_mfma;
  // transposed query rows: the video rows, then the context rows from column T N, then a tile of
  // zero padding for the last partial tile
  const int64_t Lq = (int64_t)T * N + vdn::round_up(s.n_ctx, 64) + 64;
  const size_t elt = s.dtype == VDN_BF16 ? 2 : 4;
  const int64_t ctx_elems = (int64_t)s.n_ctx * H * d;
  const int splits_all = 512, splits_read = 8;
  // layout
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += (size_t)vdn::round_up((int64_t)bytes, 256); return o; };
  const size_t o_rows6 = take((size_t)6 * rows * d * 4);
  const size_t o_dsum = take((size_t)(rows + (int64_t)s.n_ctx * H) * 4);
  const size_t o_octx = take((size_t)ctx_elems * elt), o_doctx = take((size_t)ctx_elems * 4);
  const size_t o_part = take((size_t)std::max<int64_t>(splits_all, (int64_t)nslots * H * splits_read) * dd * 4);
  const size_t o_dread = take((size_t)nslots * H * dd * 4);
  const size_t o_z = take((size_t)3 * 2 * T * H * dd * 4);
  const size_t o_g = take((size_t)2 * (T + 1) * H * dd * 4);
  const size_t o_dal = take((size_t)2 * T * H * d * 4);
  const size_t o_ds0 = take((size_t)2 * H * dd * 4);
  const size_t o_order = take(std::max<size_t>(1, order.size()) * 4), o_ms = take(mslot.size() * 4);
  const size_t o_qr = take(qr.size() * 4), o_nqr = take(nqr.size() * 4);
  const size_t o_sa = take(seg_all.size() * sizeof(vdn::Segment)), o_sr = take(seg_read.size() * sizeof(vdn::Segment));
  const size_t o_kw = take(std::max<size_t>(1, kwork.size()) * sizeof(int4));
  const size_t o_qw = take(std::max<size_t>(1, qwork.size()) * sizeof(int2));
  // matrix images: the merge's, then (reusing the space) the token gradients'
  const size_t mimg_bytes = (size_t)std::max<int64_t>(6 + 4 * (int64_t)(s.Nc + 1) * H, 6 * (int64_t)(T + 1) * H) * dd * 2;
  const size_t pack_bytes =
      mfma_bwd ? (size_t)H * d * 2 * (2 * Lq + 2 * s.Ls) + (size_t)rows * d * 2 + mimg_bytes : 0;
  const size_t o_pack = take(pack_bytes);
  char* ws = nullptr;
  if (hipMalloc(&ws, off) != hipSuccess) {
    (void)hipGetLastError();
    return VDN_ERR_OUT_OF_MEMORY;
  }
  auto up = [&](size_t o, const void* src, size_t bytes) {
    return bytes == 0 || hipMemcpy(ws + o, src, bytes, hipMemcpyHostToDevice) == hipSuccess;
  };
  if (!up(o_order, order.data(), order.size() * 4) || !up(o_ms, mslot.data(), mslot.size() * 4) ||
      !up(o_qr, qr.data(), qr.size() * 4) || !up(o_nqr, nqr.data(), nqr.size() * 4) ||
      !up(o_sa, seg_all.data(), seg_all.size() * sizeof(vdn::Segment)) ||
      !up(o_sr, seg_read.data(), seg_read.size() * sizeof(vdn::Segment)) ||
      !up(o_kw, kwork.data(), kwork.size() * sizeof(int4)) || !up(o_qw, qwork.data(), qwork.size() * sizeof(int2)) ||
      (pack_bytes && hipMemset(ws + o_pack, 0, pack_bytes) != hipSuccess)) {
    (void)hipFree(ws);
    return VDN_ERR_HIP;
  }
  vdn::BwdBuffers& w = p->bw;
  float* r6 = reinterpret_cast<float*>(ws + o_rows6);
  w.do_s = r6;
  w.do_l = r6 + rows * d;
  w.x_s = r6 + 2 * rows * d;
  w.x_l = r6 + 3 * rows * d;
  w.dz_s = r6 + 4 * rows * d;
  w.dz_l = r6 + 5 * rows * d;
  w.dsum = reinterpret_cast<float*>(ws + o_dsum);
  w.octx = ws + o_octx;
  w.do_ctx = reinterpret_cast<float*>(ws + o_doctx);
  w.dctx_out = nullptr;
  w.partial = reinterpret_cast<float*>(ws + o_part);
  w.dread = reinterpret_cast<float*>(ws + o_dread);
  float* z = reinterpret_cast<float*>(ws + o_z);
  w.zin = z;
  w.dmf = z + 2 * (int64_t)T * H * dd;
  w.dbf = z + 4 * (int64_t)T * H * dd;
  w.gsym = reinterpret_cast<float*>(ws + o_g);
  w.gdb = w.gsym + (int64_t)(T + 1) * H * dd;
  w.dalf = reinterpret_cast<float*>(ws + o_dal);
  w.ds0 = reinterpret_cast<float*>(ws + o_ds0);
  w.order = reinterpret_cast<const int*>(ws + o_order);
  w.mslot = reinterpret_cast<const int*>(ws + o_ms);
  w.qranges = reinterpret_cast<const int*>(ws + o_qr);
  w.nqranges = reinterpret_cast<const int*>(ws + o_nqr);
  w.seg_all = reinterpret_cast<const vdn::Segment*>(ws + o_sa);
  w.seg_read = reinterpret_cast<const vdn::Segment*>(ws + o_sr);
  w.splits_all = splits_all;
  w.splits_read = splits_read;
  w.nscan = (int)order.size();
  w.kwork = reinterpret_cast<const int4*>(ws + o_kw);
  w.nkwork = (int)kwork.size();
  w.qwork = reinterpret_cast<const int2*>(ws + o_qw);
  w.nqwork = (int)qwork.size();
  w.Lq = Lq;
  if (mfma_bwd) {
    uint16_t* pk = reinterpret_cast<uint16_t*>(ws + o_pack);
    w.qt = pk;
    w.dot = pk + (int64_t)H * d * Lq;
    w.kt = pk + 2 * (int64_t)H * d * Lq;
    w.vp = w.kt + (int64_t)H * d * s.Ls;
    w.dos16 = w.vp + (int64_t)H * d * s.Ls;
    w.mimg = w.dos16 + rows * d;
  }
  p->bws = ws;
  return VDN_OK;
}

}  // namespace

namespace {

vdn_status backward_impl(vdn_plan* plan, const void* q, const void* k, const void* v, const float* beta,
                         const void* text_kv, const void* ctx_q, const float* alpha, const void* gate_w,
                         const void* proj_w, const void* dout, const void* dctx_out, float* dq, float* dk, float* dv,
                         float* dbeta, float* dtext_kv, float* dctx_q, float* dgate_w, float* dproj_w, float* dalpha,
                         void* stream, bool recompute) {
  if (!plan || !q || !k || !v || !beta || !gate_w || !proj_w || !dout || !dq || !dk || !dv || !dbeta || !dgate_w ||
      !dproj_w)
    return VDN_ERR_INVALID_ARG;
  if (plan->kinds.softmax_fp8 || plan->kinds.epilogue_mx) {
    // FP8 plans: the gradient of the exact layer at the same inputs (their roundings are passed
    // straight through), computed by a bf16 plan of the same shape; the FP8 forward leaves none of
    // the exact intermediates the after-forward variant reuses
    if (!recompute) return VDN_ERR_UNSUPPORTED;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return VDN_ERR_HIP;
    if (cur != plan->device) return VDN_ERR_INVALID_ARG;
    if (!plan->exact) {
      const vdn::Shape& s = plan->s;
      const vdn_status cs = vdn_plan_create_joint(s.T, s.N, s.C, s.n_text, s.n_audio, s.H, s.d, s.anchors, s.dtype,
                                                  0, &plan->exact);
      if (cs != VDN_OK) return cs;
    }
    plan = plan->exact;
  }
  if (plan->s.n_ctx > 0 && (!text_kv || !dtext_kv)) return VDN_ERR_INVALID_ARG;
  if (dalpha && !alpha) return VDN_ERR_INVALID_ARG;
  // the context query rows: all three pointers or none; ignored without context tokens
  const int nset = (ctx_q != nullptr) + (dctx_out != nullptr) + (dctx_q != nullptr);
  if (nset != 0 && nset != 3) return VDN_ERR_INVALID_ARG;
  if (plan->s.n_ctx == 0) ctx_q = dctx_out = dctx_q = nullptr;
  const bool ctx_rows = ctx_q != nullptr;
  const void* ptrs[] = {q, k, v, beta, gate_w, proj_w, dout, dq, dk, dv, dbeta, dgate_w, dproj_w};
  for (const void* ptr : ptrs) if (!aligned16(ptr)) return VDN_ERR_INVALID_ARG;
  const void* opt[] = {text_kv, dtext_kv, alpha, dalpha, ctx_q, dctx_out, dctx_q};
  for (const void* ptr : opt) if (ptr && !aligned16(ptr)) return VDN_ERR_INVALID_ARG;
  {
    // every output's bytes are disjoint from every input's and from the other outputs'
    const vdn::Shape& s = plan->s;
    const size_t elt = s.dtype == VDN_BF16 ? 2 : 4;
    const size_t tokn = (size_t)s.T * s.N * s.H * s.d;
    const size_t brow = ((size_t)s.n_text + (size_t)s.T * s.N) * s.H;
    const size_t ctx = (size_t)s.n_ctx * s.H * s.d, dd2 = (size_t)2 * s.d * s.d;
    const size_t al = (size_t)s.T * s.H * s.d;
    const vdn::Span outs[] = {{dq, tokn * 4}, {dk, tokn * 4}, {dv, tokn * 4}, {dbeta, brow * 4},
                              {s.n_ctx > 0 ? dtext_kv : nullptr, 2 * ctx * 4}, {dgate_w, dd2 * 4},
                              {dproj_w, dd2 * 4}, {dalpha, al * 4}, {dctx_q, ctx * 4}};
    const vdn::Span ins[] = {{q, tokn * elt}, {k, tokn * elt}, {v, tokn * elt}, {beta, brow * 4},
                             {s.n_ctx > 0 ? text_kv : nullptr, 2 * ctx * elt}, {alpha, al * 4},
                             {gate_w, dd2 * elt}, {proj_w, dd2 * elt}, {dout, tokn * elt},
                             {ctx_q, ctx * elt}, {dctx_out, ctx * elt}};
    for (const vdn::Span& o : outs) {
      for (const vdn::Span& i : ins)
        if (vdn::spans_overlap(o, i)) return VDN_ERR_INVALID_ARG;
      for (const vdn::Span& o2 : outs)
        if (&o2 != &o && vdn::spans_overlap(o, o2)) return VDN_ERR_INVALID_ARG;
    }
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return VDN_ERR_HIP;
  if (dev != plan->device) return VDN_ERR_INVALID_ARG;
  if (!recompute && (!plan->fwd_valid || plan->fwd_alpha != (alpha != nullptr))) return VDN_ERR_INVALID_ARG;
  vdn_status st = ensure_backward(plan);
  if (st != VDN_OK) return st;

  const vdn::Shape& s = plan->s;
  hipStream_t main = reinterpret_cast<hipStream_t>(stream);
  vdn::BwdBuffers w = plan->bw;
  // the context rows' output is recomputed into the backward workspace
  vdn::Inputs in{q, k, v, beta, text_kv, gate_w, proj_w, nullptr, alpha, ctx_q, ctx_rows ? w.octx : nullptr};
  vdn::Buffers b = buffers_of(plan);
  w.dout = dout;
  w.lse = b.lse;
  w.dctx_out = dctx_out;
  vdn::BwdOutputs o{dq, dk, dv, dbeta, dtext_kv, dgate_w, dproj_w, dalpha, dctx_q};
#define VDN_TRY(x) do { if ((x) != hipSuccess) { (void)hipGetLastError(); return VDN_ERR_HIP; } } while (0)
  if (recompute) {
    // forward recomputation: linear-branch states, softmax output and its normalisers (with the
    // context rows' output and normalisers when they are part of this backward)
    VDN_TRY(vdn::launch_vda_stats(s, in, b, plan->kinds.stats_mfma, main));
    VDN_TRY(vdn::launch_vda_scan(s, in, b, plan->kinds.scan_mfma, main));
    if (plan->kinds.softmax_mfma) {
      VDN_TRY(vdn::launch_prep_kv(s, in, b, main));
      VDN_TRY(vdn::launch_softmax_mfma(s, in, b, main));
    } else {
      VDN_TRY(vdn::launch_softmax_simt(s, in, b, main));
    }
    plan->fwd_valid = true;                      // the workspace now holds this forward's intermediates
    plan->fwd_alpha = alpha != nullptr;
  }
  VDN_TRY(vdn::launch_backward(s, in, b, w, o, plan->kinds.softmax_mfma, main));
#undef VDN_TRY
  return VDN_OK;
}

}  // namespace

vdn_status vdn_backward(vdn_plan* plan, const void* q, const void* k, const void* v, const float* beta,
                        const void* text_kv, const float* alpha, const void* gate_w, const void* proj_w,
                        const void* dout, float* dq, float* dk, float* dv, float* dbeta, float* dtext_kv,
                        float* dgate_w, float* dproj_w, float* dalpha, void* stream) {
  return backward_impl(plan, q, k, v, beta, text_kv, nullptr, alpha, gate_w, proj_w, dout, nullptr, dq, dk, dv, dbeta,
                       dtext_kv, nullptr, dgate_w, dproj_w, dalpha, stream, true);
}

vdn_status vdn_backward_joint(vdn_plan* plan, const void* q, const void* k, const void* v, const float* beta,
                              const void* ctx_q, const void* ctx_kv, const float* alpha, const void* gate_w,
                              const void* proj_w, const void* dout, const void* dctx_out, float* dq, float* dk,
                              float* dv, float* dbeta, float* dctx_q, float* dctx_kv, float* dgate_w, float* dproj_w,
                              float* dalpha, void* stream) {
  return backward_impl(plan, q, k, v, beta, ctx_kv, ctx_q, alpha, gate_w, proj_w, dout, dctx_out, dq, dk, dv, dbeta,
                       dctx_kv, dctx_q, dgate_w, dproj_w, dalpha, stream, true);
}

vdn_status vdn_backward_after_forward(vdn_plan* plan, const void* q, const void* k, const void* v,
                                      const float* beta, const void* text_kv, const float* alpha,
                                      const void* gate_w, const void* proj_w, const void* dout, float* dq,
                                      float* dk, float* dv, float* dbeta, float* dtext_kv, float* dgate_w,
                                      float* dproj_w, float* dalpha, void* stream) {
  return backward_impl(plan, q, k, v, beta, text_kv, nullptr, alpha, gate_w, proj_w, dout, nullptr, dq, dk, dv, dbeta,
                       dtext_kv, nullptr, dgate_w, dproj_w, dalpha, stream, false);
}

vdn_status vdn_debug_buffer_bytes(const vdn_plan* plan, int which, size_t* bytes) {
  if (!plan || !bytes) return VDN_ERR_INVALID_ARG;
  const vdn::Shape& s = plan->s;
  const size_t dd = (size_t)s.d * s.d;
  switch (which) {
    case VDN_BUF_OS: *bytes = (size_t)s.T * s.N * s.H * s.d * (s.dtype == VDN_BF16 ? 2 : 4); break;
    case VDN_BUF_STATES: *bytes = (size_t)2 * (s.Nc + 1) * s.H * dd * 4; break;
    case VDN_BUF_MINV: *bytes = (size_t)(s.T + 1) * s.H * dd * 4; break;
    case VDN_BUF_BW: *bytes = (size_t)(s.T + 1) * s.H * dd * 4; break;
    case VDN_BUF_K8:
    case VDN_BUF_V8:
      if (!plan->kinds.softmax_fp8) return VDN_ERR_INVALID_ARG;
      *bytes = (size_t)s.H * s.Ls8 * s.d;
      break;
    case VDN_BUF_SCALES8:
      if (!plan->kinds.softmax_fp8) return VDN_ERR_INVALID_ARG;
      *bytes = (size_t)s.H * 2 * 4;
      break;
    default: return VDN_ERR_INVALID_ARG;
  }
  return VDN_OK;
}

vdn_status vdn_debug_copy(const vdn_plan* plan, int which, void* dst, size_t bytes, void* stream) {
  size_t want = 0;
  vdn_status st = vdn_debug_buffer_bytes(plan, which, &want);
  if (st != VDN_OK) return st;
  if (!dst || bytes != want) return VDN_ERR_INVALID_ARG;
  size_t off = which == VDN_BUF_OS ? plan->lay.os
               : which == VDN_BUF_STATES ? plan->lay.states
               : which == VDN_BUF_MINV ? plan->lay.minv
               : which == VDN_BUF_BW ? plan->lay.bw
               : which == VDN_BUF_K8 ? plan->lay.k8
               : which == VDN_BUF_V8 ? plan->lay.v8
                                     : plan->lay.scale8;
  if (hipMemcpyAsync(dst, plan->ws + off, bytes, hipMemcpyDeviceToDevice, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) {
    (void)hipGetLastError();
    return VDN_ERR_HIP;
  }
  return VDN_OK;
}

vdn_status vdn_debug_epilogue(vdn_plan* plan, const void* q, const void* o_s, const float* states, const void* gate_w,
                              const void* proj_w, void* out, void* stream) {
  if (!plan || !q || !o_s || !states || !gate_w || !proj_w || !out) return VDN_ERR_INVALID_ARG;
  if (!plan->kinds.epilogue_mfma) return VDN_ERR_UNSUPPORTED;
  const vdn::Shape& s = plan->s;
  const size_t tok = (size_t)s.T * s.N * s.H * s.d * 2;
  const size_t st_bytes = (size_t)2 * (s.Nc + 1) * s.H * s.d * s.d * 4;
  const size_t w_bytes = (size_t)2 * s.d * s.d * 2;
  const vdn::Span ins[] = {{q, tok}, {o_s, tok}, {states, st_bytes}, {gate_w, w_bytes}, {proj_w, w_bytes}};
  for (const vdn::Span& i : ins)
    if (vdn::spans_overlap({out, tok}, i) || (reinterpret_cast<uintptr_t>(i.p) & 15u)) return VDN_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(out) & 15u) return VDN_ERR_INVALID_ARG;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return VDN_ERR_HIP;
  if (dev != plan->device) return VDN_ERR_INVALID_ARG;
  plan->fwd_valid = false;                       // the workspace no longer holds a forward's intermediates
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const vdn::Buffers b = buffers_of(plan);
  vdn::Inputs in{};
  in.q = q;
  in.gate_w = gate_w;
  in.proj_w = proj_w;
  in.out = out;
  if (hipMemcpyAsync(b.os, o_s, tok, hipMemcpyDeviceToDevice, st) != hipSuccess ||
      hipMemcpyAsync(b.states, states, st_bytes, hipMemcpyDeviceToDevice, st) != hipSuccess ||
      (plan->kinds.epilogue_mx ? vdn::launch_prep_weights_mx(s, in, b, st) : vdn::launch_prep_weights(s, in, b, st)) !=
          hipSuccess ||
      vdn::launch_epilogue_mfma(s, in, b, plan->kinds.epilogue_mx, st) != hipSuccess) {
    (void)hipGetLastError();
    return VDN_ERR_HIP;
  }
  return VDN_OK;
}

vdn_status vdn_profile_enable(vdn_plan* plan, int max_calls) {
  if (!plan || max_calls < 0 || max_calls > 100000) return VDN_ERR_INVALID_ARG;
  for (hipEvent_t e : plan->prof_events) if (e) (void)hipEventDestroy(e);
  plan->prof_events.assign((size_t)max_calls * VDN_NUM_STAGES * 2, nullptr);
  plan->prof_max = 0;
  plan->prof_count = 0;
  for (auto& e : plan->prof_events)
    if (hipEventCreate(&e) != hipSuccess) { e = nullptr; return VDN_ERR_HIP; }
  plan->prof_max = max_calls;
  return VDN_OK;
}

vdn_status vdn_profile_read(vdn_plan* plan, float* ms, int n_stages, int* calls) {
  if (!plan || !ms || n_stages < 0 || n_stages > VDN_NUM_STAGES) return VDN_ERR_INVALID_ARG;
  for (int st = 0; st < n_stages; ++st) ms[st] = 0.f;
  for (int c = 0; c < plan->prof_count; ++c) {
    for (int st = 0; st < n_stages; ++st) {
      hipEvent_t a = plan->prof_events[((size_t)c * VDN_NUM_STAGES + st) * 2];
      hipEvent_t z = plan->prof_events[((size_t)c * VDN_NUM_STAGES + st) * 2 + 1];
      if (hipEventSynchronize(z) != hipSuccess) return VDN_ERR_HIP;
      float t = 0.f;
      if (hipEventElapsedTime(&t, a, z) != hipSuccess) return VDN_ERR_HIP;
      ms[st] += t;
    }
  }
  if (calls) *calls = plan->prof_count;
  return VDN_OK;
}

}  // extern "C"
