// Internal declarations shared by the host code and the kernel launchers of the VDN layer.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/vdn.h"

namespace vdn {

constexpr int kTextPad = 64;        // global (text, then audio) keys occupy [0, round_up(n_ctx, 64)) of a head's key space
constexpr int kMaxRanges = 4;       // text, window, frame 0, frame T-1

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Host-side description of the layer shape plus everything derived from it.
struct Shape {
  int T, N, C, n_text, H, d, anchors;
  vdn_dtype dtype;
  int n_audio;       // audio tokens: global softmax keys after the text, never written to the linear memory
  int n_ctx;         // n_text + n_audio: the global (context) tokens
  int Nc;            // number of chunks
  int ctx_pad;       // n_ctx rounded up to kTextPad
  int64_t Lk;        // key-space length per head: ctx_pad + T*N
  int64_t Ls;        // allocated key stride of the packed K/V: Lk + 128 zero keys of padding
  int64_t Ls8;       // key stride of the FP8 packed K/V: Lk + one zero 128-key tile
};

// Frame rules of "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section "Local
// Softmax and Long-Range Linear Memory": chunks of C consecutive frames; a chunk attends to itself
// and its two neighbours; the first and last frames are anchors seen by every frame and seeing every
// frame; the forward state covers the frames before the window and the reverse state those after
// it, neither covering window or boundary frames.  Host and device (the allocation-free forward
// builds its key-range table on the device).
__host__ __device__ inline bool is_boundary(const Shape& s, int t) { return s.anchors && (t == 0 || t == s.T - 1); }

// Key ranges of query frame t in a head's key space (see vdn_key_ranges); t == T gives the ranges
// of the context (text and audio) query rows: every key.  Writes min(count, max_ranges) ranges and
// returns the count.
__host__ __device__ inline int key_ranges(const Shape& s, int t, int64_t* r, int max_ranges) {
  int64_t tmp[2 * kMaxRanges];
  int n = 0;
  auto add = [&](int64_t a, int64_t b) {
    if (b > a) { tmp[2 * n] = a; tmp[2 * n + 1] = b; ++n; }
  };
  const int64_t base = s.ctx_pad, N = s.N;
  add(0, s.n_ctx);
  if (t == s.T || is_boundary(s, t)) {                                  // context rows, boundary frames
    add(base, base + (int64_t)s.T * N);
  } else {
    const int c = t / s.C;
    const int lo = c >= 1 ? (c - 1) * s.C : 0;
    const int hi = (c + 2) * s.C < s.T ? (c + 2) * s.C : s.T;
    if (s.anchors && lo > 0) add(base, base + N);                        // frame 0
    add(base + lo * N, base + hi * N);                                   // window
    if (s.anchors && s.T - 1 >= hi) add(base + (int64_t)(s.T - 1) * N, base + (int64_t)s.T * N);  // frame T-1
  }
  for (int i = 0; i < n && i < max_ranges; ++i) { r[2 * i] = tmp[2 * i]; r[2 * i + 1] = tmp[2 * i + 1]; }
  return n;
}

// Frames written into the forward (dir 0) / reverse (dir 1) state of query frame t, in order.
int scan_frames(const Shape& s, int t, int dir, int* frames, int max_frames);

// Device workspace layout (byte offsets from the workspace base).
struct Layout {
  size_t os;        // o_s [T*N][H][d] plan dtype
  size_t kp;        // packed keys  [H][Ls][d] bf16          (MFMA softmax path only)
  size_t vt;        // packed values, transposed [H][d][Ls] bf16
  size_t minv;      // M = (I+A)^-1  [T+1][H][d][d] f32
  size_t mhl;       // M as bf16 high and low planes [T+1][H][2][d][d] (MFMA scan only)
  size_t bw;        // B             [T+1][H][d][d] f32
  size_t cw;        // C = B M       [T+1][H][d][d] f32 (MFMA scan only)
  size_t pp;        // chunk maps P, P^T as bf16 hi/lo planes [Nc][H][2][2][d][d] (MFMA scan only)
  size_t qq;        // chunk maps Q_fwd, Q_rev [2][Nc][H][d][d] f32 (MFMA scan only)
  size_t states;    // S_fwd, S_rev  [2][Nc+1][H][d][d] f32
  size_t wt;        // transposed weights [4][d][d] bf16: Wg0^T, Wg1^T, Wp0^T, Wp1^T (MFMA epilogue)
  size_t wt8;       // MX epilogue: the same as E4M3 codes [4][d][d] bytes
  size_t wsc8;      // MX epilogue: their block scales (E8M0) [4][d][d/32] bytes
  size_t kmax_part; // largest key norm per 64-key block [H][Lk/64] f32  (MFMA softmax path only)
  size_t kmax;      // largest key norm per head [H] f32
  size_t flags;     // per-workgroup fallback flags of the MFMA softmax [softmax_grid] int32
  size_t k8;        // FP8 softmax: keys E4M3 [H][Ls8][d], values E4M3 transposed [H][d][Ls8]
  size_t v8;
  size_t part8;     // FP8 softmax: per 64-key block and head max |k|, max |v|, max key norm [H][Lk/64][3] f32
  size_t scale8;    // FP8 softmax: per head key and value scales [H][2] f32
  size_t lse;       // base-2 log of each softmax row's normaliser [T*N + n_ctx][H] f32, video rows then the
                    // context rows (not FP8 plans)
  size_t ranges;    // int32 [T+1][2*kMaxRanges] + int32 [T+1] counts (row T: context query rows)
  size_t total;
};
// Kernel selection per stage.
struct Kinds {
  bool softmax_mfma;
  bool softmax_fp8;   // FP8 (E4M3) softmax branch instead of the bf16 one
  bool stats_mfma;
  bool scan_mfma;
  bool epilogue_mfma;
  bool epilogue_mx;   // MXFP8 gate and projection products (with epilogue_mfma, d = 128)
};
Kinds choose_kinds(const Shape& s);
Layout make_layout(const Shape& s, const Kinds& k);

struct Buffers {
  void* os;
  uint16_t* kp;
  uint16_t* vt;
  float* minv;
  uint16_t* mhl;
  float* bw;
  float* cw;
  uint16_t* pp;
  float* qq;
  float* states;
  uint16_t* wt;
  uint8_t* wt8;        // MX epilogue weights and block scales, or nullptr
  uint8_t* wsc8;
  float* kmax_part;
  float* kmax;
  int* flags;
  const int* ranges;   // [T+1][2*kMaxRanges]
  const int* nranges;  // [T+1]
  uint8_t* k8;
  uint8_t* v8;
  float* part8;
  float* scale8;
  float* lse;          // [T*N + n_ctx][H] base-2 log of each row's softmax normaliser (video rows, then the
                       // context rows when they are computed), or nullptr
};

struct Inputs {
  const void *q, *k, *v;
  const float* beta;
  const void* text_kv;
  const void *gate_w, *proj_w;
  void* out;
  const float* alpha;  // [T][H][d] channel-wise decay gate of the inherited state, or nullptr (none)
  const void* ctx_q;   // [n_ctx][H][d] text and audio query rows, or nullptr (not computed)
  void* ctx_out;       // [n_ctx][H][d] their attention output (with ctx_q)
};

// Host-side helpers of the C ABI (abi.cpp).
Shape make_shape(int T, int N, int C, int n_text, int n_audio, int H, int d, int anchors, vdn_dtype dt);
bool shape_ok(int T, int N, int C, int n_text, int H, int d, int anchors);
// Validation of a plan's shape, dtype and flags (VDN_OK or the status vdn_plan_create_* returns).
vdn_status check_plan_args(int T, int N, int C, int n_text, int n_audio, int H, int d, int anchors,
                           vdn_dtype dtype, unsigned flags);
// Validation of a forward's pointers: presence, 16-byte alignment, and outputs disjoint (by byte
// range) from every input and from each other.
vdn_status check_forward_args(const Shape& s, const Inputs& in);
// Device buffers of a workspace laid out by make_layout at base ws.
Buffers make_buffers(char* ws, const Layout& lay, const Kinds& kinds, const Shape& s);
// Enqueue every stage of the forward on `main` (the linear branch on `side`, forked and joined
// through the two events, when side is not null); ev, if not null, receives the stage events
// [VDN_NUM_STAGES][2].  Returns the first launch error.
hipError_t enqueue_forward(const Shape& s, const Kinds& kinds, const Buffers& b, const Inputs& in, hipStream_t main,
                           hipStream_t side, hipEvent_t ev_fork, hipEvent_t ev_join, hipEvent_t* ev);
// A byte range [p, p + n) of caller memory; two ranges overlap when they share a byte.
struct Span {
  const void* p;
  size_t n;
};
bool spans_overlap(const Span& x, const Span& y);

// Backward pass.  Row segment for X^T Y reductions: rows [row0, row0 + nrows) of head `head`
// (head < 0: every head) of [rows][H][d] arrays.
struct Segment {
  int64_t row0;
  int nrows;
  int head;
};
// Backward workspace (device) and host-built tables.
struct BwdBuffers {
  const void* dout;                     // [T*N][H][d] plan dtype (the caller's)
  float *do_s, *do_l, *x_s, *x_l, *dz_s, *dz_l;   // [T*N][H][d] (do_s: generic kernels only)
  float *dsum, *lse;                    // [T*N + n_ctx][H]: video rows, then the context query rows
  float* partial;                       // [segments][splits][d][d]
  float* dread;                         // [Nc+2][H][d][d] readout adjoints (slots Nc, Nc+1: frames 0, T-1)
  float *zin, *dmf, *dbf;               // [2][T][H][d][d]
  float *gsym, *gdb;                    // [T+1][H][d][d]: dA + dA^T and dB per slot (0: text)
  float* dalf;                          // [2][T][H][d]
  float* ds0;                           // [2][H][d][d]
  const int* order;                     // [T] scanned frames, forward order
  const int* mslot;                     // [2][Nc+2] state index each readout slot reads
  const int* qranges;                   // [T+1][2*kMaxRanges] query-frame ranges per key slot
  const int* nqranges;                  // [T+1]
  const Segment *seg_all, *seg_read;    // 1 and (Nc+2)*H segments
  int splits_all, splits_read, nscan;
  // MFMA softmax backward (bf16 plans, d in {64, 128})
  uint16_t* dos16;                      // [T*N][H][d] do_s in bf16
  uint16_t* mimg;                       // matrix images of the merge (6 weights, 4 per chunk slot and head),
                                        // later of the token gradients (6 per frame slot and head)
  uint16_t *qt, *dot;                   // [H][d][Lq] transposed q, do_s (bf16); pad columns zero
  uint16_t *kt, *vp;                    // [H][d][Ls] transposed keys, [H][Ls][d] key-major values
  int64_t Lq;                           // T*N + round_up(n_ctx, 64) + 64 (context rows from column T*N)
  // workgroup tables of the two softmax transposes: entry w runs on XCD w % 8; an entry with a
  // negative first field is a workgroup without work
  const int4* kwork;                    // dK/dV: (key slot, first key, head, 0)
  int nkwork;
  const int2* qwork;                    // dQ: (query frame, query tile + QT head)
  int nqwork;
  // text and audio query rows (the joint backward with context rows)
  const void* dctx_out;                 // [n_ctx][H][d] plan dtype (the caller's), or nullptr: no context rows
  void* octx;                           // [n_ctx][H][d] plan dtype: their recomputed output
  float* do_ctx;                        // [n_ctx][H][d] dctx_out in fp32 (generic kernels)
};
struct BwdOutputs {
  float *dq, *dk, *dv, *dbeta, *dtext_kv, *dgate_w, *dproj_w, *dalpha;
  float* dctx_q;                        // [n_ctx][H][d] or nullptr (no context rows)
};
hipError_t launch_backward(const Shape& s, const Inputs& in, const Buffers& b, const BwdBuffers& w,
                           const BwdOutputs& o, bool mfma_softmax, hipStream_t st);
// partial[seg][split] = sum over the split's rows of x^T y (one of x, y fp32, the other bf16)
hipError_t launch_xty_mfma(int d, const void* x, bool x_f32, const void* y, bool y_f32, const Segment* segs, int nseg,
                           int splits, int H, float* partial, hipStream_t st);
hipError_t launch_frame_states_mfma(const Shape& s, const Inputs& in, const Buffers& b, const BwdBuffers& w,
                                   hipStream_t st);
hipError_t launch_scan_bwd_mfma(const Shape& s, const Inputs& in, const Buffers& b, const BwdBuffers& w,
                                hipStream_t st);
hipError_t launch_token_grads_mfma(const Shape& s, const Inputs& in, const BwdBuffers& w, const BwdOutputs& o,
                                   hipStream_t st);
hipError_t launch_merge_bwd_mfma(const Shape& s, const Inputs& in, const Buffers& b, const BwdBuffers& w,
                                 const BwdOutputs& o, hipStream_t st);
hipError_t launch_softmax_backward_mfma(const Shape& s, const Inputs& in, const Buffers& b, const BwdBuffers& w,
                                        const BwdOutputs& o, hipStream_t st);
// keys of one key slot that a workgroup of the MFMA dK/dV kernel covers (the host's block table)
int softmax_dkv_block_keys();
int softmax_dq_block_queries();

// Number of workgroups of the MFMA softmax launch.
// with_ctx: including the workgroups of the context query rows.
int softmax_grid(const Shape& s, bool with_ctx);
int softmax_fp8_grid(const Shape& s, bool with_ctx);

// Launchers (each returns hipGetLastError() after its launches).
hipError_t launch_prep_kv(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st);
hipError_t launch_softmax_simt(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st);
// after_first: if not null, recorded on st between the fixed-reference and the online-maximum launch
hipError_t launch_softmax_mfma(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st,
                               hipEvent_t after_first = nullptr);
hipError_t launch_prep_fp8(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st);
hipError_t launch_softmax_fp8(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st,
                              hipEvent_t after_first = nullptr);
hipError_t launch_vda_stats(const Shape& s, const Inputs& in, const Buffers& b, bool mfma, hipStream_t st);
hipError_t launch_vda_stats_mfma(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st);
hipError_t launch_vda_invert_mfma(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st);
hipError_t launch_vda_scan(const Shape& s, const Inputs& in, const Buffers& b, bool mfma, hipStream_t st);
hipError_t launch_vda_scan_mfma(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st);
hipError_t launch_epilogue(const Shape& s, const Inputs& in, const Buffers& b, bool mfma, hipStream_t st);
hipError_t launch_prep_weights(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st);
hipError_t launch_prep_weights_mx(const Shape& s, const Inputs& in, const Buffers& b, hipStream_t st);
hipError_t launch_epilogue_mfma(const Shape& s, const Inputs& in, const Buffers& b, bool mx, hipStream_t st);

}  // namespace vdn
