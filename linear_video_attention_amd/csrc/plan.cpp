// Host-side plan logic of the VDN layer: scan order of the linear branch, workspace layout and
// kernel selection (the key ranges of the softmax branch are in vdn_internal.h).  No GPU calls.
//
// Frame rules from "Video DeltaNet: Near-Lossless Hybrid Attention for Video Models", section
// "Local Softmax and Long-Range Linear Memory": the forward state covers the non-boundary frames
// before the window and the reverse state those after it.
#include "vdn_internal.h"

#include <algorithm>

namespace vdn {

int scan_frames(const Shape& s, int t, int dir, int* frames, int max_frames) {
  int n = 0;
  if (is_boundary(s, t)) return 0;
  const int c = t / s.C;
  if (dir == 0) {
    for (int f = 0; f < s.T; ++f)
      if (!is_boundary(s, f) && f / s.C <= c - 2) { if (n < max_frames) frames[n] = f; ++n; }
  } else {
    for (int f = s.T - 1; f >= 0; --f)
      if (!is_boundary(s, f) && f / s.C >= c + 2) { if (n < max_frames) frames[n] = f; ++n; }
  }
  return n;
}

Layout make_layout(const Shape& s, const Kinds& k) {
  const bool mfma_softmax = k.softmax_mfma, mfma_epilogue = k.epilogue_mfma;
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += (size_t)round_up((int64_t)bytes, 256); return o; };
  const size_t elt = s.dtype == VDN_BF16 ? 2 : 4;
  const size_t tok = (size_t)s.T * s.N * s.H * s.d;
  const size_t dd = (size_t)s.d * s.d;
  L.os = take(tok * elt);
  L.kp = mfma_softmax ? take((size_t)s.H * s.Ls * s.d * 2) : 0;
  L.vt = mfma_softmax ? take((size_t)s.H * s.Ls * s.d * 2) : 0;
  L.minv = take((size_t)(s.T + 1) * s.H * dd * 4);
  L.bw = take((size_t)(s.T + 1) * s.H * dd * 4);
  L.mhl = k.scan_mfma ? take((size_t)(s.T + 1) * s.H * dd * 4) : 0;
  L.cw = k.scan_mfma ? take((size_t)(s.T + 1) * s.H * dd * 4) : 0;
  L.pp = k.scan_mfma ? take((size_t)s.Nc * s.H * 4 * dd * 2) : 0;
  L.qq = k.scan_mfma ? take((size_t)2 * s.Nc * s.H * dd * 4) : 0;
  L.states = take((size_t)2 * (s.Nc + 1) * s.H * dd * 4);
  L.wt = mfma_epilogue ? take((size_t)4 * dd * 2) : 0;
  L.wt8 = k.epilogue_mx ? take((size_t)4 * dd) : 0;
  L.wsc8 = k.epilogue_mx ? take((size_t)4 * dd / 32) : 0;
  L.kmax_part = mfma_softmax ? take((size_t)s.H * ((s.Lk + 63) / 64) * 4) : 0;
  L.kmax = (mfma_softmax || k.softmax_fp8) ? take((size_t)s.H * 4) : 0;
  L.flags = mfma_softmax ? take((size_t)softmax_grid(s, true) * 4) : k.softmax_fp8 ? take((size_t)softmax_fp8_grid(s, true) * 4) : 0;
  L.k8 = k.softmax_fp8 ? take((size_t)s.H * s.Ls8 * s.d) : 0;
  L.v8 = k.softmax_fp8 ? take((size_t)s.H * s.Ls8 * s.d) : 0;
  L.part8 = k.softmax_fp8 ? take((size_t)s.H * ((s.Lk + 63) / 64) * 3 * 4) : 0;
  L.scale8 = k.softmax_fp8 ? take((size_t)s.H * 2 * 4) : 0;
  L.lse = k.softmax_fp8 ? 0 : take(((size_t)s.T * s.N + s.n_ctx) * s.H * 4);
  L.ranges = take((size_t)(s.T + 1) * (2 * kMaxRanges + 1) * 4);
  L.total = off;
  return L;
}

Kinds choose_kinds(const Shape& s) {
  Kinds k{};
  const bool bf16 = s.dtype == VDN_BF16;
  // lane offsets into one head's packed V^T are 32-bit: d * Ls * 2 bytes must stay below 2^31
  k.softmax_mfma = bf16 && (s.d == 64 || s.d == 128) && s.N % 8 == 0 && (int64_t)s.d * s.Ls * 2 < (int64_t(1) << 31);
  k.stats_mfma = bf16 && (s.d == 64 || s.d == 128);
  k.scan_mfma = k.stats_mfma;     // the MFMA statistics stage writes the MFMA scan's operands
  k.epilogue_mfma = bf16 && (s.d == 64 || s.d == 128);
  return k;
}

}  // namespace vdn
