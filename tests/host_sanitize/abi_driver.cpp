// Host-side driver of the C ABI for the address and undefined-behaviour sanitizers: exercises the
// entry points that run without a GPU (key ranges, scan order, argument validation, status strings,
// the allocation-free forward's host checks) over many shapes and checks their results against the
// frame rules written out independently here.  Exit status 0 means every check passed and the
// sanitizers reported nothing.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../include/vdn.h"

static int failures = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

// Frames whose keys query frame t sees (window of chunks c-1..c+1, anchors 0 and T-1, every frame
// for the anchors themselves), as a bitmap.
static std::vector<int> visible_frames(int T, int C, int anchors, int t) {
  std::vector<int> vis(T, 0);
  const bool bnd = anchors && (t == 0 || t == T - 1);
  for (int f = 0; f < T; ++f) {
    const int dc = f / C - t / C;
    if (bnd || (dc >= -1 && dc <= 1) || (anchors && (f == 0 || f == T - 1))) vis[f] = 1;
  }
  return vis;
}

int main() {
  for (int s = -6; s <= 0; ++s) CHECK(vdn_status_str((vdn_status)s) != nullptr);
  CHECK(vdn_status_str((vdn_status)7) != nullptr);
  vdn_plan_destroy(nullptr);
  CHECK(vdn_plan_workspace_bytes(nullptr) == 0);

  // key ranges and scan order over many shapes
  for (int T = 1; T <= 23; ++T)
    for (int C = 1; C <= 6; ++C)
      for (int anchors = 0; anchors <= 1; ++anchors)
        for (int n_text : {0, 1, 63, 64, 65}) {
          const int N = 7, pad = (n_text + 63) / 64 * 64;
          for (int t = 0; t < T; ++t) {
            int64_t r[8];
            const int n = vdn_key_ranges(T, N, C, n_text, anchors, t, r, 4);
            CHECK(n >= 1 && n <= 4);
            std::vector<int> seen(T, 0);
            int64_t prev_end = -1, text_keys = 0;
            for (int i = 0; i < n && i < 4; ++i) {
              CHECK(r[2 * i] < r[2 * i + 1]);
              CHECK(r[2 * i] >= prev_end && r[2 * i] >= 0);   // ascending, disjoint
              prev_end = r[2 * i + 1];
              for (int64_t key = r[2 * i]; key < r[2 * i + 1]; ++key) {
                if (key < n_text) { ++text_keys; continue; }
                CHECK(key >= pad && key < pad + (int64_t)T * N);
                if (key >= pad) seen[(key - pad) / N] += 1;
              }
            }
            CHECK(text_keys == n_text);
            const std::vector<int> vis = visible_frames(T, C, anchors, t);
            for (int f = 0; f < T; ++f) CHECK(seen[f] == (vis[f] ? N : 0));
            // scan order: forward frames before the window, reverse after, never a boundary frame
            std::vector<int> fr(T + 1, -1);
            const int nf = vdn_scan_frames(T, C, anchors, t, 0, fr.data(), T);
            const int nr = vdn_scan_frames(T, C, anchors, t, 1, fr.data(), T);
            CHECK(nf >= 0 && nr >= 0);
            int count_f = 0, count_r = 0;
            const bool bnd = anchors && (t == 0 || t == T - 1);
            for (int f = 0; f < T; ++f) {
              const bool b = anchors && (f == 0 || f == T - 1);
              if (!bnd && !b && f / C <= t / C - 2) ++count_f;
              if (!bnd && !b && f / C >= t / C + 2) ++count_r;
            }
            CHECK(nf == count_f && nr == count_r);
            // short output buffers are honoured
            int one = -7;
            CHECK(vdn_scan_frames(T, C, anchors, t, 0, &one, 1) == count_f);
            CHECK(vdn_key_ranges(T, N, C, n_text, anchors, t, r, 1) == n);
          }
        }
  // invalid host arguments
  int64_t r[8];
  int fr[4];
  CHECK(vdn_key_ranges(0, 4, 2, 0, 1, 0, r, 4) == -1);
  CHECK(vdn_key_ranges(4, 4, 2, 0, 1, 4, r, 4) == -1);
  CHECK(vdn_key_ranges(4, 4, 2, 0, 1, 0, nullptr, 4) == -1);
  CHECK(vdn_scan_frames(4, 2, 1, 0, 2, fr, 4) == -1);
  CHECK(vdn_scan_frames(4, 2, 3, 0, 0, fr, 4) == -1);
  vdn_plan* p = reinterpret_cast<vdn_plan*>(0x1234);
  CHECK(vdn_plan_create(0, 16, 2, 1, 1, 16, 1, VDN_F32, &p) == VDN_ERR_INVALID_ARG && p == nullptr);
  CHECK(vdn_plan_create(4, 16, 2, 1, 1, 48, 1, VDN_F32, &p) == VDN_ERR_UNSUPPORTED);
  CHECK(vdn_plan_create_ex(4, 16, 2, 1, 1, 16, 1, VDN_F32, 3u << 8, &p) == VDN_ERR_INVALID_ARG);
  CHECK(vdn_plan_create_ex(4, 16, 2, 1, 1, 128, 1, VDN_BF16, VDN_FLAG_SERIAL | VDN_FLAG_OVERLAP, &p) ==
        VDN_ERR_INVALID_ARG);
  CHECK(vdn_plan_create_ex(4, 16, 2, 1, 1, 64, 1, VDN_BF16, VDN_FLAG_FP8_SOFTMAX, &p) == VDN_ERR_UNSUPPORTED);
  CHECK(vdn_plan_create_joint(4, 16, 2, 1, -1, 1, 16, 1, VDN_F32, 0, &p) == VDN_ERR_INVALID_ARG);
  CHECK(vdn_plan_create(4, 16, 2, 1, 1, 16, 1, VDN_F32, nullptr) == VDN_ERR_INVALID_ARG);
  CHECK(vdn_forward(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) ==
        VDN_ERR_INVALID_ARG);
  // the allocation-free forward's host checks (fake, never dereferenced addresses)
  const uintptr_t base = uintptr_t(1) << 40;
  const void* a[8];
  for (int i = 0; i < 8; ++i) a[i] = reinterpret_cast<const void*>(base + (uintptr_t)i * (1u << 24));
  CHECK(vdn_forward_noalloc(75, 1536, 5, 512, 5, 128, 1, VDN_BF16, a[0], a[1], a[2], (const float*)a[3], a[4], a[5],
                            a[6], (void*)a[7], nullptr) == VDN_ERR_TOO_LARGE);
  CHECK(vdn_forward_noalloc(4, 64, 2, 4, 1, 64, 1, VDN_BF16, a[0], a[1], a[2], (const float*)a[3], a[4], a[5], a[6],
                            (void*)a[3], nullptr) == VDN_ERR_INVALID_ARG);
  CHECK(vdn_forward_noalloc(4, 64, 2, 4, 1, 64, 1, VDN_BF16, a[0], a[1], a[2], (const float*)a[3], a[4], a[5], a[6],
                            (void*)((uintptr_t)a[7] + 4), nullptr) == VDN_ERR_INVALID_ARG);
  if (failures) std::fprintf(stderr, "%d checks failed\n", failures);
  else std::printf("host ABI driver: all checks passed\n");
  return failures ? 1 : 0;
}
