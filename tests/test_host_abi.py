"""Host-side checks of the C ABI library (no GPU): it loads, exports every symbol the header
declares, rejects invalid plans before touching the GPU, and its key ranges and scan order equal
the oracle's frame sets."""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import vdn_oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def vdn():
    from linear_video_attention_amd import vdn as binding
    return binding


def declared_functions():
    text = open(os.path.join(ROOT, "include", "vdn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vdn_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(vdn):
    names = declared_functions()
    assert len(names) >= 10
    handle = ctypes.CDLL(vdn.LIB_PATH)
    for name in names:
        assert hasattr(handle, name), name
    bound = {n for n, _, _ in vdn.SIGNATURES}
    assert set(names) == bound, set(names) ^ bound


def test_status_strings(vdn):
    for s in (0, -1, -2, -3, -4, -5):
        assert vdn.status_str(s)


@pytest.mark.parametrize("args,status", [
    ((0, 16, 2, 1, 1, 16, 1, 0), -1),      # T = 0
    ((4, 0, 2, 1, 1, 16, 1, 0), -1),       # N = 0
    ((4, 16, 0, 1, 1, 16, 1, 0), -1),      # C = 0
    ((4, 16, 2, -1, 1, 16, 1, 0), -1),     # n_text < 0
    ((4, 16, 2, 1, 0, 16, 1, 0), -1),      # H = 0
    ((4, 16, 2, 1, 1, 16, 2, 0), -1),      # anchors not 0/1
    ((4, 16, 2, 1, 1, 48, 1, 0), -2),      # unsupported d
    ((4, 16, 2, 1, 1, 16, 1, 7), -2),      # unknown dtype
    ((1 << 20, 1 << 12, 2, 1, 1, 16, 1, 1), -2),   # too many tokens
])
def test_invalid_plans_rejected_on_host(vdn, args, status):
    h = ctypes.c_void_p(1234)
    st = vdn.lib().vdn_plan_create(*args, ctypes.byref(h))
    assert st == status
    assert h.value is None


@pytest.mark.parametrize("flags", [2 | 4, 32, 1 << 31, 1 | 8, 1 | 16])
def test_invalid_plan_flags_rejected_on_host(vdn, flags):
    """Serial and overlapped order together, an unknown flag bit, or an FP8 softmax or MXFP8
    epilogue with the generic kernels are argument errors."""
    h = ctypes.c_void_p(1234)
    assert vdn.lib().vdn_plan_create_ex(4, 16, 2, 1, 1, 128, 1, 1, flags, ctypes.byref(h)) == -1
    assert h.value is None


@pytest.mark.parametrize("args", [
    (4, 16, 2, 1, 1, 128, 1, 0),     # fp32 plan
    (4, 16, 2, 1, 1, 64, 1, 1),      # d = 64
    (4, 24, 2, 1, 1, 128, 1, 1),     # N not a multiple of 16
])
def test_fp8_plan_limits_rejected_on_host(vdn, args):
    """The FP8 softmax takes bf16 plans with d = 128 and N a multiple of 16 only."""
    h = ctypes.c_void_p(1234)
    assert vdn.lib().vdn_plan_create_ex(*args, 8, ctypes.byref(h)) == -2
    assert h.value is None


@pytest.mark.parametrize("args", [
    (4, 16, 2, 1, 1, 128, 1, 0),     # fp32 plan
    (4, 16, 2, 1, 1, 64, 1, 1),      # d = 64
])
def test_fp8_epilogue_plan_limits_rejected_on_host(vdn, args):
    """The MXFP8 epilogue takes bf16 plans with d = 128 only."""
    h = ctypes.c_void_p(1234)
    assert vdn.lib().vdn_plan_create_ex(*args, 16, ctypes.byref(h)) == -2
    assert h.value is None


def test_joint_plan_argument_errors(vdn):
    """A negative audio count is an argument error; an audio count that pushes the context key
    space past the supported size is unsupported."""
    h = ctypes.c_void_p(1234)
    L = vdn.lib()
    assert L.vdn_plan_create_joint(4, 16, 2, 1, -1, 1, 16, 1, 0, 0, ctypes.byref(h)) == -1
    assert h.value is None
    assert L.vdn_plan_create_joint(4, 16, 2, 1, 1, 1, 48, 1, 0, 0, ctypes.byref(h)) == -2
    assert L.vdn_plan_create_joint(4, 16, 2, 1, (1 << 31) - 2, 1, 16, 1, 0, 0, ctypes.byref(h)) == -2
    assert L.vdn_plan_create_joint(4, 16, 2, 1, 0, 1, 16, 1, 0, 0, None) == -1
    assert L.vdn_forward_joint(None, *([None] * 12)) == -1


def test_measurement_helpers_reject_bad_arguments(vdn):
    x = ctypes.c_double()
    assert vdn.lib().vdn_measure_mfma_bf16_tflops(0, ctypes.byref(x)) == -1
    assert vdn.lib().vdn_measure_mfma_bf16_tflops(10, None) == -1
    assert vdn.lib().vdn_measure_copy_gbs(0, ctypes.byref(x)) == -1
    assert vdn.lib().vdn_measure_copy_gbs(1 << 20, None) == -1


def test_null_arguments_rejected(vdn):
    L = vdn.lib()
    assert L.vdn_plan_create(4, 16, 2, 1, 1, 16, 1, 0, None) == -1
    assert L.vdn_forward(None, *([None] * 9)) == -1
    assert L.vdn_forward_decay(None, *([None] * 10)) == -1
    assert L.vdn_backward(None, *([None] * 18)) == -1
    assert L.vdn_backward_joint(None, *([None] * 21)) == -1
    assert L.vdn_backward_after_forward(None, *([None] * 18)) == -1
    L.vdn_plan_destroy(None)                       # no-op
    assert L.vdn_plan_workspace_bytes(None) == 0
    assert L.vdn_profile_enable(None, 4) == -1
    assert vdn.lib().vdn_key_ranges(4, 16, 2, 1, 1, 9, None, 0) == -1


SHAPES = [(T, C, anchors) for T in (1, 2, 3, 5, 7, 16, 20, 31) for C in (1, 2, 3, 5) for anchors in (True, False)]


@pytest.mark.parametrize("T,C,anchors", SHAPES)
def test_key_ranges_match_oracle(vdn, T, C, anchors):
    N, n_text = 3, 5
    text_pad = 64
    for t in range(T):
        ranges = vdn.vdn_key_ranges(T, N, C, n_text, anchors, t)
        keys = []
        for a, b in ranges:
            assert a < b
            keys.extend(range(a, b))
        assert keys == sorted(keys) and len(set(keys)) == len(keys)
        expect = list(range(n_text)) + [text_pad + f * N + n for f in orc.key_frames(t, T, C, anchors) for n in range(N)]
        assert keys == expect, (t, ranges)


@pytest.mark.parametrize("T,C,anchors", SHAPES)
def test_scan_frames_match_oracle(vdn, T, C, anchors):
    for t in range(T):
        _, _, fwd, rev = orc.frame_sets(t, T, C, anchors)
        assert vdn.vdn_scan_frames(T, C, anchors, t, 0) == fwd
        assert vdn.vdn_scan_frames(T, C, anchors, t, 1) == rev[::-1]


def test_key_ranges_at_768p_workload(vdn):
    # interior query frame: text + window (15 frames) + both anchors = 26 624 keys
    ranges = vdn.vdn_key_ranges(75, 1536, 5, 512, True, 37)
    assert sum(b - a for a, b in ranges) == 512 + 17 * 1536
    # boundary query frame: text + every frame
    ranges = vdn.vdn_key_ranges(75, 1536, 5, 512, True, 74)
    assert sum(b - a for a, b in ranges) == 512 + 75 * 1536



# ---- the allocation-free forward: every check runs on the host before any GPU call ----

def _fake_spans(T, N, n_text, H, d, elt):
    """Disjoint, 256-byte aligned fake device addresses for q, k, v, beta, text_kv, gate_w,
    proj_w, out (never dereferenced: the calls below return before anything is enqueued, or fail
    at the first HIP call on a machine without a GPU)."""
    tok = T * N * H * d * elt
    sizes = [tok, tok, tok, (n_text + T * N) * H * 4, 2 * n_text * H * d * elt, 2 * d * d * elt, 2 * d * d * elt,
             tok]
    addr, out = 1 << 40, []
    for sz in sizes:
        out.append(addr)
        addr += (sz + 4095) // 4096 * 4096
    return out


def test_noalloc_rejects_before_touching_the_gpu(vdn):
    L = vdn.lib()
    # the 768p head share needs 0.63 GB of workspace: beyond the static scratch
    p = _fake_spans(75, 1536, 512, 5, 128, 2)
    assert L.vdn_forward_noalloc(75, 1536, 5, 512, 5, 128, 1, vdn.VDN_BF16, *p, None) == vdn.VDN_ERR_TOO_LARGE
    assert vdn.status_str(vdn.VDN_ERR_TOO_LARGE)
    p = _fake_spans(4, 64, 4, 1, 64, 2)
    assert L.vdn_forward_noalloc(4, 64, 2, 4, 1, 48, 1, vdn.VDN_BF16, *p, None) == vdn.VDN_ERR_UNSUPPORTED
    assert L.vdn_forward_noalloc(0, 64, 2, 4, 1, 64, 1, vdn.VDN_BF16, *p, None) == vdn.VDN_ERR_INVALID_ARG
    # out overlapping any input (here each input's first or last byte) is an argument error
    elt, tok = 2, 4 * 64 * 1 * 64 * 2
    for i in range(7):
        bad = list(p)
        bad[7] = p[i]
        assert L.vdn_forward_noalloc(4, 64, 2, 4, 1, 64, 1, vdn.VDN_BF16, *bad, None) == vdn.VDN_ERR_INVALID_ARG, i
    bad = list(p)
    bad[7] = p[5] - tok + 16                      # out's last 16 bytes are gate_w's first
    assert L.vdn_forward_noalloc(4, 64, 2, 4, 1, 64, 1, vdn.VDN_BF16, *bad, None) == vdn.VDN_ERR_INVALID_ARG
    bad = list(p)
    bad[0] += 8                                   # misaligned q
    assert L.vdn_forward_noalloc(4, 64, 2, 4, 1, 64, 1, vdn.VDN_BF16, *bad, None) == vdn.VDN_ERR_INVALID_ARG
    # valid arguments pass every host check; without a GPU the first HIP call fails
    try:
        import torch
        gpu = torch.cuda.is_available()
    except Exception:
        gpu = False
    if not gpu:
        assert L.vdn_forward_noalloc(4, 64, 2, 4, 1, 64, 1, vdn.VDN_BF16, *p, None) == vdn.VDN_ERR_HIP
