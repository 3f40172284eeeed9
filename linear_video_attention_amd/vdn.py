"""Thin ctypes binding of the VDN layer C ABI (``include/vdn.h``).

Argument marshalling only: tensors are checked for device, dtype, shape and contiguity, and their
device pointers are handed to the library; every step of the layer runs in the library's HIP
kernels.  There is no fallback: if ``libvdn.so`` is missing or no GPU is visible, calls raise.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libvdn.so")

VDN_OK, VDN_ERR_INVALID_ARG, VDN_ERR_UNSUPPORTED, VDN_ERR_OUT_OF_MEMORY, VDN_ERR_HIP = 0, -1, -2, -3, -4
VDN_ERR_TOO_LARGE = -5
VDN_F32, VDN_BF16 = 0, 1
VDN_FLAG_GENERIC_KERNELS = 1
VDN_FLAG_SERIAL = 2
VDN_FLAG_OVERLAP = 4
VDN_FLAG_FP8_SOFTMAX = 8
VDN_FLAG_FP8_EPILOGUE = 16
VDN_BUF_OS, VDN_BUF_STATES, VDN_BUF_MINV, VDN_BUF_BW = 0, 1, 2, 3
VDN_BUF_K8, VDN_BUF_V8, VDN_BUF_SCALES8 = 4, 5, 6
STAGES = ("softmax", "prep", "vda_stats", "vda_scan", "epilogue", "total", "softmax_first")
(VDN_STAGE_SOFTMAX, VDN_STAGE_PREP, VDN_STAGE_VDA_STATS, VDN_STAGE_VDA_SCAN, VDN_STAGE_EPILOGUE, VDN_STAGE_TOTAL,
 VDN_STAGE_SOFTMAX_FIRST) = range(7)

# every symbol include/vdn.h declares: (name, restype, argtypes)
_c_int, _c_size, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
SIGNATURES = [
    ("vdn_plan_create", _c_int, [_c_int] * 7 + [_c_int, ctypes.POINTER(_vp)]),
    ("vdn_plan_create_ex", _c_int, [_c_int] * 7 + [_c_int, ctypes.c_uint, ctypes.POINTER(_vp)]),
    ("vdn_plan_create_joint", _c_int, [_c_int] * 8 + [_c_int, ctypes.c_uint, ctypes.POINTER(_vp)]),
    ("vdn_forward", _c_int, [_vp] * 10),
    ("vdn_forward_decay", _c_int, [_vp] * 11),
    ("vdn_forward_joint", _c_int, [_vp] * 13),
    ("vdn_forward_noalloc", _c_int, [_c_int] * 8 + [_vp] * 9),
    ("vdn_backward", _c_int, [_vp] * 19),
    ("vdn_backward_after_forward", _c_int, [_vp] * 19),
    ("vdn_backward_joint", _c_int, [_vp] * 22),
    ("vdn_plan_destroy", None, [_vp]),
    ("vdn_status_str", ctypes.c_char_p, [_c_int]),
    ("vdn_plan_workspace_bytes", _c_size, [_vp]),
    ("vdn_key_ranges", _c_int, [_c_int] * 6 + [ctypes.POINTER(ctypes.c_int64), _c_int]),
    ("vdn_scan_frames", _c_int, [_c_int] * 5 + [ctypes.POINTER(_c_int), _c_int]),
    ("vdn_debug_buffer_bytes", _c_int, [_vp, _c_int, ctypes.POINTER(_c_size)]),
    ("vdn_debug_copy", _c_int, [_vp, _c_int, _vp, _c_size, _vp]),
    ("vdn_debug_epilogue", _c_int, [_vp] * 8),
    ("vdn_profile_enable", _c_int, [_vp, _c_int]),
    ("vdn_profile_read", _c_int, [_vp, ctypes.POINTER(ctypes.c_float), _c_int, ctypes.POINTER(_c_int)]),
    ("vdn_plan_kernel_kind", _c_int, [_vp, _c_int, ctypes.POINTER(_c_int)]),
    ("vdn_measure_mfma_bf16_tflops", _c_int, [_c_int, ctypes.POINTER(ctypes.c_double)]),
    ("vdn_measure_copy_gbs", _c_int, [_c_size, ctypes.POINTER(ctypes.c_double)]),
]

_lib = None


class VdnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} ({status})")


def lib() -> ctypes.CDLL:
    """Load ``libvdn.so`` (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        handle = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_str(status: int) -> str:
    return lib().vdn_status_str(status).decode()


def _check(status: int, what: str):
    if status != VDN_OK:
        raise VdnError(status, what)


# ---- host-only helpers ----

def vdn_key_ranges(T, N, C, n_text, anchors, t, max_ranges=4):
    buf = (ctypes.c_int64 * (2 * max_ranges))()
    n = lib().vdn_key_ranges(T, N, C, n_text, int(anchors), t, buf, max_ranges)
    if n < 0:
        raise ValueError("invalid arguments")
    return [(buf[2 * i], buf[2 * i + 1]) for i in range(min(n, max_ranges))]


def vdn_scan_frames(T, C, anchors, t, direction):
    buf = (ctypes.c_int * max(T, 1))()
    n = lib().vdn_scan_frames(T, C, int(anchors), t, direction, buf, T)
    if n < 0:
        raise ValueError("invalid arguments")
    return [buf[i] for i in range(n)]


def measure_mfma_bf16_tflops(iters=20000):
    """Dense bf16 TFLOP/s of a tight MFMA loop on this GPU (on-box roofline reference)."""
    x = ctypes.c_double()
    _check(lib().vdn_measure_mfma_bf16_tflops(iters, ctypes.byref(x)), "vdn_measure_mfma_bf16_tflops")
    return x.value


def measure_copy_gbs(nbytes=1 << 30):
    """Device-to-device copy GB/s (read + write) over ``nbytes`` (on-box HBM reference)."""
    x = ctypes.c_double()
    _check(lib().vdn_measure_copy_gbs(nbytes, ctypes.byref(x)), "vdn_measure_copy_gbs")
    return x.value


# ---- plan ----

def vdn_plan_create(T, N, C, n_text, H, d, anchors=True, dtype="bf16", generic=False, serial=False,
                    overlap=False, n_audio=0, fp8=False, fp8_epilogue=False):
    """Create a plan; returns an opaque handle (int).  ``dtype`` is "bf16" or "fp32"; ``n_audio``
    audio tokens follow the text tokens (a joint plan); ``fp8`` selects the FP8 softmax branch,
    ``fp8_epilogue`` the MXFP8 gate and projection products."""
    dt = {"bf16": VDN_BF16, "fp32": VDN_F32}[dtype]
    h = _vp()
    flags = ((VDN_FLAG_GENERIC_KERNELS if generic else 0) | (VDN_FLAG_SERIAL if serial else 0)
             | (VDN_FLAG_OVERLAP if overlap else 0) | (VDN_FLAG_FP8_SOFTMAX if fp8 else 0)
             | (VDN_FLAG_FP8_EPILOGUE if fp8_epilogue else 0))
    if n_audio:
        _check(lib().vdn_plan_create_joint(T, N, C, n_text, n_audio, H, d, int(anchors), dt, flags,
                                           ctypes.byref(h)), "vdn_plan_create_joint")
    else:
        _check(lib().vdn_plan_create_ex(T, N, C, n_text, H, d, int(anchors), dt, flags, ctypes.byref(h)),
               "vdn_plan_create")
    return h.value


def vdn_plan_destroy(plan):
    lib().vdn_plan_destroy(plan)


def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def vdn_forward(plan, q, k, v, beta, text_kv, gate_w, proj_w, out, stream=None):
    """Enqueue the layer forward on ``stream`` (default: torch's current stream).  All arguments
    are device tensors laid out as in ``include/vdn.h``; ``out`` is written."""
    ptr = lambda x: None if x is None else x.data_ptr()
    _check(lib().vdn_forward(plan, ptr(q), ptr(k), ptr(v), ptr(beta), ptr(text_kv), ptr(gate_w),
                             ptr(proj_w), ptr(out), _stream_ptr(stream)), "vdn_forward")


def vdn_forward_decay(plan, q, k, v, beta, text_kv, alpha, gate_w, proj_w, out, stream=None):
    """As ``vdn_forward`` with the channel-wise decay gate ``alpha`` (fp32 [T][H][d] device tensor)
    on the linear branch's inherited state."""
    ptr = lambda x: None if x is None else x.data_ptr()
    _check(lib().vdn_forward_decay(plan, ptr(q), ptr(k), ptr(v), ptr(beta), ptr(text_kv), ptr(alpha),
                                   ptr(gate_w), ptr(proj_w), ptr(out), _stream_ptr(stream)),
           "vdn_forward_decay")


def vdn_forward_joint(plan, q, k, v, beta, ctx_q, ctx_kv, alpha, gate_w, proj_w, out, ctx_out, stream=None):
    """The joint sequence: the video rows as ``vdn_forward`` / ``vdn_forward_decay`` (``alpha`` may
    be None) and, with ``ctx_q`` and ``ctx_out``, the text and audio query rows."""
    ptr = lambda x: None if x is None else x.data_ptr()
    _check(lib().vdn_forward_joint(plan, ptr(q), ptr(k), ptr(v), ptr(beta), ptr(ctx_q), ptr(ctx_kv),
                                   ptr(alpha), ptr(gate_w), ptr(proj_w), ptr(out), ptr(ctx_out),
                                   _stream_ptr(stream)), "vdn_forward_joint")


def vdn_forward_noalloc(T, N, C, n_text, H, d, anchors, dtype, q, k, v, beta, text_kv, gate_w, proj_w, out,
                        stream=None):
    """The layer forward without a plan, on the library's static device scratch (allocates nothing;
    shapes whose workspace exceeds the scratch raise VDN_ERR_TOO_LARGE).  ``dtype`` is "bf16" or
    "fp32"; tensors as ``vdn_forward``; ``out`` is written."""
    dt = {"bf16": VDN_BF16, "fp32": VDN_F32}[dtype]
    ptr = lambda x: None if x is None else x.data_ptr()
    _check(lib().vdn_forward_noalloc(T, N, C, n_text, H, d, int(anchors), dt, ptr(q), ptr(k), ptr(v), ptr(beta),
                                     ptr(text_kv), ptr(gate_w), ptr(proj_w), ptr(out),
                                     None if stream is None and not _has_gpu() else _stream_ptr(stream)),
           "vdn_forward_noalloc")


def _has_gpu():
    import torch
    return torch.cuda.is_available()


class Plan:
    """Owning wrapper of a plan with argument checks on torch tensors."""

    def __init__(self, T, N, C, n_text, H, d, anchors=True, dtype="bf16", generic=False, serial=False,
                 overlap=False, n_audio=0, fp8=False, fp8_epilogue=False):
        import torch
        if not torch.cuda.is_available():
            raise RuntimeError("no GPU visible: the VDN layer runs only on the GPU")
        self.T, self.N, self.C, self.n_text, self.H, self.d = T, N, C, n_text, H, d
        self.n_audio = n_audio
        self.n_ctx = n_text + n_audio
        self.anchors = bool(anchors)
        self.dtype = dtype
        self.torch_dtype = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
        self.Nc = (T + C - 1) // C
        self.fp8 = bool(fp8)
        self.Ls8 = (self.n_ctx + 63) // 64 * 64 + T * N + 128
        self.fp8_epilogue = bool(fp8_epilogue)
        self.handle = vdn_plan_create(T, N, C, n_text, H, d, anchors, dtype, generic, serial, overlap, n_audio, fp8,
                                      fp8_epilogue)

    def close(self):
        if self.handle:
            vdn_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _expect(self, name, x, shape, dtype):
        import torch
        if x is None or not isinstance(x, torch.Tensor):
            raise TypeError(f"{name} must be a tensor")
        if not x.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if tuple(x.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(x.shape)}, expected {tuple(shape)}")
        if x.dtype != dtype:
            raise ValueError(f"{name} has dtype {x.dtype}, expected {dtype}")
        if not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    def forward(self, q, k, v, beta, text_kv, gate_w, proj_w, out=None, stream=None, alpha=None,
                ctx_q=None, ctx_out=None):
        """The layer forward; with ``alpha`` ([T, H, d] fp32) the linear branch's decay gate.
        ``text_kv`` holds the context tokens ([2, n_text + n_audio, H, d]).  With ``ctx_q``
        ([n_ctx, H, d]) the text and audio query rows are computed too, into ``ctx_out`` (a new
        tensor when None); the call then returns ``(out, ctx_out)``."""
        import torch
        TN, H, d = self.T * self.N, self.H, self.d
        dt = self.torch_dtype
        for name, x in (("q", q), ("k", k), ("v", v)):
            self._expect(name, x, (TN, H, d), dt)
        self._expect("beta", beta, (self.n_text + TN, H), torch.float32)
        if self.n_ctx > 0:
            self._expect("text_kv", text_kv, (2, self.n_ctx, H, d), dt)
        self._expect("gate_w", gate_w, (2, d, d), dt)
        self._expect("proj_w", proj_w, (2, d, d), dt)
        if out is None:
            out = torch.empty((TN, H, d), dtype=dt, device=q.device)
        self._expect("out", out, (TN, H, d), dt)
        if alpha is not None:
            self._expect("alpha", alpha, (self.T, H, d), torch.float32)
        tkv = text_kv if self.n_ctx > 0 else None
        if ctx_q is not None:
            self._expect("ctx_q", ctx_q, (self.n_ctx, H, d), dt)
            if ctx_out is None:
                ctx_out = torch.empty((self.n_ctx, H, d), dtype=dt, device=q.device)
            self._expect("ctx_out", ctx_out, (self.n_ctx, H, d), dt)
            vdn_forward_joint(self.handle, q, k, v, beta, ctx_q, tkv, alpha, gate_w, proj_w, out, ctx_out, stream)
            return out, ctx_out
        if alpha is None:
            vdn_forward(self.handle, q, k, v, beta, tkv, gate_w, proj_w, out, stream)
        else:
            vdn_forward_decay(self.handle, q, k, v, beta, tkv, alpha, gate_w, proj_w, out, stream)
        return out

    def backward(self, q, k, v, beta, text_kv, gate_w, proj_w, dout, alpha=None, stream=None,
                 after_forward=False, ctx_q=None, dctx_out=None):
        """Input gradients of the layer for the output gradient ``dout``; returns a dict of float32
        device tensors (q, k, v, beta, text_kv, gate_w, proj_w and, with ``alpha``, alpha).
        ``text_kv`` and its gradient hold the context tokens ([2, n_text + n_audio, H, d]).
        ``after_forward=True`` reuses the intermediates of the plan's most recent forward on the
        same inputs (vdn_backward_after_forward) instead of recomputing them.  With ``ctx_q`` and
        ``dctx_out`` ([n_ctx, H, d]) the text and audio query rows are included
        (vdn_backward_joint) and the dict also holds their gradient ctx_q."""
        import torch
        TN, H, d = self.T * self.N, self.H, self.d
        dt = self.torch_dtype
        for name, x in (("q", q), ("k", k), ("v", v), ("dout", dout)):
            self._expect(name, x, (TN, H, d), dt)
        self._expect("beta", beta, (self.n_text + TN, H), torch.float32)
        if self.n_ctx > 0:
            self._expect("text_kv", text_kv, (2, self.n_ctx, H, d), dt)
        self._expect("gate_w", gate_w, (2, d, d), dt)
        self._expect("proj_w", proj_w, (2, d, d), dt)
        if alpha is not None:
            self._expect("alpha", alpha, (self.T, H, d), torch.float32)
        joint = ctx_q is not None or dctx_out is not None
        if joint:
            if after_forward:
                raise ValueError("the context rows are recomputed: after_forward does not take them")
            self._expect("ctx_q", ctx_q, (self.n_ctx, H, d), dt)
            self._expect("dctx_out", dctx_out, (self.n_ctx, H, d), dt)
        f32 = dict(dtype=torch.float32, device=q.device)
        g = dict(q=torch.empty((TN, H, d), **f32), k=torch.empty((TN, H, d), **f32),
                 v=torch.empty((TN, H, d), **f32), beta=torch.empty((self.n_text + TN, H), **f32),
                 text_kv=torch.empty((2, self.n_ctx, H, d), **f32) if self.n_ctx > 0 else None,
                 gate_w=torch.empty((2, d, d), **f32), proj_w=torch.empty((2, d, d), **f32),
                 alpha=torch.empty((self.T, H, d), **f32) if alpha is not None else None,
                 ctx_q=torch.empty((self.n_ctx, H, d), **f32) if joint and self.n_ctx > 0 else None)
        ptr = lambda x: None if x is None else x.data_ptr()
        tkv = text_kv if self.n_ctx > 0 else None
        if joint:
            _check(lib().vdn_backward_joint(self.handle, ptr(q), ptr(k), ptr(v), ptr(beta), ptr(ctx_q), ptr(tkv),
                                            ptr(alpha), ptr(gate_w), ptr(proj_w), ptr(dout), ptr(dctx_out),
                                            ptr(g["q"]), ptr(g["k"]), ptr(g["v"]), ptr(g["beta"]), ptr(g["ctx_q"]),
                                            ptr(g["text_kv"]), ptr(g["gate_w"]), ptr(g["proj_w"]), ptr(g["alpha"]),
                                            _stream_ptr(stream)), "vdn_backward_joint")
        else:
            name = "vdn_backward_after_forward" if after_forward else "vdn_backward"
            _check(getattr(lib(), name)(self.handle, ptr(q), ptr(k), ptr(v), ptr(beta), ptr(tkv), ptr(alpha),
                                        ptr(gate_w), ptr(proj_w), ptr(dout), ptr(g["q"]), ptr(g["k"]), ptr(g["v"]),
                                        ptr(g["beta"]), ptr(g["text_kv"]), ptr(g["gate_w"]), ptr(g["proj_w"]),
                                        ptr(g["alpha"]), _stream_ptr(stream)), name)
        return {key: val for key, val in g.items() if val is not None}

    def debug_buffer(self, which, stream=None):
        """Copy an intermediate buffer of the last forward into a new device tensor."""
        import torch
        nbytes = ctypes.c_size_t()
        _check(lib().vdn_debug_buffer_bytes(self.handle, which, ctypes.byref(nbytes)), "vdn_debug_buffer_bytes")
        if which == VDN_BUF_OS:
            dst = torch.empty((self.T * self.N, self.H, self.d), dtype=self.torch_dtype, device="cuda")
        elif which == VDN_BUF_STATES:
            dst = torch.empty((2, self.Nc + 1, self.H, self.d, self.d), dtype=torch.float32, device="cuda")
        elif which == VDN_BUF_K8:
            dst = torch.empty((self.H, self.Ls8, self.d), dtype=torch.uint8, device="cuda")
        elif which == VDN_BUF_V8:
            dst = torch.empty((self.H, self.d, self.Ls8), dtype=torch.uint8, device="cuda")
        elif which == VDN_BUF_SCALES8:
            dst = torch.empty((self.H, 2), dtype=torch.float32, device="cuda")
        else:
            dst = torch.empty((self.T + 1, self.H, self.d, self.d), dtype=torch.float32, device="cuda")
        assert dst.numel() * dst.element_size() == nbytes.value
        _check(lib().vdn_debug_copy(self.handle, which, dst.data_ptr(), nbytes.value, _stream_ptr(stream)),
               "vdn_debug_copy")
        return dst

    def debug_epilogue(self, q, o_s, states, gate_w, proj_w, out=None, stream=None):
        """The plan's epilogue alone on a given softmax output o_s [T*N, H, d] and chunk-state
        buffer states [2, Nc+1, H, d, d] (float32); returns out [T*N, H, d]."""
        import torch
        shp = (self.T * self.N, self.H, self.d)
        for name, t, dt, want in (("q", q, self.torch_dtype, shp), ("o_s", o_s, self.torch_dtype, shp),
                                  ("states", states, torch.float32, (2, self.Nc + 1, self.H, self.d, self.d)),
                                  ("gate_w", gate_w, self.torch_dtype, (2, self.d, self.d)),
                                  ("proj_w", proj_w, self.torch_dtype, (2, self.d, self.d))):
            if t.dtype != dt or tuple(t.shape) != want or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name}: expected a contiguous CUDA {dt} tensor of shape {want}")
        if out is None:
            out = torch.empty(shp, dtype=self.torch_dtype, device="cuda")
        _check(lib().vdn_debug_epilogue(self.handle, q.data_ptr(), o_s.data_ptr(), states.data_ptr(), gate_w.data_ptr(),
                                        proj_w.data_ptr(), out.data_ptr(), _stream_ptr(stream)), "vdn_debug_epilogue")
        return out

    def workspace_bytes(self):
        return lib().vdn_plan_workspace_bytes(self.handle)

    def kernel_kind(self, stage):
        kind = ctypes.c_int()
        _check(lib().vdn_plan_kernel_kind(self.handle, stage, ctypes.byref(kind)), "vdn_plan_kernel_kind")
        return kind.value

    def profile_enable(self, max_calls):
        _check(lib().vdn_profile_enable(self.handle, max_calls), "vdn_profile_enable")

    def profile_read(self):
        """Summed milliseconds per stage over the recorded forwards, and their count."""
        ms = (ctypes.c_float * len(STAGES))()
        calls = ctypes.c_int()
        _check(lib().vdn_profile_read(self.handle, ms, len(STAGES), ctypes.byref(calls)), "vdn_profile_read")
        return {name: ms[i] for i, name in enumerate(STAGES)}, calls.value
