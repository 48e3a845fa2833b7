"""ctypes binding of libpfa_attn.so (the C ABI in include/pfa_attn.h).

Argument marshalling only: shapes and data pointers of torch tensors on the GPU
and the current HIP stream go to the C entry points; every step of the
attention runs in the library's HIP kernels.  torch supplies device memory and
streams.  There is no fallback: a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libpfa_attn.so")

MODES = {"bf16_out": 0, "fp32_out": 1, "tie_aware_softmax": 2}
DELTA_SRC = {"do_o": 0, "dp_p": 1, "do_ohp": 2}
PFA_OK, PFA_ERR_INVALID, PFA_ERR_UNSUPPORTED, PFA_ERR_HIP, PFA_ERR_SCRATCH = 0, -1, -2, -3, -4
EXPORTED = ("attn_fwd", "attn_bwd", "attn_bwd_prep", "attn_bwd_dkdv", "attn_bwd_dq", "attn_bwd_dq_delta",
            "attn_bwd_delta", "attn_bwd_ex", "attn_delta_error", "attn_fwd_heads", "attn_fwd_diag",
            "attn_bwd_workspace_bytes", "attn_strerror", "attn_version", "attn_bwd_noalloc",
            "attn_bwd_noalloc_max_bytes")


class TieOpts(ctypes.Structure):
    _fields_ = [("beta", ctypes.c_float), ("eps", ctypes.c_float)]


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m precision_flash_attention_attn_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, ctypes.POINTER(TieOpts), vp]
        L.attn_fwd.restype = i
        L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                               i, i, i, i, i, f, i, vp]
        L.attn_bwd.restype = i
        L.attn_bwd_prep.argtypes = [vp, vp, vp, vp, ctypes.c_size_t, i, i, i, i, i, vp]
        L.attn_bwd_prep.restype = i
        L.attn_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                    i, i, i, i, i, f, i, vp]
        L.attn_bwd_dkdv.restype = i
        L.attn_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                  i, i, i, i, i, f, i, vp]
        L.attn_bwd_dq.restype = i
        L.attn_bwd_dq_delta.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                        i, i, i, i, i, f, i, vp]
        L.attn_bwd_dq_delta.restype = i
        L.attn_bwd_delta.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                     i, i, i, i, i, f, i, i, vp]
        L.attn_bwd_delta.restype = i
        L.attn_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                  i, i, i, i, i, f, i, i, vp]
        L.attn_bwd_ex.restype = i
        L.attn_delta_error.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
        L.attn_delta_error.restype = i
        L.attn_fwd_diag.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i,
                                    ctypes.POINTER(TieOpts), vp]
        L.attn_fwd_diag.restype = i
        L.attn_fwd_heads.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp,
                                     ctypes.POINTER(TieOpts), vp]
        L.attn_fwd_heads.restype = i
        L.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
        L.attn_bwd_noalloc.restype = i
        L.attn_bwd_noalloc_max_bytes.argtypes = []
        L.attn_bwd_noalloc_max_bytes.restype = ctypes.c_size_t
        L.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
        L.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.attn_strerror.argtypes = [i]
        L.attn_strerror.restype = ctypes.c_char_p
        L.attn_version.argtypes = []
        L.attn_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def attn_strerror(status: int) -> str:
    return lib().attn_strerror(int(status)).decode()


def _check(status: int):
    if status != PFA_OK:
        raise AttnError(status, attn_strerror(status))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _expect(t, name, dtype, shape):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on the GPU, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def _mode_id(mode) -> int:
    if isinstance(mode, str):
        if mode not in MODES:
            raise ValueError(f"unknown mode {mode!r}")
        return MODES[mode]
    return int(mode)


def attn_fwd(q, k, v, o, lse, tie_flags=None, causal=True, scale=None, mode="bf16_out",
             beta=2.0, eps=1e-3, stream=None):
    """Forward pass into caller-allocated outputs (see attn_fwd in pfa_attn.h)."""
    B, H, N, d = q.shape
    mid = _mode_id(mode)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _expect(t, name, torch.bfloat16, (B, H, N, d))
    _expect(o, "o", torch.float32 if mid == 1 else torch.bfloat16, (B, H, N, d))
    _expect(lse, "lse", torch.float32, (B, H, N))
    if tie_flags is not None:
        _expect(tie_flags, "tie_flags", torch.int32, (B, H, N))
    scale = 1.0 / d ** 0.5 if scale is None else float(scale)
    opts = TieOpts(float(beta), float(eps))
    _check(lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(tie_flags),
                          B, H, N, d, int(bool(causal)), scale, mid, ctypes.byref(opts),
                          _stream(stream)))


def attn_fwd_diag(q, k, v, o, lse, tie_flags, pbar_one, o_one=None, causal=True, scale=None,
                  mode="bf16_out", beta=2.0, eps=1e-3, stream=None):
    """attn_fwd plus the per-row count of P-bar entries that round to 1
    (pbar_one, int32) and, if given, the part of O they carry (o_one, FP32)."""
    B, H, N, d = q.shape
    mid = _mode_id(mode)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _expect(t, name, torch.bfloat16, (B, H, N, d))
    _expect(o, "o", torch.float32 if mid == 1 else torch.bfloat16, (B, H, N, d))
    _expect(lse, "lse", torch.float32, (B, H, N))
    if tie_flags is not None:
        _expect(tie_flags, "tie_flags", torch.int32, (B, H, N))
    _expect(pbar_one, "pbar_one", torch.int32, (B, H, N))
    if o_one is not None:
        _expect(o_one, "o_one", torch.float32, (B, H, N, d))
    scale = 1.0 / d ** 0.5 if scale is None else float(scale)
    opts = TieOpts(float(beta), float(eps))
    _check(lib().attn_fwd_diag(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(tie_flags),
                               _ptr(pbar_one), _ptr(o_one), B, H, N, d, int(bool(causal)), scale, mid,
                               ctypes.byref(opts), _stream(stream)))


def attn_fwd_heads(q, k, v, o, lse, head_modes, tie_flags=None, causal=True, scale=None,
                   beta=2.0, eps=1e-3, stream=None):
    """Forward with one mode per head (see attn_fwd_heads in pfa_attn.h); o is FP32."""
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _expect(t, name, torch.bfloat16, (B, H, N, d))
    _expect(o, "o", torch.float32, (B, H, N, d))
    _expect(lse, "lse", torch.float32, (B, H, N))
    if tie_flags is not None:
        _expect(tie_flags, "tie_flags", torch.int32, (B, H, N))
    modes = [_mode_id(m) for m in head_modes]
    if len(modes) != H:
        raise ValueError(f"head_modes: expected {H} entries, got {len(modes)}")
    arr = (ctypes.c_int32 * H)(*modes)
    scale = 1.0 / d ** 0.5 if scale is None else float(scale)
    opts = TieOpts(float(beta), float(eps))
    _check(lib().attn_fwd_heads(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(tie_flags),
                                B, H, N, d, int(bool(causal)), scale,
                                ctypes.cast(arr, ctypes.c_void_p), ctypes.byref(opts),
                                _stream(stream)))


def attn_bwd_workspace_bytes(B, H, N, d, mode="bf16_out") -> int:
    return int(lib().attn_bwd_workspace_bytes(B, H, N, d, _mode_id(mode)))


def _delta_src_id(src) -> int:
    if isinstance(src, str):
        if src not in DELTA_SRC:
            raise ValueError(f"unknown delta source {src!r}")
        return DELTA_SRC[src]
    return int(src)


def attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, delta=None, causal=True, scale=None,
             mode="bf16_out", stream=None, delta_src="do_o"):
    """Backward pass into caller-allocated gradients (see attn_bwd and, for a
    delta_src other than "do_o", attn_bwd_ex in pfa_attn.h)."""
    B, H, N, d = q.shape
    mid = _mode_id(mode)
    io = torch.float32 if mid == 1 else torch.bfloat16
    for name, t in (("q", q), ("k", k), ("v", v), ("dq", dq), ("dk", dk), ("dv", dv)):
        _expect(t, name, torch.bfloat16, (B, H, N, d))
    _expect(o, "o", io, (B, H, N, d))
    _expect(dout, "dout", io, (B, H, N, d))
    _expect(lse, "lse", torch.float32, (B, H, N))
    if delta is not None:
        _expect(delta, "delta", torch.float32, (B, H, N))
    if workspace is None or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace: a contiguous GPU buffer is required")
    scale = 1.0 / d ** 0.5 if scale is None else float(scale)
    nbytes = workspace.numel() * workspace.element_size()
    src = _delta_src_id(delta_src)
    if src == 0:
        _check(lib().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                              _ptr(dk), _ptr(dv), _ptr(delta), _ptr(workspace), nbytes, B, H, N, d,
                              int(bool(causal)), scale, mid, _stream(stream)))
    else:
        _check(lib().attn_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                 _ptr(dk), _ptr(dv), _ptr(delta), _ptr(workspace), nbytes, B, H, N,
                                 d, int(bool(causal)), scale, mid, src, _stream(stream)))


def attn_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, delta=None, causal=True, scale=None,
                     mode="bf16_out", stream=None):
    """attn_bwd with the workspace in the library's static device scratch
    (see attn_bwd_noalloc in pfa_attn.h): nothing is allocated."""
    B, H, N, d = q.shape
    mid = _mode_id(mode)
    io = torch.float32 if mid == 1 else torch.bfloat16
    for name, t in (("q", q), ("k", k), ("v", v), ("dq", dq), ("dk", dk), ("dv", dv)):
        _expect(t, name, torch.bfloat16, (B, H, N, d))
    _expect(o, "o", io, (B, H, N, d))
    _expect(dout, "dout", io, (B, H, N, d))
    _expect(lse, "lse", torch.float32, (B, H, N))
    if delta is not None:
        _expect(delta, "delta", torch.float32, (B, H, N))
    scale = 1.0 / d ** 0.5 if scale is None else float(scale)
    _check(lib().attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                  _ptr(dk), _ptr(dv), _ptr(delta), B, H, N, d, int(bool(causal)), scale,
                                  mid, _stream(stream)))


def attn_bwd_noalloc_max_bytes() -> int:
    return int(lib().attn_bwd_noalloc_max_bytes())


def _ws(workspace):
    if workspace is None or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace: a contiguous GPU buffer is required")
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def attn_bwd_prep(o, dout, workspace, delta=None, mode="bf16_out", stream=None):
    """Backward stage 1: delta = rowsum(dO o O)."""
    B, H, N, d = o.shape
    mid = _mode_id(mode)
    io = torch.float32 if mid == 1 else torch.bfloat16
    _expect(o, "o", io, (B, H, N, d))
    _expect(dout, "dout", io, (B, H, N, d))
    if delta is not None:
        _expect(delta, "delta", torch.float32, (B, H, N))
    wp, wn = _ws(workspace)
    _check(lib().attn_bwd_prep(_ptr(o), _ptr(dout), _ptr(delta), wp, wn, B, H, N, d, mid,
                               _stream(stream)))


def attn_bwd_delta(q, k, v, o, dout, lse, workspace, delta=None, causal=True, scale=None,
                   mode="bf16_out", delta_src="do_o", stream=None):
    """Backward stage 1 with a choice of delta source ("do_o", "dp_p", "do_ohp")."""
    B, H, N, d = o.shape
    mid = _mode_id(mode)
    io = torch.float32 if mid == 1 else torch.bfloat16
    _expect(o, "o", io, (B, H, N, d))
    _expect(dout, "dout", io, (B, H, N, d))
    for name, t in (("q", q), ("k", k), ("v", v)):
        _expect(t, name, torch.bfloat16, (B, H, N, d))
    _expect(lse, "lse", torch.float32, (B, H, N))
    if delta is not None:
        _expect(delta, "delta", torch.float32, (B, H, N))
    scale = 1.0 / d ** 0.5 if scale is None else float(scale)
    wp, wn = _ws(workspace)
    _check(lib().attn_bwd_delta(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                _ptr(delta), wp, wn, B, H, N, d, int(bool(causal)), scale, mid,
                                _delta_src_id(delta_src), _stream(stream)))


def attn_delta_error(q, k, v, o, dout, lse, err, causal=True, scale=None, mode="bf16_out",
                     stream=None):
    """err = rowsum(dO o O) - rowsum(dO o O_hp) per row (delta_lp - delta_hp)."""
    B, H, N, d = o.shape
    mid = _mode_id(mode)
    io = torch.float32 if mid == 1 else torch.bfloat16
    _expect(o, "o", io, (B, H, N, d))
    _expect(dout, "dout", io, (B, H, N, d))
    for name, t in (("q", q), ("k", k), ("v", v)):
        _expect(t, name, torch.bfloat16, (B, H, N, d))
    _expect(lse, "lse", torch.float32, (B, H, N))
    _expect(err, "err", torch.float32, (B, H, N))
    scale = 1.0 / d ** 0.5 if scale is None else float(scale)
    _check(lib().attn_delta_error(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                  _ptr(err), B, H, N, d, int(bool(causal)), scale, mid,
                                  _stream(stream)))


def _stage_args(q, k, v, dout, lse, delta, mode):
    B, H, N, d = q.shape
    mid = _mode_id(mode)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _expect(t, name, torch.bfloat16, (B, H, N, d))
    _expect(dout, "dout", torch.float32 if mid == 1 else torch.bfloat16, (B, H, N, d))
    _expect(lse, "lse", torch.float32, (B, H, N))
    if delta is not None:
        _expect(delta, "delta", torch.float32, (B, H, N))
    return B, H, N, d, mid


def attn_bwd_dkdv(q, k, v, dout, lse, dk, dv, workspace, delta=None, causal=True, scale=None,
                  mode="bf16_out", stream=None):
    """Backward stage 2: dK and dV."""
    B, H, N, d, mid = _stage_args(q, k, v, dout, lse, delta, mode)
    _expect(dk, "dk", torch.bfloat16, (B, H, N, d))
    _expect(dv, "dv", torch.bfloat16, (B, H, N, d))
    scale = 1.0 / d ** 0.5 if scale is None else float(scale)
    wp, wn = _ws(workspace)
    _check(lib().attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(delta),
                               _ptr(dk), _ptr(dv), wp, wn, B, H, N, d, int(bool(causal)), scale, mid,
                               _stream(stream)))


def attn_bwd_dq(q, k, v, dout, lse, dq, workspace, delta=None, causal=True, scale=None,
                mode="bf16_out", stream=None):
    """Backward stage 3: dQ."""
    B, H, N, d, mid = _stage_args(q, k, v, dout, lse, delta, mode)
    _expect(dq, "dq", torch.bfloat16, (B, H, N, d))
    scale = 1.0 / d ** 0.5 if scale is None else float(scale)
    wp, wn = _ws(workspace)
    _check(lib().attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(delta),
                             _ptr(dq), wp, wn, B, H, N, d, int(bool(causal)), scale, mid,
                             _stream(stream)))


def attn_bwd_dq_delta(q, k, v, o, dout, lse, dq, workspace, delta=None, causal=True, scale=None,
                      mode="bf16_out", stream=None):
    """Backward stages 1 and 3 in one kernel: dQ, delta and (FP32 output) the
    BF16 dO copy; attn_bwd_dkdv afterwards completes the backward."""
    B, H, N, d, mid = _stage_args(q, k, v, dout, lse, delta, mode)
    _expect(o, "o", torch.float32 if mid == 1 else torch.bfloat16, (B, H, N, d))
    _expect(dq, "dq", torch.bfloat16, (B, H, N, d))
    scale = 1.0 / d ** 0.5 if scale is None else float(scale)
    wp, wn = _ws(workspace)
    _check(lib().attn_bwd_dq_delta(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                   _ptr(delta), wp, wn, B, H, N, d, int(bool(causal)), scale, mid,
                                   _stream(stream)))


# ---- conveniences that allocate with torch and call the entry points above ----

def forward(q, k, v, causal=True, scale=None, mode="bf16_out", beta=2.0, eps=1e-3, flags=True):
    """Allocate outputs and run attn_fwd.  Returns (o, lse, tie_flags or None)."""
    B, H, N, d = q.shape
    mid = _mode_id(mode)
    o = torch.empty((B, H, N, d), device=q.device, dtype=torch.float32 if mid == 1 else torch.bfloat16)
    lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
    fl = torch.empty((B, H, N), device=q.device, dtype=torch.int32) if flags else None
    attn_fwd(q, k, v, o, lse, fl, causal=causal, scale=scale, mode=mode, beta=beta, eps=eps)
    return o, lse, fl


def forward_heads(q, k, v, head_modes, causal=True, scale=None, beta=2.0, eps=1e-3, flags=True):
    """Allocate outputs and run attn_fwd_heads.  Returns (o FP32, lse, tie_flags or None)."""
    B, H, N, d = q.shape
    o = torch.empty((B, H, N, d), device=q.device, dtype=torch.float32)
    lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
    fl = torch.empty((B, H, N), device=q.device, dtype=torch.int32) if flags else None
    attn_fwd_heads(q, k, v, o, lse, head_modes, fl, causal=causal, scale=scale, beta=beta, eps=eps)
    return o, lse, fl


def backward(q, k, v, o, dout, lse, causal=True, scale=None, mode="bf16_out", want_delta=False,
             delta_src="do_o"):
    """Allocate gradients and workspace and run attn_bwd (attn_bwd_ex for another
    delta source).  Returns (dq, dk, dv, delta or None)."""
    B, H, N, d = q.shape
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws = torch.empty(attn_bwd_workspace_bytes(B, H, N, d, mode), device=q.device, dtype=torch.uint8)
    delta = torch.empty((B, H, N), device=q.device, dtype=torch.float32) if want_delta else None
    attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, delta=delta, causal=causal, scale=scale, mode=mode,
             delta_src=delta_src)
    return dq, dk, dv, delta
