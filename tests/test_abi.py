"""The C ABI library: loads, exports what include/pfa_attn.h declares, and
rejects invalid arguments before launching anything (runs without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pfa_attn.h")

pfa = pytest.importorskip("precision_flash_attention_attn_amd")
from precision_flash_attention_attn_amd import _binding as bnd  # noqa: E402


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bnd.LIB_PATH):
        from precision_flash_attention_attn_amd.build import build_library
        build_library()
    return bnd.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(attn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    assert set(bnd.EXPORTED) == set(names)


def test_library_exports_every_declared_symbol(L):
    for name in _declared_functions():
        assert hasattr(L, name), name
    assert L.attn_version().decode().startswith("pfa_attn")


def test_strerror(L):
    assert L.attn_strerror(0) == b"ok"
    assert b"invalid" in L.attn_strerror(-1)
    assert b"64 or 128" in L.attn_strerror(-2)
    assert L.attn_strerror(12345) == b"unknown status"


def test_workspace_bytes(L):
    rows = 16 * 8192
    assert L.attn_bwd_workspace_bytes(1, 16, 8192, 128, 0) == rows * 4   # the delta vector
    assert L.attn_bwd_workspace_bytes(1, 16, 8192, 128, 1) == rows * 4 + rows * 128 * 2  # + BF16 dO
    assert L.attn_bwd_workspace_bytes(1, 1, 1, 64, 0) == 256             # 256-byte aligned
    assert L.attn_bwd_workspace_bytes(1, 1, 1, 96, 0) == 0
    assert L.attn_bwd_workspace_bytes(0, 1, 1, 64, 0) == 0
    assert L.attn_bwd_workspace_bytes(1, 1, 1, 64, 7) == 0


FAKE = 0x10000  # a 16-byte-aligned non-null address; never dereferenced (checks fail first)


def _fwd(L, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, flags=None, B=1, H=1, N=128, d=64, causal=1,
         scale=0.125, mode=0, opts=None):
    return L.attn_fwd(q, k, v, o, lse, flags, B, H, N, d, causal, scale, mode,
                      ctypes.byref(opts) if opts is not None else None, None)


def test_fwd_rejects_invalid_arguments(L):
    inv, uns = bnd.PFA_ERR_INVALID, bnd.PFA_ERR_UNSUPPORTED
    assert _fwd(L, q=None) == inv
    assert _fwd(L, lse=None) == inv
    assert _fwd(L, o=FAKE + 8) == inv                      # misaligned
    assert _fwd(L, flags=FAKE + 2) == inv                  # misaligned flags
    assert _fwd(L, B=0) == inv
    assert _fwd(L, N=-5) == inv
    assert _fwd(L, d=96) == uns
    assert _fwd(L, d=256) == uns
    assert _fwd(L, scale=float("nan")) == inv
    assert _fwd(L, scale=0.0) == inv
    assert _fwd(L, scale=-1.0) == inv
    assert _fwd(L, mode=3) == inv
    assert _fwd(L, mode=-1) == inv
    assert _fwd(L, opts=bnd.TieOpts(1.0, 1e-3)) == inv     # beta must exceed 1
    assert _fwd(L, opts=bnd.TieOpts(float("inf"), 1e-3)) == inv
    assert _fwd(L, opts=bnd.TieOpts(2.0, -1e-3)) == inv
    assert _fwd(L, opts=bnd.TieOpts(2.0, float("nan"))) == inv
    assert _fwd(L, B=1 << 16, H=1 << 16, N=1 << 10, d=128) == inv   # too many elements
    # launch size: B*H*ceil(N/64) < 2^23 (with up to 512 threads per workgroup)
    assert _fwd(L, B=1 << 13, H=1 << 4, N=1 << 12, d=64) == inv     # 2^23 blocks of 64 keys
    assert _fwd(L, B=1 << 13, H=1 << 4, N=(1 << 12) - 64, d=64, q=None) == inv   # accepted, then NULL q
    # one (batch, head) slice must keep 32-bit byte offsets: N*d < 2^29
    assert _fwd(L, N=1 << 22, d=128) == uns
    assert _fwd(L, N=(1 << 22) - 1, d=128, q=None) == inv   # size accepted, then the NULL q


def _bwd(L, ws=FAKE, ws_bytes=1 << 30, q=FAKE, dq=FAKE, o=FAKE, B=1, H=1, N=128, d=64, mode=0,
         scale=0.125, delta=None):
    return L.attn_bwd(q, FAKE, FAKE, o, FAKE, FAKE, dq, FAKE, FAKE, delta, ws, ws_bytes,
                      B, H, N, d, 1, scale, mode, None)


def test_bwd_rejects_invalid_arguments(L):
    inv, uns = bnd.PFA_ERR_INVALID, bnd.PFA_ERR_UNSUPPORTED
    need = L.attn_bwd_workspace_bytes(1, 1, 128, 64, 0)
    assert _bwd(L, ws=None) == inv
    assert _bwd(L, ws_bytes=need - 1) == inv
    assert _bwd(L, ws=FAKE + 4) == inv
    assert _bwd(L, q=None) == inv
    assert _bwd(L, dq=FAKE + 2) == inv
    assert _bwd(L, o=None) == inv
    assert _bwd(L, d=80) == uns
    assert _bwd(L, mode=5) == inv
    assert _bwd(L, scale=float("inf")) == inv
    assert _bwd(L, delta=FAKE + 1) == inv
    assert _bwd(L, N=1 << 23, d=64) == uns


def test_python_binding_validates_before_calling(L):
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)       # CPU tensor: rejected
    with pytest.raises(ValueError):
        pfa.forward(q, q, q)
    with pytest.raises(ValueError):
        pfa.attn_fwd(q, q, q, q, None, mode="bf16_out")
    with pytest.raises(ValueError):
        bnd._mode_id("fp16_out")


def test_backward_stages_reject_invalid_arguments(L):
    inv, uns = bnd.PFA_ERR_INVALID, bnd.PFA_ERR_UNSUPPORTED
    need = L.attn_bwd_workspace_bytes(1, 1, 128, 64, 0)
    assert L.attn_bwd_prep(FAKE, FAKE, None, FAKE, need - 16, 1, 1, 128, 64, 0, None) == inv
    assert L.attn_bwd_prep(None, FAKE, None, FAKE, need, 1, 1, 128, 64, 0, None) == inv
    assert L.attn_bwd_prep(FAKE, FAKE, None, FAKE, need, 1, 1, 128, 32, 0, None) == uns
    assert L.attn_bwd_prep(FAKE, FAKE, FAKE + 2, FAKE, need, 1, 1, 128, 64, 0, None) == inv
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, need, 1, 1, 128, 64, 1, 0.125, 0, None]
    for fn in (L.attn_bwd_dkdv,):
        for pos, val in ((4, None), (7, FAKE + 8), (15, float("nan")), (16, 9), (9, need - 1)):
            bad = list(args)
            bad[pos] = val
            assert fn(*bad) == inv, pos
    dq_args = [FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, need, 1, 1, 128, 64, 1, 0.125, 0, None]
    for pos, val in ((0, None), (6, FAKE + 4), (14, 0.0), (15, 3), (8, 0)):
        bad = list(dq_args)
        bad[pos] = val
        assert L.attn_bwd_dq(*bad) == inv, pos
    bad = list(dq_args)
    bad[12] = 48
    assert L.attn_bwd_dq(*bad) == uns
    # attn_bwd_dq_delta: the dQ arguments plus o
    dd_args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, need, 1, 1, 128, 64, 1, 0.125, 0, None]
    for pos, val in ((3, None), (3, FAKE + 2), (5, None), (6, FAKE + 4), (7, FAKE + 1), (9, need - 1),
                     (15, float("inf")), (16, 4)):
        bad = list(dd_args)
        bad[pos] = val
        assert L.attn_bwd_dq_delta(*bad) == inv, pos
    bad = list(dd_args)
    bad[13] = 96
    assert L.attn_bwd_dq_delta(*bad) == uns


def test_delta_entry_points_reject_invalid_arguments(L):
    inv = bnd.PFA_ERR_INVALID
    need = L.attn_bwd_workspace_bytes(1, 1, 128, 64, 0)
    # attn_bwd_delta: unknown source, NULL q for a source that needs it, small workspace
    args = lambda src, q=FAKE, ws_bytes=need, lse=FAKE: (q, FAKE, FAKE, FAKE, FAKE, lse, None, FAKE, ws_bytes,
                                                           1, 1, 128, 64, 1, 0.125, 0, src, None)
    assert L.attn_bwd_delta(*args(3)) == inv
    assert L.attn_bwd_delta(*args(-1)) == inv
    assert L.attn_bwd_delta(*args(1, q=None)) == inv
    assert L.attn_bwd_delta(*args(2, lse=None)) == inv
    assert L.attn_bwd_delta(*args(1, ws_bytes=need - 1)) == inv
    # attn_bwd_ex: unknown source, misaligned output
    ex = lambda src, dq=FAKE: (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dq, FAKE, FAKE, None, FAKE, need,
                               1, 1, 128, 64, 1, 0.125, 0, src, None)
    assert L.attn_bwd_ex(*ex(7)) == inv
    assert L.attn_bwd_ex(*ex(1, dq=FAKE + 2)) == inv
    # attn_delta_error: NULL or misaligned err, bad mode
    er = lambda err=FAKE, mode=0: (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, err, 1, 1, 128, 64, 1, 0.125, mode, None)
    assert L.attn_delta_error(*er(err=None)) == inv
    assert L.attn_delta_error(*er(err=FAKE + 2)) == inv
    assert L.attn_delta_error(*er(mode=9)) == inv


def test_per_head_forward_rejects_invalid_arguments(L):
    inv, uns = bnd.PFA_ERR_INVALID, bnd.PFA_ERR_UNSUPPORTED
    modes = (ctypes.c_int32 * 4)(0, 1, 2, 1)
    bad = (ctypes.c_int32 * 4)(0, 1, 3, 1)
    call = lambda hm, H=4, o=FAKE, d=64: L.attn_fwd_heads(FAKE, FAKE, FAKE, o, FAKE, None, 1, H, 128, d, 1,
                                                          0.125, hm, None, None)
    assert call(None) == inv
    assert call(ctypes.cast(bad, ctypes.c_void_p)) == inv
    assert call(ctypes.cast(modes, ctypes.c_void_p), o=FAKE + 4) == inv
    assert call(ctypes.cast(modes, ctypes.c_void_p), d=80) == uns
    many = (ctypes.c_int32 * 257)(*([0] * 257))
    assert call(ctypes.cast(many, ctypes.c_void_p), H=257) == uns


def test_diag_forward_requires_the_count_buffer(L):
    inv = bnd.PFA_ERR_INVALID
    f = lambda cnt, one=None: L.attn_fwd_diag(FAKE, FAKE, FAKE, FAKE, FAKE, None, cnt, one, 1, 1, 128, 64, 1,
                                              0.125, 0, None, None)
    assert f(None) == inv
    assert f(FAKE + 2) == inv
    assert f(FAKE, one=FAKE + 4) == inv   # o_one must be 16-byte aligned


def test_noalloc_backward_rejects_problems_beyond_its_scratch(L):
    """attn_bwd_noalloc: sizes whose workspace exceeds the static scratch return
    PFA_ERR_SCRATCH, other bad arguments PFA_ERR_INVALID, all before any HIP
    call (every case here fails a check; none launches)."""
    mx = L.attn_bwd_noalloc_max_bytes()
    assert mx == 72 << 20
    args = lambda N, mode=1, d=128, dq=FAKE, lse=FAKE: (FAKE, FAKE, FAKE, FAKE, FAKE, lse, dq, FAKE, FAKE, None,
                                                       1, 1, N, d, 1, 0.088, mode, None)
    # FP32-output mode at d = 128: 4 + 256 bytes of workspace per row
    rows_fit = mx // 260
    assert L.attn_bwd_workspace_bytes(1, 1, rows_fit + 4096, 128, 1) > mx
    assert L.attn_bwd_noalloc(*args(rows_fit + 4096)) == bnd.PFA_ERR_SCRATCH
    assert L.attn_bwd_noalloc(*args(1 << 21)) == bnd.PFA_ERR_SCRATCH
    # BF16 modes need only the delta vector: 2^21 rows fit, so these fail on pointers
    assert L.attn_bwd_noalloc(*args(1 << 21, mode=0, dq=FAKE + 2)) == bnd.PFA_ERR_INVALID
    assert L.attn_bwd_noalloc(*args(128, mode=0, lse=None)) == bnd.PFA_ERR_INVALID
    assert L.attn_bwd_noalloc(*args(0, mode=0)) == bnd.PFA_ERR_INVALID
    assert L.attn_bwd_noalloc(*args(128, mode=5)) == bnd.PFA_ERR_INVALID
    assert L.attn_bwd_noalloc(*args(128, d=96)) == bnd.PFA_ERR_UNSUPPORTED
    assert b"scratch" in L.attn_strerror(bnd.PFA_ERR_SCRATCH)
