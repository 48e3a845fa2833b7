"""GPU test of attn_bwd_noalloc, the backward whose workspace is the library's
static device scratch: called through the C ABI, its dQ, dK, dV and delta
equal attn_bwd's bit for bit (the same kernels on the same inputs), on two
calls in a row, the second with a smaller problem (the scratch keeps the
first call's contents), in every mode."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from synth.inputs import Workload, generate  # noqa: E402

pytestmark = pytest.mark.gpu

# (first call, second call): the second is smaller in rows, and at d = 64
CALLS = [
    (Workload(140, "noalloc large", 2, 4, 1000, 128, tie_frac=0.05, tie_q_scale=4.0),
     Workload(141, "noalloc small", 1, 2, 300, 64, tie_frac=0.05, tie_q_scale=8.0)),
]
MODES = ("bf16_out", "fp32_out", "tie_aware_softmax")


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_util
    return gpu_util


def _both(gpu, wl, mode):
    import precision_flash_attention_attn_amd as pfa
    inp = generate(wl)
    q, k, v = (gpu.dev_bf16(x) for x in (inp.q, inp.k, inp.v))
    do = gpu.dev_f32(inp.do_f32) if mode == "fp32_out" else gpu.dev_bf16(inp.do_bf16)
    o, lse, _ = pfa.forward(q, k, v, mode=mode)
    B, H, N, d = q.shape
    assert pfa.attn_bwd_workspace_bytes(B, H, N, d, mode) <= pfa.attn_bwd_noalloc_max_bytes()
    ref = pfa.backward(q, k, v, o, do, lse, mode=mode, want_delta=True)
    got = [torch.full_like(q, 7.0) for _ in range(3)]
    delta = torch.full((B, H, N), 7.0, device=q.device, dtype=torch.float32)
    pfa.attn_bwd_noalloc(q, k, v, o, do, lse, *got, delta=delta, mode=mode)
    torch.cuda.synchronize()
    return ref, (*got, delta)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("first,second", CALLS, ids=["large_then_small"])
def test_noalloc_backward_equals_attn_bwd(gpu, first, second, mode):
    for wl in (first, second):
        print(f"[noalloc] {wl.name} {wl.b, wl.h, wl.n, wl.d} mode={mode}", flush=True)
        ref, got = _both(gpu, wl, mode)
        for name, a, b in zip(("dq", "dk", "dv", "delta"), ref, got):
            assert np.array_equal(gpu.host(a), gpu.host(b)), (wl.name, mode, name)


def test_noalloc_backward_without_delta_output(gpu):
    """delta = NULL: the scratch holds delta, the gradients are unchanged."""
    import precision_flash_attention_attn_amd as pfa
    wl = Workload(142, "noalloc no delta", 1, 3, 257, 128, tie_frac=0.05, tie_q_scale=4.0)
    inp = generate(wl)
    q, k, v, do = (gpu.dev_bf16(x) for x in (inp.q, inp.k, inp.v, inp.do_bf16))
    o, lse, _ = pfa.forward(q, k, v)
    dq, dk, dv, _ = pfa.backward(q, k, v, o, do, lse)
    got = [torch.empty_like(q) for _ in range(3)]
    pfa.attn_bwd_noalloc(q, k, v, o, do, lse, *got)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv), got):
        assert np.array_equal(gpu.host(a), gpu.host(b))
