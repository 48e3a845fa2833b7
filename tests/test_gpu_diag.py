"""GPU parity of the diagnostic forward (attn_fwd_diag): its O, LSE and tie
flags are the plain forward's bit for bit, and its per-row count of P-bar
entries that round to 1 in BF16 (the P-bar = 1 additions the pages'
cumulative-error trace singles out, paper-graph-ui summary of arXiv 2510.04212,
section 3.4.4) agrees with the BF16 flash emulator's count (for the FP32-output
mode: the BF16 mode's count, which has the same running maximum).

The count is an integer decided by floating point: P-bar rounds to 1 when
exp(S - m) >= 1 - 2^-9.  The kernel forms the exponent with one fma from the
raw dot product, the emulator rounds S and S - m separately, so an element
whose exponent lies within an ulp of that boundary can fall on either side.
Such elements are rare; the bar is equal counts on at least 98% of rows and
totals within 1%.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import flash_emu as fe  # noqa: E402
from synth.inputs import Workload, generate, workload  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = [
    ("cfg1", workload(1), True),
    ("ragged333_d64", Workload(90, "ragged", 1, 2, 333, 64, tie_frac=0.05, tie_q_scale=4.0), True),
    ("b2_n200_d128", Workload(91, "d128", 2, 1, 200, 128, tie_frac=0.05, tie_q_scale=4.0), True),
    ("noncausal_n257_d128", Workload(94, "nc", 1, 3, 257, 128, tie_frac=0.05, tie_q_scale=8.0), False),
    # 32 (batch, head) slices at d = 128: the forward's 128-query geometry
    ("bh32_n160_d128", Workload(95, "bh32", 2, 16, 160, 128, tie_frac=0.05, tie_q_scale=4.0), True),
]


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_util
    return gpu_util


@pytest.mark.parametrize("mode", ["bf16_out", "fp32_out", "tie_aware_softmax"])
@pytest.mark.parametrize("name,wl,causal", CASES, ids=[c[0] for c in CASES])
def test_pbar_one_count(gpu, name, wl, causal, mode):
    import precision_flash_attention_attn_amd as pfa
    print(f"[diag] {name} mode={mode}", flush=True)
    inp = generate(wl)
    q, k, v = gpu.dev_bf16(inp.q), gpu.dev_bf16(inp.k), gpu.dev_bf16(inp.v)
    o, lse, fl = pfa.forward(q, k, v, causal=causal, mode=mode)
    o2, lse2, fl2 = torch.empty_like(o), torch.empty_like(lse), torch.empty_like(fl)
    cnt = torch.empty_like(fl)
    pfa.attn_fwd_diag(q, k, v, o2, lse2, fl2, cnt, causal=causal, mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2) and torch.equal(fl, fl2)
    B, H, N, d = wl.b, wl.h, wl.n, wl.d
    # the count is of P-bar rounded to BF16; in the FP32-output mode the running
    # maximum, and so exp(S - m), is that of the plain BF16 mode
    emu_mode = "bf16_out" if mode == "fp32_out" else mode
    emu = fe.flash_forward(*(x.reshape(B * H, N, d) for x in (inp.q, inp.k, inp.v)), mode=emu_mode,
                           causal=causal, scale=wl.scale)
    got = cnt.cpu().numpy().reshape(B * H, N)
    want = emu.n_pbar_one
    agree = np.mean(got == want)
    print(f"  rows with equal counts: {agree:.4f}; totals {got.sum()} vs {want.sum()}")
    assert agree >= 0.98
    assert abs(int(got.sum()) - int(want.sum())) <= 0.01 * want.sum() + 2


def test_pbar_one_count_natural_ties(gpu):
    """GPT-2-medium shape with natural ties only (B8 H16 N1024 d64, Q x4):
    the counts of batch 0 against the emulator, head by head."""
    import precision_flash_attention_attn_amd as pfa
    wl = workload(3)
    inp = generate(wl)
    q, k, v = gpu.dev_bf16(inp.q), gpu.dev_bf16(inp.k), gpu.dev_bf16(inp.v)
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
    fl = torch.empty((B, H, N), device=q.device, dtype=torch.int32)
    cnt = torch.empty_like(fl)
    pfa.attn_fwd_diag(q, k, v, o, lse, fl, cnt)
    torch.cuda.synchronize()
    got = cnt[0].cpu().numpy()
    emu = fe.flash_forward(inp.q[0], inp.k[0], inp.v[0], mode="bf16_out", causal=True, scale=wl.scale)
    agree = np.mean(got == emu.n_pbar_one)
    print(f"  rows with equal counts: {agree:.4f}; totals {got.sum()} vs {emu.n_pbar_one.sum()}")
    assert agree >= 0.98
    assert abs(int(got.sum()) - int(emu.n_pbar_one.sum())) <= 0.01 * emu.n_pbar_one.sum() + 2
