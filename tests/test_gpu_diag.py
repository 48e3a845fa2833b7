"""GPU parity of the diagnostic forward (attn_fwd_diag): its O, LSE and tie
flags are the plain forward's bit for bit; its per-row count of P-bar entries
that round to 1 in BF16 (the P-bar = 1 additions the pages' cumulative-error
trace singles out, paper-graph-ui summary of arXiv 2510.04212, section 3.4.4)
equals the BF16 flash emulator's count on every row; and the part of O those
entries carry (o_one) agrees with the emulator's to FP32 accuracy.

The count is an integer decided by floating point: both sides decide it on
d = fp32(fp32(q.k) * scale) - m against the threshold of a correctly rounded
FP32 exp (P-bar = bf16(fp32(exp(d))) is 1), so the counts must be equal.
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
    # 32 (batch, head) slices at d = 128
    ("bh32_n160_d128", Workload(95, "bh32", 2, 16, 160, 128, tie_frac=0.05, tie_q_scale=4.0), True),
    # several key tiles with sharp rows whose maximum moves (the rescale of o_one)
    ("n1000_d128_q4", Workload(96, "sharp", 1, 2, 1000, 128, q_scale=4.0, tie_frac=0.02, tie_q_scale=2.0), True),
]


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_util
    return gpu_util


def _diag(gpu, wl, causal, mode):
    import precision_flash_attention_attn_amd as pfa
    inp = generate(wl)
    q, k, v = gpu.dev_bf16(inp.q), gpu.dev_bf16(inp.k), gpu.dev_bf16(inp.v)
    o, lse, fl = pfa.forward(q, k, v, causal=causal, mode=mode)
    o2, lse2, fl2 = torch.empty_like(o), torch.empty_like(lse), torch.empty_like(fl)
    cnt = torch.empty_like(fl)
    one = torch.full(q.shape, 7.0, device=q.device, dtype=torch.float32)
    pfa.attn_fwd_diag(q, k, v, o2, lse2, fl2, cnt, one, causal=causal, mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2) and torch.equal(fl, fl2)
    return inp, gpu.host(lse2), cnt.cpu().numpy(), gpu.host(one)


@pytest.mark.parametrize("mode", ["bf16_out", "fp32_out", "tie_aware_softmax"])
@pytest.mark.parametrize("name,wl,causal", CASES, ids=[c[0] for c in CASES])
def test_pbar_one_count_and_part_of_o(gpu, name, wl, causal, mode):
    print(f"[diag] {name} mode={mode}", flush=True)
    inp, lse, cnt, one = _diag(gpu, wl, causal, mode)
    B, H, N, d = wl.b, wl.h, wl.n, wl.d
    emu = fe.flash_forward(*(x.reshape(B * H, N, d) for x in (inp.q, inp.k, inp.v)), mode=mode,
                           causal=causal, scale=wl.scale)
    got = cnt.reshape(B * H, N)
    print(f"  P-bar = 1 entries: gpu {int(got.sum())} oracle {int(emu.n_pbar_one.sum())}; rows that "
          f"differ {int(np.sum(got != emu.n_pbar_one))}", flush=True)
    assert np.array_equal(got, emu.n_pbar_one)
    if mode != "tie_aware_softmax":
        assert np.all(got >= 1)          # every row has its maximum at least
    # o_one * l with l from the kernel's own LSE (l = exp(LSE - m), m the
    # emulator's final shift, the same FP32 value as the kernel's) against the
    # emulator's FP32 sum: the same V rows, summed in another order.  The
    # bound is FP32 level: LSE (|LSE| < 128 here) is rounded to 2^-17, which
    # carries into l as 7.6e-6 relative, plus the two sums' roundings.
    ell = np.exp(lse.reshape(B * H, N) - emu.m_final)
    got_bar = one.reshape(B * H, N, d) * ell[..., None]
    want = emu.obar_one
    scale_ = np.max(np.abs(want), axis=-1, keepdims=True) + 1e-30
    rel = np.max(np.abs(got_bar - want) / scale_)
    print(f"  o_one: max error {rel:.2e} of the row's largest entry", flush=True)
    assert rel <= 4e-5
    # rows without P-bar = 1 entries carry no such part
    assert np.all(one.reshape(B * H, N, d)[emu.n_pbar_one == 0] == 0.0)


def test_pbar_one_count_natural_ties(gpu):
    """GPT-2-medium shape with natural ties only (B8 H16 N1024 d64, Q x4):
    the counts of batch 0 against the emulator, head by head, on every row."""
    wl = workload(3)
    inp, lse, cnt, one = _diag(gpu, wl, True, "bf16_out")
    got = cnt[0]
    emu = fe.flash_forward(inp.q[0], inp.k[0], inp.v[0], mode="bf16_out", causal=True, scale=wl.scale)
    print(f"  rows that differ {int(np.sum(got != emu.n_pbar_one))}; totals {got.sum()} vs "
          f"{emu.n_pbar_one.sum()}", flush=True)
    assert np.array_equal(got, emu.n_pbar_one)


def test_signed_error_by_number_of_pbar_one(gpu):
    """The pages trace the negative bias of plain BF16 to rows with more than
    one P-bar = 1 (section 3.4.4, Claim 3: the sum of the tied V values
    overflows the significand and the tail's sticky bits round it up in
    magnitude).  With the diagnostic count, on the tied-rows workload pooled
    over 4096 repetitions (V ~ N(0,1), errors oriented by the tail as in the
    signed-error gate): in plain BF16, rows with two or more P-bar = 1 entries
    carry a negative mean error (< -5 SE), while rows with exactly one carry a
    positive one (> +5 SE: a single BF16-exact V plus a tail smaller than half
    an ulp rounds the tail away).  In the tie-aware mode the rows with repeated
    P-bar = 1 are gone but for a few whose shift still rounds to 1, and no
    group is below -5 SE.  o_one gives the part of O those entries carry."""
    import precision_flash_attention_attn_amd as pfa
    from oracle import attention64 as a64
    from oracle import stats as st
    from synth.inputs import generate_reps
    wl = workload(1)
    reps = 4096
    x = generate_reps(wl, reps)
    b = x.q.shape[0]
    q3, k3, v3 = (a.reshape(b, 128, 64) for a in (x.q, x.k, x.v))
    o64 = np.stack([a64.fwd_slice(q3[i], k3[i], v3[i], True, wl.scale)[0] for i in range(b)])
    tau = st.tail_sums(q3, k3, v3, scale=wl.scale)
    q, k, v = gpu.dev_bf16(x.q), gpu.dev_bf16(x.k), gpu.dev_bf16(x.v)
    res = {}
    for mode in ("bf16_out", "tie_aware_softmax"):
        o = torch.empty_like(q)
        lse = torch.empty((b, 1, 128), device=q.device, dtype=torch.float32)
        fl = torch.empty((b, 1, 128), device=q.device, dtype=torch.int32)
        cnt = torch.empty_like(fl)
        one = torch.empty(q.shape, device=q.device, dtype=torch.float32)
        pfa.attn_fwd_diag(q, k, v, o, lse, fl, cnt, one, mode=mode)
        torch.cuda.synchronize()
        go = gpu.host(o).reshape(b, 128, 64)
        n1 = cnt.cpu().numpy().reshape(b, 128)
        share = np.abs(gpu.host(one).reshape(b, 128, 64)).sum(-1) / (np.abs(go).sum(-1) + 1e-30)
        tail, _, kept = st.row_values(go, o64, tau, np.ones((b, 128), bool))
        n1, share = n1.reshape(-1), share.reshape(-1)
        for name, sel in (("repeated", n1 >= 2), ("single", n1 == 1), ("none", n1 == 0)):
            vals = tail[sel & kept]
            if len(vals) < 2:
                continue
            r = {"rows": int(len(vals)), "mean": float(vals.mean()), "se": float(vals.std(ddof=1) / np.sqrt(len(vals))),
                 "share_of_o_from_pbar_one": float(share[sel & kept].mean())}
            res[(mode, name)] = r
            print(f"[pbar=1 split] {mode} {name}: {r}", flush=True)
            gpu.record("signed_error_by_pbar_one_cfg1_x4096", f"{mode}_{name}", r)
    rep_, one_ = res[("bf16_out", "repeated")], res[("bf16_out", "single")]
    assert rep_["mean"] < -5 * rep_["se"]
    assert one_["mean"] > 5 * one_["se"]
    for (mode, name), r in res.items():
        if mode == "tie_aware_softmax":
            assert r["mean"] > -5 * r["se"], (name, r)
    assert res[("tie_aware_softmax", "repeated")]["rows"] < 0.2 * rep_["rows"]
