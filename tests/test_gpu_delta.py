"""GPU parity of the alternative delta sources and the delta-error export
against the CPU oracle (paper-graph-ui summary of arXiv 2510.04212, section
3.2: the isolation experiments; section 3.4.4: the error of delta).

Tolerances, from the arithmetic: the kernels form P in FP32 (one exp2 and one
fma per score), products of BF16 operands exactly, and their sums in FP32, so
each delta errs by a small multiple of 2^-24 times the sum of the magnitudes it
adds up -- cond_p = rowsum(P |dP|) for rowsum(dP o P) and cond_o =
sum |dO| (P |V|) for rowsum(dO o O_hp), both computed by the oracle.  The bound
used is 1e-4 times that magnitude (P split into BF16 hi + lo carries a relative
error up to 2^-17 into O_hp).  The delta_lp - delta_hp export is compared with
the oracle's rowsum(dO o O_emu) - rowsum(dO o O_exact), where O_emu is the
BF16 flash emulator's output: the kernel's O differs from it by at most two
BF16 ulps in a few elements, so the bound adds 2^-7 sum |dO| |O|.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import attention64 as a64  # noqa: E402
from oracle import flash_emu as fe  # noqa: E402
from oracle import stats as st  # noqa: E402
from synth.inputs import Workload, generate, workload  # noqa: E402

pytestmark = pytest.mark.gpu

GRAD_TOL = 5e-2

CASES = [
    ("cfg1", workload(1), True),
    ("ragged333_d64", Workload(90, "ragged", 1, 2, 333, 64, tie_frac=0.05, tie_q_scale=4.0), True),
    ("b2_n200_d128", Workload(91, "d128", 2, 1, 200, 128, tie_frac=0.05, tie_q_scale=4.0), True),
    ("n1", Workload(92, "n1", 1, 1, 1, 64), True),
    ("noncausal_n257_d128", Workload(94, "nc", 1, 3, 257, 128, tie_frac=0.05, tie_q_scale=8.0), False),
]


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_util
    return gpu_util


def _deltas(gpu, inp, wl, mode, causal):
    """Forward, then delta from each source and the error export, on the GPU."""
    import precision_flash_attention_attn_amd as pfa
    q, k, v = gpu.dev_bf16(inp.q), gpu.dev_bf16(inp.k), gpu.dev_bf16(inp.v)
    o, lse, _ = pfa.forward(q, k, v, causal=causal, mode=mode)
    do = gpu.dev_f32(inp.do_f32) if mode == "fp32_out" else gpu.dev_bf16(inp.do_bf16)
    B, H, N, d = q.shape
    ws = torch.empty(pfa.attn_bwd_workspace_bytes(B, H, N, d, mode), device=q.device, dtype=torch.uint8)
    out = {}
    for src in ("do_o", "dp_p", "do_ohp"):
        delta = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
        pfa.attn_bwd_delta(q, k, v, o, do, lse, ws, delta=delta, causal=causal, mode=mode, delta_src=src)
        out[src] = gpu.host(delta)
    err = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
    pfa.attn_delta_error(q, k, v, o, do, lse, err, causal=causal, mode=mode)
    out["err"] = gpu.host(err)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("mode", ["bf16_out", "fp32_out"])
@pytest.mark.parametrize("name,wl,causal", CASES, ids=[c[0] for c in CASES])
def test_delta_sources_against_oracle(gpu, name, wl, causal, mode):
    print(f"[delta] {name} mode={mode} shape={wl.b, wl.h, wl.n, wl.d} causal={causal}", flush=True)
    inp = generate(wl)
    g = _deltas(gpu, inp, wl, mode, causal)
    B, H, N, d = wl.b, wl.h, wl.n, wl.d
    q, k, v = (x.reshape(B * H, N, d) for x in (inp.q, inp.k, inp.v))
    do_given = inp.do_for(mode).reshape(B * H, N, d)
    do_mfma = inp.do_bf16.reshape(B * H, N, d)    # dP is formed from BF16 dO in every mode
    emu = fe.flash_forward(q, k, v, mode=mode, causal=causal, scale=wl.scale)
    for i in range(B * H):
        ref = a64.bwd_slice(q[i], k[i], v[i], do_given[i], causal, wl.scale)
        ref_b = a64.bwd_slice(q[i], k[i], v[i], do_mfma[i], causal, wl.scale)
        dp = g["dp_p"].reshape(B * H, N)[i]
        assert np.all(np.abs(dp - ref_b["delta_p"]) <= 1e-4 * ref_b["cond_p"] + 1e-30), "dp_p"
        ohp = g["do_ohp"].reshape(B * H, N)[i]
        assert np.all(np.abs(ohp - ref["delta"]) <= 1e-4 * ref["cond_o"] + 1e-30), "do_ohp"
        # the export against the oracle's delta_lp - delta_hp with the emulator's O
        o_emu = emu.o[i]
        want = np.sum(do_given[i] * o_emu, axis=-1) - ref["delta"]
        mag = np.sum(np.abs(do_given[i]) * np.abs(o_emu), axis=-1)
        lp_tol = (1e-5 if mode == "fp32_out" else 2.0 ** -7) * mag
        e = g["err"].reshape(B * H, N)[i]
        assert np.all(np.abs(e - want) <= lp_tol + 1e-4 * ref["cond_o"]), "delta error export"
    # the export is the stored-O delta minus the recomputed one, up to FP32 sums
    mag_all = np.sum(np.abs(inp.do_for(mode)) * np.abs(emu.o.reshape(inp.q.shape)), axis=-1)
    assert np.all(np.abs(g["err"] - (g["do_o"] - g["do_ohp"])) <= 4e-5 * mag_all + 1e-30)


def test_recomputed_delta_removes_the_low_precision_error(gpu):
    """On rows with tied maxima (config 1), delta from the BF16 O errs by the
    rounding of O; either alternative source is orders of magnitude closer to
    the exact delta (the pages' reason for the experiments)."""
    wl = workload(1)
    inp = generate(wl)
    g = _deltas(gpu, inp, wl, "bf16_out", True)
    q, k, v, do = (x.reshape(-1, wl.n, wl.d) for x in (inp.q, inp.k, inp.v, inp.do_bf16))
    ref = a64.bwd_slice(q[0], k[0], v[0], do[0], True, wl.scale)
    e_lp = np.mean(np.abs(g["do_o"].reshape(-1) - ref["delta"]))
    e_p = np.mean(np.abs(g["dp_p"].reshape(-1) - ref["delta_p"]))
    e_hp = np.mean(np.abs(g["do_ohp"].reshape(-1) - ref["delta"]))
    print(f"  mean |delta - exact|: stored O {e_lp:.3e}, dP.P {e_p:.3e}, O_hp {e_hp:.3e}")
    assert e_p < e_lp / 100 and e_hp < e_lp / 100


@pytest.mark.parametrize("src", ["dp_p", "do_ohp"])
@pytest.mark.parametrize("mode", ["bf16_out", "fp32_out", "tie_aware_softmax"])
def test_backward_with_delta_source(gpu, src, mode):
    import precision_flash_attention_attn_amd as pfa
    for name, wl, causal in (CASES[1], CASES[2], CASES[4]):
        print(f"[bwd-delta] {name} mode={mode} src={src}", flush=True)
        inp = generate(wl)
        q, k, v = gpu.dev_bf16(inp.q), gpu.dev_bf16(inp.k), gpu.dev_bf16(inp.v)
        o, lse, _ = pfa.forward(q, k, v, causal=causal, mode=mode)
        do = gpu.dev_f32(inp.do_f32) if mode == "fp32_out" else gpu.dev_bf16(inp.do_bf16)
        dq, dk, dv, delta = pfa.backward(q, k, v, o, do, lse, causal=causal, mode=mode,
                                         want_delta=True, delta_src=src)
        torch.cuda.synchronize()
        B, H, N, d = q.shape
        r = (lambda t: gpu.host(t).reshape(B * H, N, d))
        gq, gk, gv = r(dq), r(dk), r(dv)
        qs, ks, vs = (x.reshape(B * H, N, d) for x in (inp.q, inp.k, inp.v))
        dos = inp.do_for(mode).reshape(B * H, N, d)
        for i in range(B * H):
            ref = a64.bwd_slice(qs[i], ks[i], vs[i], dos[i], causal, wl.scale)
            for key, got in (("dq", gq[i]), ("dk", gk[i]), ("dv", gv[i])):
                err = st.max_rel_err(got, ref[key])
                assert err <= GRAD_TOL, (name, key, err)
        # the delta the gradients used is the one the stage writes on its own
        ws = torch.empty(pfa.attn_bwd_workspace_bytes(B, H, N, d, mode), device=q.device, dtype=torch.uint8)
        d2 = torch.empty_like(delta)
        pfa.attn_bwd_delta(q, k, v, o, do, lse, ws, delta=d2, causal=causal, mode=mode, delta_src=src)
        torch.cuda.synchronize()
        assert torch.equal(delta, d2)


def test_delta_sources_long_context_one_head(gpu):
    """Long-context shape (B1 H16 N8192 d128, causal): every row of head 0 of
    both alternative sources against the oracle."""
    wl = workload(4)
    inp = generate(wl)
    print("[delta] long context, head 0 of 16", flush=True)
    g = _deltas(gpu, inp, wl, "bf16_out", True)
    ref = a64.slice_reference(inp.q[0, 0], inp.k[0, 0], inp.v[0, 0], inp.do_bf16[0, 0],
                              causal=True, scale=wl.scale)
    assert np.all(np.abs(g["dp_p"][0, 0] - ref["delta_p"]) <= 1e-4 * ref["cond_p"])
    assert np.all(np.abs(g["do_ohp"][0, 0] - ref["delta"]) <= 1e-4 * ref["cond_o"])


def test_delta_sources_gpt2_small_shape(gpu):
    """GPT-2-small layer shape (B8 H12 N1024 d64, low-rank keys, forced ties):
    both alternative sources against the oracle on heads 0 and 11 of batch 0
    and 7."""
    wl = workload(2)
    inp = generate(wl)
    print("[delta] GPT-2-small shape", flush=True)
    g = _deltas(gpu, inp, wl, "bf16_out", True)
    for b, h in ((0, 0), (0, 11), (7, 0), (7, 11)):
        ref = a64.bwd_slice(inp.q[b, h], inp.k[b, h], inp.v[b, h], inp.do_bf16[b, h], True, wl.scale)
        assert np.all(np.abs(g["dp_p"][b, h] - ref["delta_p"]) <= 1e-4 * ref["cond_p"] + 1e-30)
        assert np.all(np.abs(g["do_ohp"][b, h] - ref["delta"]) <= 1e-4 * ref["cond_o"] + 1e-30)


@pytest.mark.parametrize("mode", ["bf16_out", "fp32_out"])
def test_delta_stage_then_gradient_stages_equal_one_call(gpu, mode):
    """attn_bwd_delta followed by attn_bwd_dkdv and attn_bwd_dq on one stream
    gives bit for bit what attn_bwd_ex gives (in the FP32-output mode the
    delta stage also leaves the BF16 dO copy the gradient stages read)."""
    import precision_flash_attention_attn_amd as pfa
    name, wl, causal = CASES[2]
    inp = generate(wl)
    q, k, v = gpu.dev_bf16(inp.q), gpu.dev_bf16(inp.k), gpu.dev_bf16(inp.v)
    o, lse, _ = pfa.forward(q, k, v, causal=causal, mode=mode)
    do = gpu.dev_f32(inp.do_f32) if mode == "fp32_out" else gpu.dev_bf16(inp.do_bf16)
    B, H, N, d = q.shape
    for src in ("dp_p", "do_ohp"):
        dq1, dk1, dv1, _ = pfa.backward(q, k, v, o, do, lse, causal=causal, mode=mode, delta_src=src)
        ws = torch.empty(pfa.attn_bwd_workspace_bytes(B, H, N, d, mode), device=q.device, dtype=torch.uint8)
        dq2, dk2, dv2 = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        pfa.attn_bwd_delta(q, k, v, o, do, lse, ws, causal=causal, mode=mode, delta_src=src)
        pfa.attn_bwd_dkdv(q, k, v, do, lse, dk2, dv2, ws, causal=causal, mode=mode)
        pfa.attn_bwd_dq(q, k, v, do, lse, dq2, ws, causal=causal, mode=mode)
        torch.cuda.synchronize()
        assert torch.equal(dq1, dq2) and torch.equal(dk1, dk2) and torch.equal(dv1, dv2), src
