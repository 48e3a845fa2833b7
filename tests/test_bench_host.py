"""Host-side parts of bench.py (no GPU): the tail sums behind the tail-oriented
signed O error equal the oracle's, and the multi-GPU request is refused."""
import os
import subprocess
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import stats as st  # noqa: E402
from synth.inputs import generate_reps, workload  # noqa: E402


def test_bench_tail_sums_equal_the_oracle():
    x = generate_reps(workload(1), 3)
    to = lambda a: torch.from_numpy(a).to(torch.bfloat16).contiguous()
    q, k, v = to(x.q), to(x.k), to(x.v)
    B, H, N, d = q.shape
    tau = bench.tail_sums(torch, q, k, v).numpy()
    qf, kf, vf = (t.float().numpy().reshape(B * H, N, d) for t in (q, k, v))
    ref = np.asarray(st.tail_sums(qf, kf, vf, causal=True, scale=1 / d ** 0.5)).reshape(tau.shape)
    assert np.allclose(tau, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.sign(tau), np.sign(ref))
    # the tied rows of the workload have a non-trivial remainder
    assert np.count_nonzero(tau) > 0.9 * tau.size


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)


def test_bench_exact_attention_equals_the_oracle():
    """The float64 reference the bench measures signed errors against is the
    oracle's plain attention (here on the CPU)."""
    from oracle import attention64 as a64
    x = generate_reps(workload(1), 2)
    to = lambda a: torch.from_numpy(a).to(torch.bfloat16).contiguous()
    q, k, v = to(x.q), to(x.k), to(x.v)
    ref = bench.exact_attention(torch, q, k, v, chunk=1).numpy()
    for b in range(2):
        o, _ = a64.attention_fwd(x.q[b, 0], x.k[b, 0], x.v[b, 0], causal=True, scale=0.125)
        assert np.allclose(ref[b, 0], o, rtol=1e-12, atol=1e-13)


def test_bench_ratio_interval_equals_the_oracle():
    """The bench's bootstrap interval of the plain / tie-aware ratio and the
    oracle's ratio_ci agree on the same rows, groups and seed."""
    rng = np.random.default_rng(4)
    g = np.repeat(np.arange(300), 3)
    p = -10.0 + rng.standard_normal(g.size)
    t = 0.8 + rng.standard_normal(g.size)
    a = bench.ratio_interval(torch, torch.from_numpy(p), torch.from_numpy(t), torch.from_numpy(g),
                             n_boot=1000, seed=3)
    b = st.ratio_ci(p, t, g, n_boot=1000, seed=3)
    assert a["ratio"] == pytest.approx(b["ratio"], rel=1e-12)
    assert a["lo"] == pytest.approx(b["lo"], rel=0.05) and a["hi"] == pytest.approx(b["hi"], rel=0.05)
