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
