"""Seeded synthetic attention inputs.

The pages measure on GPT-2 training over OpenWebText (paper-graph-ui summary of
arXiv 2510.04212, section 3.4.1); neither the data nor trained weights are used
here.  Instead five synthetic workloads stand in for the attention-layer shapes
the pages study (GPT-2 small: 12 heads of 64 features at context 1024; GPT-2
medium: 16 heads) plus a long-context and an FP32-output stress shape.

Recipe (every workload):
  * numpy Generator(PCG64(seed)), seed = 1000 * workload id + repetition;
  * draw order Q, Z (key noise), V, dO, each N(0, 1) float32 [B, H, N, d];
    then the structure below; then rounding of Q, K, V (and of dO for the BF16
    modes) to BF16 with round-to-nearest-even;
  * forced ties: in a chosen fraction of query rows T (T >= 3, handled in
    increasing T) the key t* with the largest q_T . k_t (t <= T) is copied to
    k - 1 other distinct positions in [0, T], k uniform in {2, 3, 4}, so that
    row has k exactly equal maxima whatever arithmetic computes the scores.
    A later copy can undo an earlier row's tie; the kernels' and the oracle's
    own tie flags are the truth, the generator only reports what it forced.

The structure per workload is described in WORKLOADS.  This module does no
attention arithmetic; the argmax that picks t* is input construction.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    b: int
    h: int
    n: int
    d: int
    causal: bool = True
    tie_frac: float = 0.0        # fraction of rows with forced tied maxima
    tie_q_scale: float = 1.0     # Q multiplier applied to the forced rows only
    q_scale: float = 1.0         # Q multiplier applied everywhere
    low_rank: int = 0            # rank of the shared key component (0 = none)
    k_noise: float = 1.0         # multiplier of the key noise Z
    v_shift: float = 0.0         # added to V (negative-V paper condition)
    modes: tuple = ("bf16_out", "fp32_out", "tie_aware_softmax")
    note: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def flops(self) -> int:
        """Algorithmic forward + backward FLOPs (7 * 2 N^2 d per head, halved
        when causal): 2 products forward, 5 backward incl. the S recompute."""
        f = 14 * self.b * self.h * self.n * self.n * self.d
        return f // 2 if self.causal else f


WORKLOADS = {
    1: Workload(1, "single-head tied rows", 1, 1, 128, 64, tie_frac=0.25, tie_q_scale=8.0,
                note="25% of rows with 2-4 duplicated argmax keys and Q x8 on those rows"),
    2: Workload(2, "GPT-2-small layer", 8, 12, 1024, 64, tie_frac=0.05, low_rank=4, k_noise=0.5,
                modes=("bf16_out", "fp32_out", "tie_aware_softmax"),
                note="K = 0.5 Z + U c_t (U fixed 64x4), 5% forced tied rows"),
    3: Workload(3, "GPT-2-medium layer", 8, 16, 1024, 64, q_scale=4.0, low_rank=4, k_noise=0.5,
                note="as GPT-2-small with Q x4, natural ties only"),
    4: Workload(4, "long context", 1, 16, 8192, 128, tie_frac=0.01,
                modes=("bf16_out", "tie_aware_softmax"),
                note="N(0,1) inputs, 1% forced tied rows"),
    5: Workload(5, "FP32-output stress", 2, 32, 4096, 128, q_scale=8.0,
                modes=("fp32_out", "bf16_out"),
                note="N(0,1) inputs with Q x8 everywhere"),
}


def workload(wid: int, **over) -> Workload:
    return replace(WORKLOADS[wid], **over)


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round float32 to BF16 (round to nearest even) and return as float32."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


@dataclass
class Inputs:
    wl: Workload
    seed: int
    q: np.ndarray          # [B,H,N,d] float32 holding BF16 values
    k: np.ndarray
    v: np.ndarray
    do_bf16: np.ndarray    # dO rounded to BF16 (BF16 modes)
    do_f32: np.ndarray     # dO in FP32 (FP32-output mode)
    forced_rows: list = field(default_factory=list)  # (b, h, T, k) per forced row

    def do_for(self, mode: str) -> np.ndarray:
        return self.do_f32 if mode == "fp32_out" else self.do_bf16


def _force_ties(rng, q, k, rows, tie_q_scale):
    """Duplicate each chosen row's argmax key; q, k are one [N, d] head (BF16 values)."""
    done = []
    for t_row in rows:
        if tie_q_scale != 1.0:
            q[t_row] = q[t_row] * np.float32(tie_q_scale)
        sc = k[: t_row + 1].astype(np.float64) @ q[t_row].astype(np.float64)
        t_star = int(np.argmax(sc))
        kk = int(rng.integers(2, 5))
        others = np.delete(np.arange(t_row + 1), t_star)   # [0, T] without t*, in order
        pos = rng.choice(others, size=kk - 1, replace=False)
        k[pos] = k[t_star]
        done.append((t_row, kk))
    return done


def generate(wl: Workload, rep: int = 0, seed: int | None = None) -> Inputs:
    """Inputs of one repetition of a workload (see module docstring)."""
    if seed is None:
        seed = 1000 * wl.wid + rep
    rng = np.random.Generator(np.random.PCG64(seed))
    shp = (wl.b, wl.h, wl.n, wl.d)
    q = rng.standard_normal(shp, dtype=np.float32)
    z = rng.standard_normal(shp, dtype=np.float32)
    v = rng.standard_normal(shp, dtype=np.float32)
    do = rng.standard_normal(shp, dtype=np.float32)
    if wl.low_rank:
        u = rng.standard_normal((wl.d, wl.low_rank), dtype=np.float32)
        c = rng.standard_normal((wl.b, wl.h, wl.n, wl.low_rank), dtype=np.float32)
        k = np.float32(wl.k_noise) * z + c @ u.T
    else:
        k = np.float32(wl.k_noise) * z
    q = q * np.float32(wl.q_scale)
    v = v + np.float32(wl.v_shift)
    q = to_bf16_values(q)
    k = to_bf16_values(k)
    v = to_bf16_values(v)
    forced = []
    if wl.tie_frac > 0:
        n_rows = int(round(wl.tie_frac * wl.n))
        for b in range(wl.b):
            for h in range(wl.h):
                rows = np.sort(rng.choice(np.arange(3, wl.n), size=n_rows, replace=False))
                for t_row, kk in _force_ties(rng, q[b, h], k[b, h], rows, wl.tie_q_scale):
                    forced.append((b, h, t_row, kk))
    return Inputs(wl=wl, seed=seed, q=q, k=k, v=v, do_bf16=to_bf16_values(do),
                  do_f32=do.copy(), forced_rows=forced)


def generate_reps(wl: Workload, reps: int, start: int = 0) -> Inputs:
    """Concatenate repetitions along the batch axis (seed 1000*wid + rep each)."""
    parts = [generate(wl, rep=r) for r in range(start, start + reps)]
    cat = lambda name: np.concatenate([getattr(p, name) for p in parts], axis=0)
    forced = []
    for i, p in enumerate(parts):
        forced += [(b + i * wl.b, h, t, kk) for (b, h, t, kk) in p.forced_rows]
    return Inputs(wl=replace(wl, b=wl.b * reps), seed=parts[0].seed, q=cat("q"), k=cat("k"),
                  v=cat("v"), do_bf16=cat("do_bf16"), do_f32=cat("do_f32"), forced_rows=forced)
