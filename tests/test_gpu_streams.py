"""The C ABI on a caller's stream and under HIP graph capture: the library
launches only on the stream it is given and allocates, copies and
synchronises nothing, so a forward + backward step can be captured into a
graph and replayed.  Every result is compared bit for bit with the eager
call on the default stream (no atomics anywhere, so results are
deterministic)."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from synth.inputs import Workload, generate  # noqa: E402

pytestmark = pytest.mark.gpu

MODES = ("bf16_out", "fp32_out", "tie_aware_softmax")


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_util
    return gpu_util


class Step:
    """Static buffers for one forward + backward step and the calls that fill them."""

    def __init__(self, pfa, shape, mode):
        B, H, N, d = shape
        dev = "cuda:0"
        io = torch.float32 if mode == "fp32_out" else torch.bfloat16
        self.mode = mode
        self.q, self.k, self.v = (torch.empty(shape, device=dev, dtype=torch.bfloat16) for _ in range(3))
        self.do = torch.empty(shape, device=dev, dtype=io)
        self.o = torch.empty(shape, device=dev, dtype=io)
        self.lse = torch.empty((B, H, N), device=dev, dtype=torch.float32)
        self.flags = torch.empty((B, H, N), device=dev, dtype=torch.int32)
        self.dq, self.dk, self.dv = (torch.empty(shape, device=dev, dtype=torch.bfloat16) for _ in range(3))
        self.delta = torch.empty((B, H, N), device=dev, dtype=torch.float32)
        self.ws = torch.empty(pfa.attn_bwd_workspace_bytes(B, H, N, d, mode), device=dev, dtype=torch.uint8)
        self.pfa = pfa

    def load(self, gpu, inp):
        self.q.copy_(gpu.dev_bf16(inp.q))
        self.k.copy_(gpu.dev_bf16(inp.k))
        self.v.copy_(gpu.dev_bf16(inp.v))
        self.do.copy_(gpu.dev_f32(inp.do_f32) if self.mode == "fp32_out" else gpu.dev_bf16(inp.do_bf16))

    def run(self, stream=None):
        p = self.pfa
        p.attn_fwd(self.q, self.k, self.v, self.o, self.lse, self.flags, mode=self.mode, stream=stream)
        p.attn_bwd(self.q, self.k, self.v, self.o, self.do, self.lse, self.dq, self.dk, self.dv, self.ws,
                   delta=self.delta, mode=self.mode, stream=stream)

    def outputs(self):
        return {k: getattr(self, k).clone() for k in ("o", "lse", "flags", "dq", "dk", "dv", "delta")}


def _same(a, b):
    return all(torch.equal(a[k], b[k]) for k in a)


@pytest.mark.parametrize("mode", MODES)
def test_caller_stream(gpu, mode):
    import precision_flash_attention_attn_amd as pfa
    wl = Workload(110, "stream", 2, 3, 200, 128, tie_frac=0.05, tie_q_scale=4.0)
    st = Step(pfa, (wl.b, wl.h, wl.n, wl.d), mode)
    st.load(gpu, generate(wl))
    st.run()
    torch.cuda.synchronize()
    ref = st.outputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run(stream=side)
    torch.cuda.synchronize()
    assert _same(st.outputs(), ref)


@pytest.mark.parametrize("mode", MODES)
def test_graph_capture_and_replay(gpu, mode):
    import precision_flash_attention_attn_amd as pfa
    wls = [Workload(111 + i, "graph", 1, 4, 333, 64 if mode == "fp32_out" else 128,
                    tie_frac=0.05, tie_q_scale=8.0) for i in range(2)]
    shape = (wls[0].b, wls[0].h, wls[0].n, wls[0].d)
    inps = [generate(w) for w in wls]
    st = Step(pfa, shape, mode)
    refs = []
    for inp in inps:                      # eager results on the default stream
        st.load(gpu, inp)
        st.run()
        torch.cuda.synchronize()
        refs.append(st.outputs())
    # capture (after a warm-up on a side stream, as capture requires)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run()
    torch.cuda.synchronize()
    for rep in range(4):
        i = rep % 2
        st.load(gpu, inps[i])              # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(st.outputs(), refs[i]), (mode, rep)
