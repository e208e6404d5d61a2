"""Capture of the library's launches in a HIP graph (torch.cuda.CUDAGraph),
as a serving loop replays one decode step of a block.

Nothing the library enqueues is a memset or an allocation, so a captured
step is a fixed sequence of kernel launches with fixed arguments; every
replay must give the bits of the eager call.  The replays are separated by
other eager work and host synchronisations, and each one is checked.
"""

import sys

import numpy as np
import pytest

from global_attention_zg_amd import inputs
from tests import zg_cases as zc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

KW = dict(rope_dim=42, rope_theta=10000.0, rms_eps=1e-6)
D = 128


@pytest.fixture(autouse=True)
def _gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"\n[case] {request.node.nodeid}", file=sys.stderr, flush=True)
    yield
    torch.cuda.synchronize()


def _binding():
    from global_attention_zg_amd import binding
    return binding


class Layer:
    """Device buffers of one layer's decode step (B sequences)."""

    def __init__(self, tag, B, Hq, Hkv, cap, ring, window, L, gated):
        bits = lambda t, shape: zc.to_dev(zc.bits((tag, 0, t), shape), torch)  # noqa: E731
        self.q = bits(inputs.T_Q, (B, Hq, D))
        self.kn = bits(inputs.T_KNEW, (B, Hkv, D))
        self.vn = bits(inputs.T_VNEW, (B, Hkv, D))
        self.kc = bits(inputs.T_KCACHE, (B, Hkv, cap, D))
        self.vc = bits(inputs.T_VCACHE, (B, Hkv, cap, D))
        self.g = bits(inputs.T_GATE, (B, Hq, D)) if gated else None
        self.gq = torch.from_numpy(inputs.norm_weight((tag, 0, inputs.T_GQ), D)).cuda()
        self.gk = torch.from_numpy(inputs.norm_weight((tag, 0, inputs.T_GK), D)).cuda()
        self.sl = torch.tensor(L, dtype=torch.int32, device="cuda")
        self.out = torch.empty_like(self.q)
        self.ring, self.window, self.cap = ring, window, cap
        bd = _binding()
        p = bd.make_params(B, 0, Hq, Hkv, D, window)
        self.ws = torch.empty(max(16, bd.zg_attn_decode_workspace_size(p, cap, 0)),
                              dtype=torch.uint8, device="cuda")

    def __call__(self):
        _binding().zg_attn_decode(self.q, self.kn, self.vn, self.kc, self.vc, self.sl,
                                  ring=self.ring, window=self.window, gate=self.g,
                                  q_norm_w=self.gq, k_norm_w=self.gk, out=self.out,
                                  workspace=self.ws, **KW)


def test_decode_block_step_replays_equal_eager():
    lens = [5, 300, 1000, 77]
    layers = [Layer(500 + i, 4, 16, 4, 128, True, 128, lens, True) for i in range(5)]
    layers.append(Layer(505, 4, 16, 4, 1024, False, 0, lens, False))  # several splits

    def step():
        for layer in layers:
            layer()

    step()
    torch.cuda.synchronize()
    ref = [layer.out.clone() for layer in layers]
    caches = [(layer.kc.clone(), layer.vc.clone()) for layer in layers]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for layer in layers:
            layer.out.fill_(float("nan"))
        noise = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        del noise
        for i, layer in enumerate(layers):
            assert torch.equal(layer.out.view(torch.int16), ref[i].view(torch.int16)), (rep, i)
            # the append is idempotent: the caches hold the same bits as after
            # the eager step
            assert torch.equal(layer.kc.view(torch.int16), caches[i][0].view(torch.int16))
            assert torch.equal(layer.vc.view(torch.int16), caches[i][1].view(torch.int16))


@pytest.mark.parametrize("window", [128, 0])
def test_forward_replays_equal_eager(window):
    """A captured forward replays to the eager bits; at window 0 this runs the
    persistent causal kernel, whose work-queue counters the captured key
    prologue clears on every replay."""
    bd = _binding()
    c = zc.fwd_case(510, 1, 700, 16, 4, gated=True)
    q, k, v, g = (zc.to_dev(c[n], torch) for n in ("q", "k", "v", "gate"))
    gq = torch.from_numpy(c["gq"]).cuda()
    gk = torch.from_numpy(c["gk"]).cuda()
    out = torch.empty_like(q)
    lse = torch.empty((1, 16, 700), dtype=torch.float32, device="cuda")
    ko = torch.empty_like(k)
    run = lambda: bd.zg_attn_fwd(q, k, v, g, gq, gk, window=window, out=out, lse=lse,  # noqa: E731
                                 k_out=ko, **KW)
    run()
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone(), ko.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ko.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref[0].view(torch.int16)), rep
        assert torch.equal(lse.view(torch.int32), ref[1].view(torch.int32)), rep
        assert torch.equal(ko.view(torch.int16), ref[2].view(torch.int16)), rep
    assert np.isfinite(ref[0].float().cpu().numpy()).all()
