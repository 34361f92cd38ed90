"""The library's entry points under HIP graph capture: they allocate nothing and record
no memset, so a captured whole-layer forward (and backward) replays to the eager bits.

Each graph is replayed several times with unrelated eager work and synchronizations in
between, and every replay is compared with the eager result."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_gemm_amd import synth
from tests.gpu_common import DeviceLayer, host, say

pytestmark = pytest.mark.gpu

moe = None


def setup_module(module):
    global moe
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_gemm_amd import moe as m
    moe = m


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm, not captured
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    return g, out


def unrelated_eager_work():
    a = torch.randn(512, 512, device="cuda")
    (a @ a).sum().item()


@pytest.mark.parametrize("name", ["S_stream_cap", "S_capgate", "S_rankcap"])
def test_forward_graph_replays_match_eager(name):
    L = DeviceLayer(synth.get_config(name))
    c = L.cfg
    say(f"graph forward {name}")
    acc = torch.zeros(c.N, dtype=torch.int32, device="cuda")
    lay = moe.MoELayer(L.x, L.w_router, L.w_gate, L.w_up, L.w_down, c.K, keep_intermediates=True,
                       balance_stats=True, count_accum=acc, **L.layer_kwargs())
    y0 = lay.forward().clone()
    st0 = lay.out["balance_stats"].clone()
    torch.cuda.synchronize()
    creq = host(lay.out["C_req"]).astype(np.int64)
    g, _ = capture(lambda: lay.forward())
    done = 2  # the eager call and the warm-up call before capture
    for i in range(3):
        lay.y.zero_()
        unrelated_eager_work()
        g.replay()
        torch.cuda.synchronize()
        done += 1
        assert torch.equal(bits(lay.y), bits(y0)), f"replay {i}: y"
        assert torch.equal(bits(lay.out["balance_stats"]), bits(st0)), f"replay {i}: statistics"
        assert np.array_equal(host(acc).astype(np.int64), done * creq), f"replay {i}: counts"


def test_backward_graph_replays_match_eager():
    L = DeviceLayer(synth.get_config("S_stream_cap"))
    c = L.cfg
    say("graph backward S_stream_cap")
    lay = moe.MoELayer(L.x, L.w_router, L.w_gate, L.w_up, L.w_down, c.K, trainable=True,
                       **L.layer_kwargs())
    lay.forward()
    dy = torch.randn(L.T, c.d_model, device="cuda").to(torch.bfloat16)
    eager = lay.backward(dy)
    ref = {k: v.clone() for k, v in eager.items() if k != "_workspace" and v is not None}
    torch.cuda.synchronize()
    g, out = capture(lambda: lay.backward(dy))
    for i in range(3):
        for k in ref:
            out[k].zero_()
        unrelated_eager_work()
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(bits(out[k]), bits(v)), f"replay {i}: {k}"
