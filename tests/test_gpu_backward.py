"""GPU parity of the fixed-router backward (Section 21.3 of the merge page: gradients with
the router coefficients held fixed, through the Eq. 80 combine and the Eq. 74 SwiGLU
experts) against the oracle's backward, through the C ABI.

The oracle is given the GPU forward's own routing (selected experts, kept routes, fp32
coefficients, shared gate) and the same bf16 upstream gradient. Bars: the packed
transposed weights bit-exact; dx and every expert's and shared expert's weight
gradients within relative L2 1e-2 (bf16 intermediates dF, A, B, dH, dA, dB, H with fp32
accumulation); weight gradients of experts without kept rows exactly zero."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from mixture_experts_layer_gemm_amd import synth
from tests.gpu_common import DeviceLayer, assert_close, host, rel_l2, say, to_device, BF16_REL_L2

pytestmark = pytest.mark.gpu

moe = None


def setup_module(module):
    global moe
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_gemm_amd import moe as m
    moe = m


@pytest.mark.parametrize("G,Ka,Kb,Nn", [(3, 128, 0, 192), (2, 192, 192, 256), (1, 64, 128, 64)])
def test_pack_weights_transposed_bit_exact(G, Ka, Kb, Nn):
    """The transposed packing equals moe_pack_weights of the explicitly transposed stack."""
    say(f"pack transposed G={G} Ka={Ka} Kb={Kb} N={Nn}")
    g = torch.Generator().manual_seed(G * 1000 + Ka + Kb)
    wa = torch.randn(G, Ka, Nn, generator=g).to(torch.bfloat16).cuda()
    wb = torch.randn(G, Kb, Nn, generator=g).to(torch.bfloat16).cuda() if Kb else None
    got = moe.moe_pack_weights_transposed(wa, wb)
    stack = wa if wb is None else torch.cat([wa, wb], 1)
    want = moe.moe_pack_weights(stack.transpose(1, 2).contiguous())
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


def run_backward(L, seed=0):
    c = L.cfg
    lay = moe.MoELayer(L.x, L.w_router, L.w_gate, L.w_up, L.w_down, c.K, trainable=True,
                       **L.layer_kwargs())
    lay.forward()
    g = torch.Generator().manual_seed(1234 + seed)
    dy_f = torch.randn(L.T, c.d_model, generator=g)
    dy = dy_f.to(torch.bfloat16).cuda()
    grads = lay.backward(dy)
    torch.cuda.synchronize()
    return lay, dy, grads


def oracle_grads(L, lay, dy, experts=None):
    c = L.cfg
    o = lay.out
    idx = host(o["topk_idx"])
    kept = host(o["dest_row"]) >= 0
    r = host(o["topk_r"]).astype(np.float64)
    s = host(o["s_tok"]).astype(np.float64) if "s_tok" in o else c.s
    dy_f = host(dy).astype(np.float64)
    inp = L.inp
    return O.backward(L.x_f(), idx, kept, r, inp.expert_f32, c.N, dy_f, inp.shared_f32(), s), kept


@pytest.mark.parametrize("name", ["S_softmax", "S_capgate", "S_cap3shared", "S_selected",
                                  "S_stream", "S_stream_cap", "S_rankcap", "S_KeqN"])
def test_backward_matches_oracle(name):
    L = DeviceLayer(synth.get_config(name))
    if L.cfg.dtype != "bf16":
        pytest.skip("the backward is bf16")
    check_backward(L)


def check_backward(L):
    """dx, every expert's weight gradients (exactly zero without kept rows) and every
    shared expert's weight gradients against the oracle's backward."""
    c = L.cfg
    say(f"backward {c.name} T={L.T} N={c.N} K={c.K} d_r={c.d_r} d_s={c.d_s} capacity={L.capacity}")
    lay, dy, gr = run_backward(L)
    ref, kept = oracle_grads(L, lay, dy)
    err = assert_close(host(gr["dx"]), ref.dx, "bf16", "dx")
    idx = host(lay.out["topk_idx"])
    worst = 0.0
    for e in range(c.N):
        if not np.any((idx == e) & kept):
            for k in ("dw_gate", "dw_up", "dw_down"):
                assert not gr[k][e].any(), f"{k} of expert {e} without rows"
            continue
        for k in ("dw_gate", "dw_up", "dw_down"):
            worst = max(worst, assert_close(host(gr[k][e]), getattr(ref, k)[e], "bf16", f"{k} expert {e}"))
    off = 0
    for j, w in enumerate(c.shared_widths):
        sl = slice(off, off + w)
        assert_close(host(gr["dws_gate"])[sl], ref.shared[j][0], "bf16", f"dws_gate {j}")
        assert_close(host(gr["dws_up"])[sl], ref.shared[j][1], "bf16", f"dws_up {j}")
        assert_close(host(gr["dws_down"])[:, sl], ref.shared[j][2], "bf16", f"dws_down {j}")
        off += w
    say(f"  dx err {err:.3g}; worst expert weight-gradient err {worst:.3g}")


def test_backward_is_deterministic_and_capacity_zero():
    """Repeated backward passes give the same bits; with capacity 0 every route is
    dropped, the routed weight gradients are zero and dx is the shared branch's alone."""
    L = DeviceLayer(synth.get_config("S_capgate"))
    c = L.cfg
    lay, dy, g1 = run_backward(L)
    g2 = lay.backward(dy)
    torch.cuda.synchronize()
    for k in ("dx", "dw_gate", "dw_up", "dw_down", "dws_gate", "dws_up", "dws_down"):
        a, b = g1[k], g2[k]
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), k
    kw = L.layer_kwargs()
    kw["capacity"] = 0
    lay0 = moe.MoELayer(L.x, L.w_router, L.w_gate, L.w_up, L.w_down, c.K, trainable=True, **kw)
    lay0.forward()
    g0 = lay0.backward(dy)
    torch.cuda.synchronize()
    assert not g0["dw_gate"].any() and not g0["dw_up"].any() and not g0["dw_down"].any()
    ref, _ = oracle_grads(L, lay0, dy)
    assert_close(host(g0["dx"]), ref.dx, "bf16", "dx, every route dropped")


@pytest.mark.timeout(900)
def test_backward_full_size_whole_oracle():
    """The 64-expert top-4 layer (T = 4096, d_model = 2048, d_r = 2560, d_s = 1280): dx on
    every token and the weight gradients of every expert and of the shared MLP against
    the oracle's backward of the whole layer (about 1.4 TFLOP of fp64 host BLAS)."""
    cfg = synth.get_config("C1")
    L = DeviceLayer(cfg)
    say("backward C1 (full size, whole oracle)")
    lay, dy, gr = run_backward(L)
    ref, kept = oracle_grads(L, lay, dy)
    err = assert_close(host(gr["dx"]), ref.dx, "bf16", "dx")
    idx = host(lay.out["topk_idx"])
    worst = 0.0
    for e in range(cfg.N):
        assert np.any((idx == e) & kept), f"expert {e} has no rows at this size"
        for k in ("dw_gate", "dw_up", "dw_down"):
            worst = max(worst, assert_close(host(gr[k][e]), getattr(ref, k)[e], "bf16", f"{k} expert {e}"))
    assert_close(host(gr["dws_gate"]), ref.shared[0][0], "bf16", "dws_gate")
    assert_close(host(gr["dws_up"]), ref.shared[0][1], "bf16", "dws_up")
    assert_close(host(gr["dws_down"]), ref.shared[0][2], "bf16", "dws_down")
    say(f"  dx err {err:.3g}; worst expert weight-gradient err {worst:.3g}")
