"""GPU parity of the balance statistics and drop diagnostics (Section 10 of the
Mixture-of-Experts layer page: Eq. 22, 27, 30, 38, 39 and Sections 10.2-10.3) against the
oracle, on the routing the forward actually took.

The oracle is handed the kernel's own fp32 logits, top-K, kept mask and coefficients, so
the comparison isolates the statistics. Bars: integer-valued statistics bit-exact; P,
the scalar N f.P and the ratios within 1e-5 absolute (fp32 per-token normalization,
fixed-order fp32 partial sums of 64 tokens, fp64 totals)."""
import math

import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from mixture_experts_layer_gemm_amd import synth
from tests.gpu_common import DeviceLayer, host, say

pytestmark = pytest.mark.gpu

moe = None
STAT_TOL = 1e-5
INTEGER_STATS = ("never_selected", "tokens_lost_any", "tokens_lost_all")


def setup_module(module):
    global moe
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_gemm_amd import moe as m
    moe = m


def oracle_stats(o, N, score, group=0):
    z = host(o["logits"]).astype(np.float64)
    idx = host(o["topk_idx"])
    kept = host(o["dest_row"]) >= 0
    r = host(o["topk_r"]).astype(np.float64)
    return O.balance_stats(O.normalized_scores(z, score), idx, kept, r, N, group=group)


def compare(P, st: dict, ref: O.BalanceStats, what: str):
    P = host(P).astype(np.float64)
    assert np.max(np.abs(P - ref.P)) <= STAT_TOL, f"{what}: P"
    for name in moe.STAT_NAMES:
        got, want = st[name], float(getattr(ref, name))
        if math.isnan(want):
            assert math.isnan(got), f"{what}: {name} {got} (want NaN)"
        elif name in INTEGER_STATS:
            assert got == want, f"{what}: {name} {got} != {want}"
        else:
            assert abs(got - want) <= STAT_TOL * max(1.0, abs(want)), f"{what}: {name} {got} vs {want}"


@pytest.mark.parametrize("name", ["C0", "S_softmax", "S_sigmoid", "S_selected", "S_capgate",
                                  "S_cap3shared", "S_f32", "S_KeqN", "S_N1", "S_stream_cap",
                                  "S_rankcap", "S_rankcap_stream"])
def test_balance_stats_match_oracle(name):
    L = DeviceLayer(synth.get_config(name))
    c = L.cfg
    say(f"balance stats {name} T={L.T} N={c.N} K={c.K} capacity={L.capacity}")
    lay = moe.MoELayer(L.x, L.w_router, L.w_gate, L.w_up, L.w_down, c.K,
                       keep_intermediates=True, balance_stats=True, **L.layer_kwargs())
    lay.forward()
    torch.cuda.synchronize()
    o = lay.out
    ref = oracle_stats(o, c.N, c.score, c.capacity_group)
    compare(o["balance_P"], moe.stats_dict(o["balance_stats"]), ref, f"{name} (forward)")
    # the standalone entry point on the same routing gives the same bits
    P, st = moe.moe_balance_stats(o["logits"], o["C_req"], o["C_keep"], o["dest_row"],
                                  o["topk_r"], score=c.score, expert_group=c.capacity_group)
    torch.cuda.synchronize()
    assert torch.equal(P, o["balance_P"])
    assert torch.equal(st.view(torch.int32), o["balance_stats"].view(torch.int32))
    d = moe.stats_dict(st)
    say(f"  lbl {d['lbl']:.4f} imax_req {d['imax_req']:.3f} imax_keep {d['imax_keep']:.3f} "
        f"delta {d['delta_route']:.4f} lost_any {d['tokens_lost_any']:.0f}")


def test_balance_stats_capacity_edges():
    """Capacity 0 drops every route (Eq. 27 = 1, every token loses all K routes and all of
    its selected weight, kept-count ratios undefined); capacity 1 on a single token."""
    L = DeviceLayer(synth.get_config("S_softmax"))
    c = L.cfg
    for cap in (0, 1):
        kw = L.layer_kwargs()
        kw["capacity"] = cap
        lay = moe.MoELayer(L.x, L.w_router, L.w_gate, L.w_up, L.w_down, c.K,
                           keep_intermediates=True, balance_stats=True, **kw)
        lay.forward()
        torch.cuda.synchronize()
        o = lay.out
        st = moe.stats_dict(o["balance_stats"])
        compare(o["balance_P"], st, oracle_stats(o, c.N, c.score), f"capacity {cap}")
        if cap == 0:
            assert st["delta_route"] == 1.0 and st["tokens_lost_all"] == L.T
            assert math.isnan(st["imax_keep"]) and abs(st["weight_removed"] - 1.0) <= STAT_TOL
    L1 = DeviceLayer(synth.get_config("S_sigmoid"), T=1)
    lay = moe.MoELayer(L1.x, L1.w_router, L1.w_gate, L1.w_up, L1.w_down, L1.cfg.K,
                       keep_intermediates=True, balance_stats=True, **L1.layer_kwargs())
    lay.forward()
    torch.cuda.synchronize()
    compare(lay.out["balance_P"], moe.stats_dict(lay.out["balance_stats"]),
            oracle_stats(lay.out, L1.cfg.N, L1.cfg.score), "T=1")


def test_balance_stats_on_given_logits_many_blocks():
    """Standalone entry on synthetic routing spanning many 64-token blocks and a ragged
    tail, with N = 256 (one expert per thread of the final reduction), both score kinds."""
    rng = np.random.default_rng(7)
    T, N, K = 64 * 37 + 19, 256, 8
    z = (rng.standard_normal((T, N)) * 1.5).astype(np.float32)
    idx = O.topk_select(z, K)
    C_req = O.requested_counts(idx, N)
    cap = int(np.median(C_req))
    kept = O.keep_routes(idx, N, cap)
    perm = O.permutation(idx, kept, N)
    for score, group in ((O.SOFTMAX, 0), (O.SIGMOID, 32), (O.SOFTMAX, 256), (O.SIGMOID, 1)):
        r = O.route_coefficients(z.astype(np.float64), idx, score, True, 1.0).astype(np.float32)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        P, st = moe.moe_balance_stats(dev(z), dev(C_req.astype(np.int32)),
                                      dev(perm.C_keep.astype(np.int32)),
                                      dev(perm.dest_row.astype(np.int32)), dev(r), score=score,
                                      expert_group=group)
        torch.cuda.synchronize()
        ref = O.balance_stats(O.normalized_scores(z.astype(np.float64), score), idx, kept,
                              r.astype(np.float64), N, group=group)
        compare(P, moe.stats_dict(st), ref, f"synthetic score={score} group={group}")
