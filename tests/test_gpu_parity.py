"""GPU parity: every stage of the HIP path against the CPU oracle on the same seeded
inputs, through the C ABI.

Bars: bit-exact for top-K indices (given identical fp32 logits), counts, offsets, the
restoration map, the row owners and the packed rows; max abs error <= 1e-4 for fp32
values (logits, coefficients, gates, fp32 layers); relative L2 <= 1e-2 for bf16 tensors
(whole tensor, or each expert segment for H and F).
"""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from mixture_experts_layer_gemm_amd import synth
from tests.gpu_common import (DeviceLayer, assert_close, host, rel_l2, say, to_device,
                              F32_MAX_ABS, BF16_REL_L2)

pytestmark = pytest.mark.gpu

moe = None


def setup_module(module):
    global moe
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_gemm_amd import moe as m
    moe = m


SMALL = ["C0", "S_softmax", "S_sigmoid", "S_selected", "S_capgate", "S_cap3shared", "S_f32",
         "S_tied", "S_KeqN", "S_N1", "S_stream", "S_stream_cap", "S_rankcap", "S_rankcap_stream",
         "S_wide", "S_wide192", "S_longT", "S_mid40", "S_mid100", "S_mid200"]
_cache = {}


def layer(name) -> DeviceLayer:
    if name not in _cache:
        _cache.clear()
        _cache[name] = DeviceLayer(synth.get_config(name))
    return _cache[name]


# ---------------------------------------------------------------------------------------
# a2: top-K and coefficients on identical fp32 logits
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("N,K", [(8, 2), (64, 4), (256, 8), (16, 16), (5, 3), (1, 1), (200, 7),
                                 (65, 16), (256, 16), (130, 1), (128, 5)])
@pytest.mark.parametrize("score,renorm", [(0, 1), (0, 0), (1, 1), (1, 0), (2, 1)])
def test_topk_bit_exact_on_identical_logits(N, K, score, renorm):
    if K > N:
        pytest.skip("K > N")
    say(f"topk N={N} K={K} score={score} renorm={renorm}")
    rng = np.random.default_rng(N * 100 + K)
    T = 333
    z = (rng.integers(-6, 7, size=(T, N)) * 0.25).astype(np.float32)   # many exact ties
    z[::7] = rng.standard_normal((len(z[::7]), N)).astype(np.float32)
    z[1, :] = 0.0
    z[1, ::2] = -0.0                                                     # -0.0 ties +0.0
    out = moe.moe_route(None, None, K, score=score, renorm=bool(renorm), alpha=2.5,
                        logits=torch.from_numpy(z).cuda(), logits_mode=1, want_counts=True)
    torch.cuda.synchronize()
    idx = O.topk_select(z, K)
    assert np.array_equal(host(out["topk_idx"]), idx)
    assert np.array_equal(host(out["C_req"]), O.requested_counts(idx, N))
    r = O.route_coefficients(z.astype(np.float64), idx, score, bool(renorm), 2.5)
    assert np.max(np.abs(host(out["topk_r"]) - r)) <= F32_MAX_ABS


# ---------------------------------------------------------------------------------------
# a1+a2: the router from x
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("name", SMALL)
def test_route_stage(name):
    L = layer(name)
    c = L.cfg
    say(f"route {name}")
    out = moe.moe_route(L.x, L.w_router, c.K, score=c.score, renorm=c.renorm, alpha=c.alpha,
                        logit_bias=L.bias, w_shared_gate=L.gate, want_logits=True)
    torch.cuda.synchronize()
    inp = L.inp
    z_ref = O.router_logits(L.x_f(), inp.as_float(inp.w_router), inp.logit_bias)
    z_gpu = host(out["logits"])
    assert np.max(np.abs(z_gpu - z_ref)) <= F32_MAX_ABS
    idx = O.topk_select(z_gpu, c.K)                    # selection decided on identical fp32 values
    assert np.array_equal(host(out["topk_idx"]), idx)
    assert np.array_equal(host(out["C_req"]), O.requested_counts(idx, c.N))
    r = O.route_coefficients(z_gpu.astype(np.float64), idx, c.score, c.renorm, c.alpha)
    assert np.max(np.abs(host(out["topk_r"]) - r)) <= F32_MAX_ABS
    if L.gate is not None:
        s_ref = O.shared_gate(L.x_f(), inp.as_float(inp.w_shared_gate))
        assert np.max(np.abs(host(out["s_tok"]) - s_ref)) <= F32_MAX_ABS
    flips = int(np.sum(np.any(O.topk_select(z_ref, c.K) != idx, axis=1)))
    say(f"  tokens whose fp64-logit selection differs: {flips}")


# ---------------------------------------------------------------------------------------
# a3+a4: counts, capacity, offsets, restoration map and packed rows
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("copy_rows", [True, False])
@pytest.mark.parametrize("name", SMALL)
def test_permute_stage(name, copy_rows):
    L = layer(name)
    c = L.cfg
    say(f"permute {name} capacity={L.capacity} copy_rows={copy_rows}")
    inp = L.inp
    z = O.router_logits(L.x_f(), inp.as_float(inp.w_router), inp.logit_bias)
    idx = O.topk_select(z, c.K)
    out = moe.moe_permute(L.x, torch.from_numpy(idx).cuda(), c.N, L.capacity,
                          capacity_group=c.capacity_group,
                          copy_rows=copy_rows)
    torch.cuda.synchronize()
    kept = L.keep(idx)
    perm = O.permutation(idx, kept, c.N)
    R = int(perm.offsets[-1])
    assert np.array_equal(host(out["C_req"]), O.requested_counts(idx, c.N))
    assert np.array_equal(host(out["C_keep"]), perm.C_keep)
    assert np.array_equal(host(out["offsets"]), perm.offsets)
    assert np.array_equal(host(out["dest_row"]), perm.dest_row)
    assert np.array_equal(host(out["row_token"])[:R], perm.row_token)
    if not copy_rows:
        assert out["x_perm"] is None
        return
    xp = out["x_perm"][:R]
    xs = L.x[torch.from_numpy(perm.row_token).long().cuda()]
    assert torch.equal(xp.view(torch.int16) if xp.dtype == torch.bfloat16 else xp.view(torch.int32),
                       xs.view(torch.int16) if xs.dtype == torch.bfloat16 else xs.view(torch.int32))


@pytest.mark.parametrize("copy_rows", [True, False])
@pytest.mark.parametrize("T,group,budget", [(64 * 256, 0, 700), (64 * 257 + 5, 0, 700),
                                            (64 * 257 + 5, 32, 9000)])
def test_permute_histogram_sizes(T, group, budget, copy_rows):
    """256 experts, top-8, Zipf-skewed and at capacity: 64 * 256 tokens give 65536
    histogram entries (placement in one launch, each workgroup re-reading them all), one
    more 64-token row (65792 entries) switches to the scan, then the map or row copy.
    Kept counts, offsets, restoration map and rows bit-exact on both sides of the switch
    ("Section 10", Eq. 21, 23, 25, 26)."""
    N, K = 256, 8
    say(f"permute T={T} N={N} K={K} group={group} budget={budget} copy_rows={copy_rows}")
    rng = np.random.default_rng(T + group)
    z = (rng.standard_normal((T, N)) + 2.0 * np.log(1.0 / np.arange(1, N + 1) ** 1.1)).astype(np.float32)
    idx = O.topk_select(z, K)
    xh = rng.standard_normal((T, 64)).astype(np.float32)
    x = torch.from_numpy(xh).cuda().to(torch.bfloat16)
    out = moe.moe_permute(x, torch.from_numpy(idx).cuda(), N, budget, copy_rows=copy_rows,
                          capacity_group=group)
    torch.cuda.synchronize()
    if group > 0:
        kept = O.keep_routes_rank_wide(idx, N, group, budget, n_sources=1)
    else:
        kept = O.keep_routes(idx, N, budget)
    perm = O.permutation(idx, kept, N)
    R = int(perm.offsets[-1])
    assert R < T * K  # routes were dropped
    assert np.array_equal(host(out["C_req"]), O.requested_counts(idx, N))
    assert np.array_equal(host(out["C_keep"]), perm.C_keep)
    assert np.array_equal(host(out["offsets"]), perm.offsets)
    assert np.array_equal(host(out["dest_row"]), perm.dest_row)
    assert np.array_equal(host(out["row_token"])[:R], perm.row_token)
    if copy_rows:
        xs = x[torch.from_numpy(perm.row_token).long().cuda()]
        assert torch.equal(out["x_perm"][:R].view(torch.int16), xs.view(torch.int16))


@pytest.mark.parametrize("N,K,group,budget", [(64, 4, 8, 1500), (64, 4, 8, 0), (64, 4, 64, 9000),
                                               (64, 4, 1, 300), (256, 8, 32, 2000),
                                               (16, 2, 4, 10 ** 6), (5, 3, 5, 7)])
def test_rank_wide_capacity_permute(N, K, group, budget):
    """Rank-wide capacity (Section 10.3, Eq. 23): kept counts, offsets and the restoration
    map bit-exact against the oracle's admission (local-expert-major, then source rank,
    prefix per split, four contiguous source shards), and the drops of every destination
    equal [R_q^req - B]_+ (Eq. 28)."""
    say(f"rank-wide capacity N={N} K={K} group={group} budget={budget}")
    rng = np.random.default_rng(N + K + group)
    T = 64 * 70 + 13
    z = (rng.standard_normal((T, N)) + 2.0 * np.log(1.0 / np.arange(1, N + 1) ** 1.1)).astype(np.float32)
    idx = O.topk_select(z, K)
    x = torch.zeros(T, 64, dtype=torch.bfloat16, device="cuda")
    out = moe.moe_permute(x, torch.from_numpy(idx).cuda(), N, budget, copy_rows=False,
                          capacity_group=group)
    torch.cuda.synchronize()
    kept = O.keep_routes_rank_wide(idx, N, group, budget, n_sources=4)
    perm = O.permutation(idx, kept, N)
    R = int(perm.offsets[-1])
    assert np.array_equal(host(out["C_keep"]), perm.C_keep)
    assert np.array_equal(host(out["offsets"]), perm.offsets)
    assert np.array_equal(host(out["dest_row"]), perm.dest_row)
    assert np.array_equal(host(out["row_token"])[:R], perm.row_token)
    Rq_req = O.rank_loads(host(out["C_req"]), group)
    Rq_keep = O.rank_loads(host(out["C_keep"]), group)
    assert [int(a - b) for a, b in zip(Rq_req, Rq_keep)] == \
        [O.drops_rank_wide(host(out["C_req"])[q * group:(q + 1) * group], budget)
         for q in range(N // group)]
    say(f"  kept {R} of {K * T}; destination loads kept {Rq_keep.tolist()[:8]}")


# ---------------------------------------------------------------------------------------
# a5+a6: grouped SwiGLU GEMM over ragged segments
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,packed", [("bf16", True), ("bf16", False), ("f32", False)])
@pytest.mark.parametrize("seg", [[0, 1, 129, 0, 400, 31, 256, 257], [300], [0, 0, 5], [1000, 2]])
def test_grouped_swiglu_ragged(seg, dtype, packed):
    say(f"grouped swiglu segments={seg} {dtype} packed={packed}")
    rng = np.random.default_rng(len(seg) + sum(seg))
    G, d, dff = len(seg), 192, 320
    rows = sum(seg)
    offsets = np.concatenate([[0], np.cumsum(seg)]).astype(np.int32)
    cfg = synth.Config("t", 0, T=1, d_model=d, N=1, K=1, d_r=dff, dtype=dtype)

    def draw(shape, std):
        v = (rng.standard_normal(shape) * std).astype(np.float32)
        return synth.bf16_bits(v) if dtype == "bf16" else v

    a_s = draw((rows + 7, d), 1.0)
    wg_s, wu_s, wd_s = draw((G, dff, d), 0.05), draw((G, dff, d), 0.05), draw((G, d, dff), 0.05)
    dec = (lambda b: synth.bf16_to_f32(b)) if dtype == "bf16" else (lambda b: b)
    wg_d, wu_d, wd_d = to_device(wg_s, dtype), to_device(wu_s, dtype), to_device(wd_s, dtype)
    if packed:
        wg_d, wu_d, wd_d = (moe.moe_pack_weights(w) for w in (wg_d, wu_d, wd_d))
    h, out = moe.moe_grouped_swiglu(to_device(a_s, dtype), torch.from_numpy(offsets).cuda(),
                                    wg_d, wu_d, wd_d, packed=packed)
    torch.cuda.synchronize()
    h, out = host(h), host(out)
    for g in range(G):
        lo, hi = offsets[g], offsets[g + 1]
        if hi == lo:
            continue
        H, F = O.swiglu(dec(a_s[lo:hi]), dec(wg_s[g]), dec(wu_s[g]), dec(wd_s[g]))
        assert_close(h[lo:hi], H, dtype, f"H segment {g}")
        assert_close(out[lo:hi], F, dtype, f"F segment {g}")


@pytest.mark.parametrize("dtype,packed", [("bf16", True), ("bf16", False), ("f32", False)])
def test_grouped_swiglu_gathered_rows(dtype, packed):
    """Packed row r of the gate/up pass reads a[row_index[r]] (the permutation fused into
    the operand load): ragged groups, repeated and out-of-order source rows."""
    say(f"grouped swiglu gathered rows {dtype} packed={packed}")
    rng = np.random.default_rng(11)
    seg = [0, 77, 130, 1, 0, 258]
    G, d, dff = len(seg), 128, 192
    rows = sum(seg)
    offsets = np.concatenate([[0], np.cumsum(seg)]).astype(np.int32)
    n_src = 150
    row_index = rng.integers(0, n_src, size=rows + 5).astype(np.int32)

    def draw(shape, std):
        v = (rng.standard_normal(shape) * std).astype(np.float32)
        return synth.bf16_bits(v) if dtype == "bf16" else v

    a_s = draw((n_src, d), 1.0)
    wg_s, wu_s, wd_s = draw((G, dff, d), 0.05), draw((G, dff, d), 0.05), draw((G, d, dff), 0.05)
    dec = (lambda b: synth.bf16_to_f32(b)) if dtype == "bf16" else (lambda b: b)
    wg_d, wu_d, wd_d = to_device(wg_s, dtype), to_device(wu_s, dtype), to_device(wd_s, dtype)
    if packed:
        wg_d, wu_d, wd_d = (moe.moe_pack_weights(w) for w in (wg_d, wu_d, wd_d))
    h, out = moe.moe_grouped_swiglu(to_device(a_s, dtype), torch.from_numpy(offsets).cuda(),
                                    wg_d, wu_d, wd_d, packed=packed,
                                    row_index=torch.from_numpy(row_index).cuda())
    torch.cuda.synchronize()
    assert h.shape[0] == rows + 5
    h, out = host(h), host(out)
    for g in range(G):
        lo, hi = offsets[g], offsets[g + 1]
        if hi == lo:
            continue
        H, F = O.swiglu(dec(a_s[row_index[lo:hi]]), dec(wg_s[g]), dec(wu_s[g]), dec(wd_s[g]))
        assert_close(h[lo:hi], H, dtype, f"H segment {g}")
        assert_close(out[lo:hi], F, dtype, f"F segment {g}")


SEG_MANY = [0, 1, 129, 0, 1000, 31, 256, 257, 700, 300, 640, 5, 900, 128, 511, 2]
# at least 1024 rows per group on average: the two-row-half (256-row tile) shape, with
# ragged last tiles of 164, 52, 20 and 33 rows and an empty group
SEG_LARGE = [1700, 0, 2100, 1300, 33]
# one group holds nearly every row, the rest a row or two: the XCD split falls inside
# the large group and among tiles of one or two rows
SEG_SKEW = [1, 0, 2999, 3, 0, 0, 64, 1, 2, 0, 1]


@pytest.mark.parametrize("seg", [SEG_MANY, SEG_LARGE, SEG_SKEW],
                         ids=["many_groups", "large_groups", "skewed_groups"])
@pytest.mark.parametrize("gathered", [False, True])
def test_grouped_swiglu_persistent_shapes(gathered, seg):
    """Shapes of the persistent GEMM (d_model, d_ff multiples of 256): ragged groups
    (empty, one row, many 128-row tiles) and more tiles than compute units, so that each
    workgroup runs several tiles back to back; few groups of many rows (two row halves
    per tile); optionally gathered rows."""
    say(f"grouped swiglu, persistent-kernel shapes, gathered={gathered}, seg={seg}")
    rng = np.random.default_rng(29 + gathered + 7 * len(seg))
    G, d, dff = len(seg), 768, 1024
    rows = sum(seg)
    offsets = np.concatenate([[0], np.cumsum(seg)]).astype(np.int32)

    def draw(shape, std):
        return synth.bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))

    n_src = 3000 if gathered else rows
    a_s = draw((n_src, d), 1.0)
    ri = rng.integers(0, n_src, size=rows).astype(np.int32) if gathered else None
    wg_s, wu_s, wd_s = draw((G, dff, d), 0.03), draw((G, dff, d), 0.03), draw((G, d, dff), 0.03)
    dec = synth.bf16_to_f32
    wg_d, wu_d, wd_d = (moe.moe_pack_weights(to_device(w, "bf16")) for w in (wg_s, wu_s, wd_s))
    h, out = moe.moe_grouped_swiglu(to_device(a_s, "bf16"), torch.from_numpy(offsets).cuda(),
                                    wg_d, wu_d, wd_d, packed=True,
                                    row_index=None if ri is None else torch.from_numpy(ri).cuda())
    torch.cuda.synchronize()
    h, out = host(h), host(out)
    for g in range(G):
        lo, hi = offsets[g], offsets[g + 1]
        if hi == lo:
            continue
        src = a_s[ri[lo:hi]] if gathered else a_s[lo:hi]
        H, F = O.swiglu(dec(src), dec(wg_s[g]), dec(wu_s[g]), dec(wd_s[g]))
        assert_close(h[lo:hi], H, "bf16", f"H segment {g}")
        assert_close(out[lo:hi], F, "bf16", f"F segment {g}")


@pytest.mark.parametrize("name", ["S_stream", "S_stream_cap", "S_softmax"])
def test_expert_stage(name):
    """moe_experts (routed experts + shared MLP; one launch per pass when the shapes fit
    the persistent kernel, else separate grouped GEMMs): the gate/up and down passes run
    separately give the same bits as both at once, and the outputs match the oracle."""
    L = layer(name)
    c = L.cfg
    say(f"expert stage {name}")
    inp = L.inp
    z = O.router_logits(L.x_f(), inp.as_float(inp.w_router), inp.logit_bias)
    idx = O.topk_select(z, c.K)
    pm = moe.moe_permute(L.x, torch.from_numpy(idx).cuda(), c.N, L.capacity, copy_rows=False,
                         capacity_group=c.capacity_group)
    perm = O.permutation(idx, L.keep(idx), c.N)
    rows = moe.max_rows(L.T, c.N, c.K, L.capacity, c.capacity_group)
    wg, wu, wd = (moe.moe_pack_weights(w) for w in (L.w_gate, L.w_up, L.w_down))
    sm = moe.pack_shared(L.shared) if L.shared else None
    if sm is not None:
        sm = tuple(moe.moe_pack_weights(w[None])[0] for w in sm)
    both = moe.moe_experts(L.x, pm["row_token"], pm["offsets"], rows, wg, wu, wd, shared=sm,
                           packed=True)
    split = moe.moe_experts(L.x, pm["row_token"], pm["offsets"], rows, wg, wu, wd, shared=sm,
                            packed=True, pass_=1)
    moe.moe_experts(L.x, pm["row_token"], pm["offsets"], rows, wg, wu, wd, shared=sm,
                    packed=True, pass_=2, out=split)
    torch.cuda.synchronize()
    R = int(perm.offsets[-1])
    for k in ("h_perm", "f_perm", "h_shared", "g"):
        if both[k] is None:
            continue
        n = R if k in ("h_perm", "f_perm") else L.T
        assert torch.equal(both[k][:n].view(torch.int16), split[k][:n].view(torch.int16)), k
    Hg, Fg = host(both["h_perm"])[:R], host(both["f_perm"])[:R]
    xs = L.x_f()
    for e in range(c.N):
        lo, hi = perm.offsets[e], perm.offsets[e + 1]
        if hi > lo:
            H, F = O.swiglu(xs[perm.row_token[lo:hi]], *inp.expert_f32(e))
            assert_close(Hg[lo:hi], H, "bf16", f"H expert {e}")
            assert_close(Fg[lo:hi], F, "bf16", f"F expert {e}")
    if sm is not None:
        assert_close(host(both["g"]), O.shared_output(xs, inp.shared_f32()), "bf16", "G")


# ---------------------------------------------------------------------------------------
# a8: combine
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["C0", "S_capgate", "S_selected"])
def test_combine_stage(name):
    L = layer(name)
    c = L.cfg
    say(f"combine {name}")
    res = L.oracle_forward()
    dt = c.dtype
    F_in = synth.bf16_bits(res.F_perm.astype(np.float32)) if dt == "bf16" else res.F_perm.astype(np.float32)
    dec = synth.bf16_to_f32 if dt == "bf16" else (lambda v: v)
    G_in = None
    if res.G is not None:
        G_in = synth.bf16_bits(res.G.astype(np.float32)) if dt == "bf16" else res.G.astype(np.float32)
    r32 = res.r.astype(np.float32)
    s_tok = None if res.s_tok is None else res.s_tok.astype(np.float32)
    Fd = to_device(F_in if len(F_in) else np.zeros((1, c.d_model), F_in.dtype), dt)
    y = moe.moe_combine(Fd, torch.from_numpy(res.perm.dest_row.astype(np.int32)).cuda(),
                        torch.from_numpy(r32).cuda(),
                        None if G_in is None else to_device(G_in, dt), s=c.s,
                        s_tok=None if s_tok is None else torch.from_numpy(s_tok).cuda())
    torch.cuda.synchronize()
    # reference: Eq. 80 on the exact values the kernel was given
    y_ref = O.combine(dec(F_in), res.perm.dest_row, r32, None if G_in is None else dec(G_in),
                      s_tok if s_tok is not None else c.s)
    assert_close(host(y), y_ref, dt, "y")


# ---------------------------------------------------------------------------------------
# whole layer, small workloads: every intermediate against the oracle
# ---------------------------------------------------------------------------------------
def check_forward(L: DeviceLayer, full=True, sample_tokens=None, keep_x_perm=False):
    c = L.cfg
    dt = c.dtype
    say(f"forward {c.name} T={L.T} capacity={L.capacity} keep_x_perm={keep_x_perm}")
    lay = moe.MoELayer(L.x, L.w_router, L.w_gate, L.w_up, L.w_down, c.K,
                       keep_intermediates=True, keep_x_perm=keep_x_perm, **L.layer_kwargs())
    y = lay.forward()
    torch.cuda.synchronize()
    o = lay.out
    z_gpu = host(o["logits"])
    inp = L.inp
    z_ref = O.router_logits(L.x_f(), inp.as_float(inp.w_router), inp.logit_bias)
    assert np.max(np.abs(z_gpu - z_ref)) <= F32_MAX_ABS
    flips = int(np.sum(np.any(O.topk_select(z_ref, c.K) != O.topk_select(z_gpu, c.K), axis=1)))
    say(f"  tokens whose fp64-logit selection would differ: {flips}")
    if full:
        res = L.oracle_forward(logits_override=z_gpu)
        idx, r, s_tok, perm = res.idx, res.r, res.s_tok, res.perm
    else:
        idx = O.topk_select(z_gpu, c.K)
        r = O.route_coefficients(z_gpu.astype(np.float64), idx, c.score, c.renorm, c.alpha)
        s_tok = None if inp.w_shared_gate is None else O.shared_gate(L.x_f(), inp.as_float(inp.w_shared_gate))
        perm = O.permutation(idx, L.keep(idx), c.N)
    R = int(perm.offsets[-1])
    assert np.array_equal(host(o["topk_idx"]), idx)
    assert np.max(np.abs(host(o["topk_r"]) - r)) <= F32_MAX_ABS
    if s_tok is not None:
        assert np.max(np.abs(host(o["s_tok"]) - s_tok)) <= F32_MAX_ABS
    assert np.array_equal(host(o["C_req"]), O.requested_counts(idx, c.N))
    assert np.array_equal(host(o["C_keep"]), perm.C_keep)
    assert np.array_equal(host(o["offsets"]), perm.offsets)
    assert np.array_equal(host(o["dest_row"]), perm.dest_row)
    assert np.array_equal(host(o["row_token"])[:R], perm.row_token)
    if keep_x_perm:
        row_tok = torch.from_numpy(perm.row_token).long().cuda()
        assert torch.equal(o["x_perm"][:R], L.x[row_tok])
    else:
        assert "x_perm" not in o
    say(f"  routing bit-exact; R={R} kept of {c.K * L.T}")
    if full:
        Hg, Fg = host(o["h_perm"])[:R], host(o["f_perm"])[:R]
        worst = 0.0
        for e in range(c.N):
            lo, hi = perm.offsets[e], perm.offsets[e + 1]
            if hi > lo:
                worst = max(worst, assert_close(Hg[lo:hi], res.H_perm[lo:hi], dt, f"H expert {e}"))
                worst = max(worst, assert_close(Fg[lo:hi], res.F_perm[lo:hi], dt, f"F expert {e}"))
        if res.G is not None:
            assert_close(host(o["g"]), res.G, dt, "G")
        err = assert_close(host(y), res.y, dt, "y")
        say(f"  y err {err:.3g}; worst H/F segment err {worst:.3g}")
    else:
        toks = sample_tokens
        y_ref = O.forward_tokens(L.spec(), toks, L.x_f(), idx, r, perm.dest_row, inp.expert_f32,
                                 inp.shared_f32(), s_tok)
        err = assert_close(host(y)[toks], y_ref, dt, "y (sampled tokens)")
        say(f"  sampled y err {err:.3g} over {len(toks)} tokens")
    return lay


@pytest.mark.parametrize("name", SMALL)
def test_forward_small(name):
    check_forward(layer(name))


@pytest.mark.parametrize("name", ["S_capgate", "S_f32"])
def test_forward_with_x_perm_copy(name):
    check_forward(layer(name), keep_x_perm=True)


def test_forward_is_deterministic():
    L = layer("S_capgate")
    lay = moe.MoELayer(L.x, L.w_router, L.w_gate, L.w_up, L.w_down, L.cfg.K, **L.layer_kwargs())
    a = lay.forward().clone()
    for _ in range(3):
        b = lay.forward()
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_forward_edge_cases():
    cfg = synth.get_config("S_softmax")
    say("edge: T=1, T=0, capacity 0")
    L1 = DeviceLayer(cfg, T=1)
    check_forward(L1)
    # capacity 0: every route dropped, y = s * g
    L = layer("S_softmax")
    kw = L.layer_kwargs()
    kw["capacity"] = 0
    lay = moe.MoELayer(L.x, L.w_router, L.w_gate, L.w_up, L.w_down, cfg.K, keep_intermediates=True, **kw)
    y = lay.forward()
    torch.cuda.synchronize()
    assert np.all(host(lay.out["dest_row"]) == -1)
    assert np.all(host(lay.out["C_keep"]) == 0)
    G = O.shared_output(L.x_f(), L.inp.shared_f32())
    assert_close(host(y), cfg.s * G, "bf16", "y with every route dropped")
    # T = 0: nothing enqueued, status OK
    x0 = L.x[:0]
    st = moe.lib.moe_route(0, cfg.d_model, cfg.N, cfg.K, 0, 1, 1.0, 1, x0.data_ptr() or 1,
                           L.w_router.data_ptr(), None, None, None, None, 0, 1, 1, None, None, None,
                           0, None)
    assert st == moe.MOE_OK


def test_pack_weights_layout_bit_exact():
    """moe_pack_weights writes w[g][32 nb + (l & 31)][16 kb + 8 (l >> 5) + e] at
    packed[g][nb][kb][l][e] (the layout documented in include/moe.h)."""
    rng = np.random.default_rng(3)
    G, N, K = 3, 128, 192
    w = rng.integers(0, 1 << 16, size=(G, N, K), dtype=np.uint16)
    p = host_bits(moe.moe_pack_weights(to_device(w, "bf16")))
    ref = w.reshape(G, N // 32, 32, K // 16, 2, 8).transpose(0, 1, 3, 4, 2, 5).reshape(G, N, K)
    assert np.array_equal(p, ref)


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name", ["S_softmax", "S_capgate"])
def test_forward_row_major_weights(name):
    """The row-major weight path (no packing) gives the same results."""
    L = layer(name)
    c = L.cfg
    say(f"forward row-major {name}")
    a = moe.MoELayer(L.x, L.w_router, L.w_gate, L.w_up, L.w_down, c.K, pack_weights=False,
                     **L.layer_kwargs())
    b = moe.MoELayer(L.x, L.w_router, L.w_gate, L.w_up, L.w_down, c.K, pack_weights=True,
                     **L.layer_kwargs())
    ya = a.forward().float().cpu().numpy()
    yb = b.forward().float().cpu().numpy()
    torch.cuda.synchronize()
    assert rel_l2(ya, yb) <= 2e-3
    res = L.oracle_forward()
    assert_close(ya, res.y, c.dtype, "y row-major")
