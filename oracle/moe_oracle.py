"""Plain, slow, fp64 CPU oracle for the forward pass of one mixture-of-experts layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import or call it. It shares no code with the HIP library and imports nothing from
the package; callers hand it plain NumPy arrays (bf16 inputs already widened to float).

Every value is computed in float64 from the exact stored input values, with no
intermediate rounding. Each step cites the passage of the source pages it follows:

* p1 = "Section 21: Merging Routed and Shared Expert Activations" (Olmo-core MoE report)
* p2 = "Appendix E: Expert-Merge Normalization in Public MoE Models"
* p3 = "Shared and Fine-Grained Experts" (AI wiki entry with a PyTorch listing)
* p4 = "Section 20: One Shared Expert Is All You Need"
* p5 = "Section 10: Routing, Capacity, and Load Balancing"

Weights use the layout of a PyTorch ``Linear.weight``: the pages write the SwiGLU expert
in row-vector form, E(x) = [SiLU(x W_g) * (x W_u)] W_d (p4, Eq. 74); here
``w_gate = W_g^T`` with shape [d_ff, d_model], ``w_up = W_u^T`` [d_ff, d_model] and
``w_down = W_d^T`` [d_model, d_ff].

Readings taken where the pages leave a step open:
  * top-K ties go to the lower expert index; -0.0 and +0.0 compare equal;
  * the K output slots of a token are ordered by descending key, ties by index;
  * selection uses the (biased) logit for every score function;
  * without renormalization the routed coefficient is alpha * q_i;
  * per-expert capacity keeps the first `capacity` routes in token-index order;
  * kept segments are laid out in ascending expert order, rows by ascending token.
Parity pins for every function live in tests/test_oracle_pins.py; no function here is
"parity unpinned".
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Optional, Sequence

import numpy as np

SOFTMAX = 0            # softmax over all N logits (p1 Eq. 83 with renorm; p2 Qwen/OLMoE rows without)
SIGMOID = 1            # sigmoid affinities (p2 Table 52, DeepSeek-V3 row)
SOFTMAX_SELECTED = 2   # softmax over the K selected logits only (p2 Table 52, Mixtral row)


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _sigmoid(v: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-v))


def silu(v: np.ndarray) -> np.ndarray:
    """SiLU(v) = v * sigmoid(v), the gate nonlinearity of SwiGLU (p4 Eq. 74)."""
    return _f64(v) * _sigmoid(_f64(v))


# ----------------------------------------------------------------------------------------
# a1: router logits
# ----------------------------------------------------------------------------------------
def router_logits(x, w_router, logit_bias=None) -> np.ndarray:
    """z = x W_r^T (+ b): the bias-free router projection of the p3 listing (`gate`,
    a Linear from d_model to n_routed without bias; "Router projection and gating
    function" in p5 Table 16). An optional per-expert bias b is added to every logit."""
    z = _f64(x) @ _f64(w_router).T
    if logit_bias is not None:
        z = z + _f64(logit_bias)[None, :]
    return z


def shared_gate(x, w_shared_gate) -> np.ndarray:
    """s(x) = sigmoid(x w_s): the learned sigmoid shared-expert gate (p2 Table 52,
    Qwen rows), one scalar per token from a d_model-vector."""
    return _sigmoid(_f64(x) @ _f64(w_shared_gate))


# ----------------------------------------------------------------------------------------
# a2: selection and routed coefficients
# ----------------------------------------------------------------------------------------
def topk_select(keys, K: int) -> np.ndarray:
    """S(x): the K experts whose keys outrank every unselected expert (p1 Eq. 80 with
    |S| = K; p5 Section 10.7.1 ordering constraint). Ties go to the lower index, and
    the slots come out by descending key, then ascending index. The comparison is done
    in the precision of `keys` (pass float32 logits to decide in float32)."""
    keys = np.asarray(keys)
    T, N = keys.shape
    if not (1 <= K <= N):
        raise ValueError("need 1 <= K <= N")
    neg = -keys
    neg = np.where(neg == 0, np.zeros_like(neg), neg)  # -0.0 and +0.0 are the same key
    index = np.broadcast_to(np.arange(N), (T, N))
    order = np.lexsort((index, neg), axis=-1)        # primary: -key, secondary: index
    return order[:, :K].astype(np.int32)


def selection_keys(z, score: int, expert_bias=None) -> np.ndarray:
    """Keys of auxiliary-loss-free biased selection S_t = TopK_i(a_{t,i} + b_i) (p5
    Eq. 35): a = z for the softmax rules, a = sigmoid(z) for sigmoid affinities. The
    persistent bias b moves only the selection, never the weights. Without a bias the
    keys are the logits themselves (sigmoid is monotone). The sum is taken in the
    precision of the inputs (pass float32 logits and bias to decide in float32)."""
    z = np.asarray(z)
    if expert_bias is None:
        return z
    b = np.asarray(expert_bias, dtype=z.dtype)
    a = 1.0 / (1.0 + np.exp(-z)) if score == SIGMOID else z
    return a.astype(z.dtype) + b[None, :]


def bias_update(expert_bias, C_fb, gamma: float) -> np.ndarray:
    """One step of the hard-count controller (p5 Eq. 36-37):
    b_i <- b_i + gamma sign(mean(C^fb) - C_i^fb) over a feedback window of requested
    counts. The sign is taken exactly, as sign(sum_j C_j - N C_i); the bias is kept in
    float32, the precision the selection keys use, and an expert exactly at the mean is
    left untouched."""
    C = np.asarray(C_fb, dtype=np.int64)
    N = C.size
    sgn = np.sign(C.sum() - N * C)
    b = np.asarray(expert_bias, dtype=np.float32).copy()
    moved = sgn != 0
    b[moved] = b[moved] + np.float32(gamma) * sgn[moved].astype(np.float32)
    return b


def route_coefficients(z, idx, score: int, renorm: bool, alpha: float) -> np.ndarray:
    """r_{t,k} for the selected experts.

    * SOFTMAX: q = softmax over all N logits; with renorm p_i = q_i / sum_S q_j and
      r_i = alpha p_i (p1 Eq. 83 for alpha = K; p2 Appendix E), without renorm
      r_i = alpha q_i, whose routed mass m_K = sum_S q_i < 1 (p2 Qwen1.5/2, OLMoE rows).
    * SIGMOID: selected sigmoid affinities, renormalized and scaled by alpha
      (p2 Table 52, DeepSeek-V3 row, alpha = 2.5).
    * SOFTMAX_SELECTED: softmax over the selected logits only, times alpha
      (p2 Table 52, Mixtral row; p3 closing paragraph).
    """
    z = _f64(z)
    zS = np.take_along_axis(z, idx.astype(np.int64), axis=1)
    if score == SOFTMAX:
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        q = e / e.sum(axis=1, keepdims=True)
        qS = np.take_along_axis(q, idx.astype(np.int64), axis=1)
        p = qS / qS.sum(axis=1, keepdims=True) if renorm else qS
    elif score == SIGMOID:
        a = _sigmoid(zS)
        p = a / a.sum(axis=1, keepdims=True) if renorm else a
    elif score == SOFTMAX_SELECTED:
        m = zS.max(axis=1, keepdims=True)
        e = np.exp(zS - m)
        p = e / e.sum(axis=1, keepdims=True)
    else:
        raise ValueError(f"unknown score function {score}")
    return float(alpha) * p


# ----------------------------------------------------------------------------------------
# a3: requested and kept counts, capacity, offsets, restoration map
# ----------------------------------------------------------------------------------------
def requested_counts(idx, N: int) -> np.ndarray:
    """C_i^req = number of tokens whose selected set contains i (p5 Eq. 19)."""
    return np.bincount(np.asarray(idx).reshape(-1), minlength=N).astype(np.int64)


def capacity_from_factor(c: float, K: int, T: int, N: int) -> int:
    """Independent per-expert capacity ceil(c T_route / N_local) (p5 Eq. 25), with
    T_route = K T routes from the one source and N_local = N experts."""
    return int(math.ceil(float(c) * K * T / N))


def keep_routes(idx, N: int, capacity: int) -> np.ndarray:
    """Kept-route mask under per-expert first-come capacity: scanning tokens in index
    order, route (t, i) is admitted while fewer than `capacity` routes to expert i have
    been admitted (p5 Eq. 21 kept vs dropped; Eq. 25 per-expert limit). A negative
    capacity means unlimited (every requested route is kept)."""
    idx = np.asarray(idx)
    T, K = idx.shape
    kept = np.zeros((T, K), dtype=bool)
    used = np.zeros(N, dtype=np.int64)
    for t in range(T):
        for k in range(K):
            e = int(idx[t, k])
            if capacity < 0 or used[e] < capacity:
                kept[t, k] = True
                used[e] += 1
    return kept


# ----------------------------------------------------------------------------------------
# f2: rank-wide capacity (one budget shared by the experts of a destination group)
# ----------------------------------------------------------------------------------------
def rank_capacity_from_factor(c: float, K: int, T_s: int) -> int:
    """Destination-rank budget C_rank = max(1, ceil(c T_route)) with T_route = K T_s, the
    routes one source rank produces (p5 Eq. 23)."""
    return max(1, int(math.ceil(float(c) * K * T_s)))


def destination_of(N: int, group: int) -> np.ndarray:
    """rho(i): the destination that owns expert i when consecutive groups of `group`
    experts share a destination (p5 Eq. 20)."""
    if group <= 0 or N % group:
        raise ValueError("every destination owns the same number of experts")
    return np.arange(N) // group


def rank_loads(C, group: int) -> np.ndarray:
    """R_q = sum of the counts of the experts destination q owns (p5 Eq. 20 for requested
    counts, Eq. 21 for kept counts)."""
    C = np.asarray(C)
    rho = destination_of(len(C), group)
    return np.bincount(rho, weights=C, minlength=int(rho.max()) + 1).astype(np.int64)


def split_requested_counts(idx, N: int, n_sources: int) -> np.ndarray:
    """C_{s,i}^req (p5 Eq. 19) when the batch's tokens are split, in index order, into
    n_sources contiguous source shards (np.array_split sizes)."""
    idx = np.asarray(idx)
    shards = np.array_split(np.arange(idx.shape[0]), n_sources)
    return np.stack([requested_counts(idx[sh], N) for sh in shards])


def keep_routes_rank_wide(idx, N: int, group: int, budget: int, n_sources: int = 1) -> np.ndarray:
    """Kept-route mask under rank-wide capacity (p5 Section 10.3, Eq. 23): each
    destination q owns `group` consecutive experts and one shared budget. Its requested
    split counts are flattened local-expert-major, then source-rank order; routes are
    admitted cumulatively until the budget is reached, and inside each (source, expert)
    split the admitted routes are a prefix in token order. A negative budget keeps
    every route. Sources are the n_sources contiguous token shards."""
    idx = np.asarray(idx)
    T, K = idx.shape
    if budget < 0:
        return np.ones((T, K), dtype=bool)
    rho = destination_of(N, group)
    shards = np.array_split(np.arange(T), n_sources)
    C = split_requested_counts(idx, N, n_sources)           # [S, N]
    admit = np.zeros_like(C)                               # C_{s,i}^keep
    for q in range(int(rho.max()) + 1):
        room = budget
        for e in np.flatnonzero(rho == q):                 # local-expert-major
            for s in range(n_sources):                     # then source-rank order
                admit[s, e] = min(C[s, e], room)
                room -= admit[s, e]
    kept = np.zeros((T, K), dtype=bool)
    for s, sh in enumerate(shards):
        taken = np.zeros(N, dtype=np.int64)
        for t in sh:                                       # prefix of each split
            for k in range(K):
                e = int(idx[t, k])
                if taken[e] < admit[s, e]:
                    kept[t, k] = True
                    taken[e] += 1
    return kept


def drops_rank_wide(C_req, budget: int) -> int:
    """D^rank = [sum_j C_j^req - B]_+ for the local experts of one destination (p5 Eq. 28)."""
    return max(int(np.sum(C_req)) - int(budget), 0)


def drops_per_expert(C_req, budgets) -> int:
    """D^expert = sum_j [C_j^req - b_j]_+ under independent expert budgets (p5 Eq. 28)."""
    return int(sum(max(int(c) - int(b), 0) for c, b in zip(C_req, budgets)))


@dataclass
class Permutation:
    C_keep: np.ndarray        # [N]   M_i, rows presented to expert i (p5 Eq. 21)
    offsets: np.ndarray       # [N+1] o_0 = 0, o_{i+1} = o_i + M_i (p5 Eq. 26)
    dest_row: np.ndarray      # [T,K] packed row of each kept route, -1 when dropped
    row_token: np.ndarray     # [R]   source token of each packed row


def permutation(idx, kept, N: int) -> Permutation:
    """Pack kept routes into dense per-expert segments: expert i owns rows
    [o_i, o_{i+1}) with o given by the cumulative kept counts (p5 Eq. 26: the valid rows
    sit densely from row 0); inside a segment rows follow ascending token index.
    Dropped routes get no row and are left out of restoration and combine (p5 Section
    10.3)."""
    idx = np.asarray(idx)
    T, K = idx.shape
    C_keep = np.bincount(idx[kept].reshape(-1), minlength=N).astype(np.int64)
    offsets = np.zeros(N + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(C_keep)
    fill = offsets[:-1].copy()
    dest = np.full((T, K), -1, dtype=np.int64)
    row_token = np.zeros(int(offsets[-1]), dtype=np.int64)
    for t in range(T):
        for k in range(K):
            if kept[t, k]:
                e = int(idx[t, k])
                dest[t, k] = fill[e]
                row_token[fill[e]] = t
                fill[e] += 1
    return Permutation(C_keep, offsets, dest, row_token)


# ----------------------------------------------------------------------------------------
# f1: router balance statistics and drop diagnostics (forward values, no gradients)
# ----------------------------------------------------------------------------------------
def normalized_scores(z, score: int) -> np.ndarray:
    """p_{t,i}: each token's router scores normalized across all N experts (p5 Eq. 38).
    Softmax routing: the full softmax of the (biased) logits, whatever the combine rule;
    sigmoid routing: the affinities divided by their sum over the experts (p5 Section
    10.7, the scores of the balance loss are normalized across experts)."""
    z = _f64(z)
    if score == SIGMOID:
        a = _sigmoid(z)
        return a / a.sum(axis=1, keepdims=True)
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def imbalance_max(x) -> float:
    """Max/mean imbalance n * max_j x_j / sum_j x_j of a load vector (p5 Eq. 22, Eq. 39);
    NaN for an all-zero vector."""
    x = _f64(x)
    tot = x.sum()
    return float(x.size * x.max() / tot) if tot > 0 else float("nan")


def entropy_deficit(x) -> float:
    """Normalized entropy deficit 1 - H(pi) / log n of the load distribution
    pi = x / sum x, with 0 log 0 = 0 (p5 Section 10.2); NaN for an all-zero vector."""
    x = _f64(x)
    tot = x.sum()
    if tot <= 0:
        return float("nan")
    if x.size == 1:
        return 0.0      # a single expert carries the whole load: balanced, log n = 0
    pi = x / tot
    nz = pi[pi > 0]
    H = float(-(nz * np.log(nz)).sum())
    return 1.0 - H / math.log(x.size)


def coefficient_of_variation(x) -> float:
    """Standard deviation over mean of the counts (population form; p5 Section 10.2)."""
    x = _f64(x)
    m = x.mean()
    return float(x.std() / m) if m > 0 else float("nan")


@dataclass
class BalanceStats:
    f: np.ndarray                 # [N] requested-route fractions C_req / (K T)
    P: np.ndarray                 # [N] mean normalized router scores
    lbl: float                    # N f . P (p5 Eq. 30)
    imax_req: float               # Eq. 39 on requested counts
    imax_keep: float              # Eq. 22 on kept counts
    ih_req: float                 # entropy deficit of requested counts
    ih_keep: float                # entropy deficit of kept counts
    cv_req: float
    cv_keep: float
    never_selected: int           # experts with no requested route
    delta_route: float            # dropped / requested routes (p5 Eq. 27)
    tokens_lost_any: int          # tokens with at least one dropped route
    tokens_lost_all: int          # tokens whose K routes were all dropped
    weight_removed: float         # dropped share of the selected coefficient mass
    imax_rank_req: float = float("nan")    # Eq. 22 on requested destination totals (Eq. 20)
    imax_rank_keep: float = float("nan")   # Eq. 22 on kept destination totals (Eq. 21)


def balance_stats(p, idx, kept, r, N: int, group: int = 0) -> BalanceStats:
    """Forward balance and drop statistics of one routed batch: the hard and soft
    marginals f and P and the Switch-style scalar N f.P (p5 Eq. 38, 30); requested and
    kept max/mean imbalance, entropy deficit, coefficient of variation and never-selected
    count (p5 Eq. 22, 39, Section 10.2); the route-drop fraction (Eq. 27) and, as Section
    10.3 asks, the tokens losing at least one and all K routes and the selected mixture
    weight removed. `p` are the normalized scores, `kept` the kept-route mask and `r` the
    routed coefficients of the selected slots. With `group` > 0, consecutive groups of
    that many experts form the destinations, and the max/mean imbalance of their
    requested and kept totals is the rank-level pair of p5 Eq. 22 (Table 17)."""
    p = _f64(p)
    idx = np.asarray(idx)
    kept = np.asarray(kept, dtype=bool)
    r = _f64(r)
    T, K = idx.shape
    C_req = requested_counts(idx, N)
    C_keep = np.bincount(idx[kept].reshape(-1), minlength=N).astype(np.int64)
    f = C_req / float(K * T)
    P = p.mean(axis=0)
    lbl = float(N * f @ P)
    dropped = ~kept
    n_drop = dropped.sum(axis=1)
    sel = r.sum()
    return BalanceStats(
        f=f, P=P, lbl=lbl,
        imax_req=imbalance_max(C_req), imax_keep=imbalance_max(C_keep),
        ih_req=entropy_deficit(C_req), ih_keep=entropy_deficit(C_keep),
        cv_req=coefficient_of_variation(C_req), cv_keep=coefficient_of_variation(C_keep),
        never_selected=int((C_req == 0).sum()),
        delta_route=float(dropped.sum() / float(K * T)),
        tokens_lost_any=int((n_drop > 0).sum()),
        tokens_lost_all=int((n_drop == K).sum()),
        weight_removed=float(r[dropped].sum() / sel) if sel > 0 else float("nan"),
        imax_rank_req=imbalance_max(rank_loads(C_req, group)) if group > 0 else float("nan"),
        imax_rank_keep=imbalance_max(rank_loads(C_keep, group)) if group > 0 else float("nan"),
    )


# ----------------------------------------------------------------------------------------
# a5-a7: SwiGLU experts
# ----------------------------------------------------------------------------------------
def swiglu(X, w_gate, w_up, w_down):
    """E(X) = [SiLU(X W_g) * (X W_u)] W_d (p4 Eq. 74), with stored-transposed weights.
    Returns (H, F): the intermediate activation [M, d_ff] and the output [M, d_model]."""
    X = _f64(X)
    H = silu(X @ _f64(w_gate).T) * (X @ _f64(w_up).T)
    return H, H @ _f64(w_down).T


def shared_output(x, shared_experts: Sequence) -> Optional[np.ndarray]:
    """g(x) = sum_j E_j(x) over the ungated shared experts, each evaluated on its own
    (p4 Eq. 76 left-hand side). Returns None when there is no shared expert."""
    if not shared_experts:
        return None
    g = None
    for (wg, wu, wd) in shared_experts:
        _, Fj = swiglu(x, wg, wu, wd)
        g = Fj if g is None else g + Fj
    return g


# ----------------------------------------------------------------------------------------
# f4: backward of the layer with the routing coefficients held fixed
# ----------------------------------------------------------------------------------------
def swiglu_backward(X, w_gate, w_up, w_down, dF):
    """Chain rule through E(X) = [SiLU(X W_g) * (X W_u)] W_d (p4 Eq. 74) for an upstream
    gradient dF of its output: with A = X W_g, B = X W_u, S = SiLU(A), H = S * B,
      dH = dF W_d^T,  dB = dH * S,  dA = dH * B * SiLU'(A),  SiLU'(a) = s(a)(1 + a(1 - s(a))),
      dX = dA W_g^T + dB W_u^T,  dW_g = X^T dA,  dW_u = X^T dB,  dW_d = H^T dF,
    returned in the stored-transposed layouts of the weights: (dX, dw_gate [d_ff, d_model],
    dw_up [d_ff, d_model], dw_down [d_model, d_ff])."""
    X, dF = _f64(X), _f64(dF)
    Wg, Wu, Wd = _f64(w_gate), _f64(w_up), _f64(w_down)
    A = X @ Wg.T
    B = X @ Wu.T
    sg = _sigmoid(A)
    S = A * sg
    H = S * B
    dH = dF @ Wd
    dB = dH * S
    dA = dH * B * sg * (1.0 + A * (1.0 - sg))
    dX = dA @ Wg + dB @ Wu
    return dX, dA.T @ X, dB.T @ X, dF.T @ H


@dataclass
class Gradients:
    dx: np.ndarray                # [T, d_model]
    dw_gate: np.ndarray           # [N, d_r, d_model]
    dw_up: np.ndarray             # [N, d_r, d_model]
    dw_down: np.ndarray           # [N, d_model, d_r]
    shared: list                  # per shared expert: (dw_gate, dw_up, dw_down)


def backward(x, idx, kept, r, expert_weights: Callable[[int], tuple], N: int, dy,
             shared_experts: Sequence = (), s=1.0) -> Gradients:
    """Gradients of the layer output y (p1 Eq. 80) for an upstream gradient dy, with the
    router held fixed: the selected experts, the kept routes, the coefficients r and the
    shared gain s (scalar or per-token gate) are constants (the fixed-router input
    gradient of p1 Section 21.3). Expert i's output row of kept route (t, i) receives
    r_{t,i} dy_t; each expert's rows are back-propagated through Eq. 74; the input
    gradient of token t sums its kept routes' rows and the shared branch, which receives
    s_t dy_t. Experts without kept rows get zero weight gradients."""
    x, dy = _f64(x), _f64(dy)
    idx = np.asarray(idx)
    kept = np.asarray(kept, dtype=bool)
    r = _f64(r)
    T, K = idx.shape
    dx = np.zeros_like(x)
    dwg = dwu = dwd = None
    for e in range(N):
        wg, wu, wd = expert_weights(e)
        if dwg is None:
            dwg = np.zeros((N,) + np.shape(wg))
            dwu = np.zeros((N,) + np.shape(wu))
            dwd = np.zeros((N,) + np.shape(wd))
        toks, slots = np.nonzero((idx == e) & kept)      # ascending token order
        if toks.size == 0:
            continue
        dF = r[toks, slots, None] * dy[toks]
        dX, dwg[e], dwu[e], dwd[e] = swiglu_backward(x[toks], wg, wu, wd, dF)
        np.add.at(dx, toks, dX)
    gain = np.broadcast_to(_f64(s), (T,))[:, None]
    shared = []
    for (wg, wu, wd) in shared_experts:
        dX, g1, g2, g3 = swiglu_backward(x, wg, wu, wd, gain * dy)
        dx += dX
        shared.append((g1, g2, g3))
    return Gradients(dx, dwg, dwu, dwd, shared)


# ----------------------------------------------------------------------------------------
# a8: combine
# ----------------------------------------------------------------------------------------
def combine(F_perm, dest_row, r, G=None, s=1.0) -> np.ndarray:
    """y_t = sum_{i in S_t, kept} r_{t,i} f_i(x_t) + s_t g(x_t) (p1 Eq. 80), reading each
    expert output from its packed row. Dropped routes contribute nothing and the kept
    coefficients are not renormalized (p5 Section 10.3: routes that capacity dropped
    are left out of restoration and combine). `s` is a scalar gain or a per-token gate vector."""
    dest_row = np.asarray(dest_row)
    T, K = dest_row.shape
    F_perm = _f64(F_perm)
    d = F_perm.shape[1] if F_perm.ndim == 2 and F_perm.shape[0] else (
        G.shape[1] if G is not None else 0)
    y = np.zeros((T, d))
    r = _f64(r)
    for k in range(K):
        m = dest_row[:, k] >= 0
        if m.any():
            y[m] += r[m, k, None] * F_perm[dest_row[m, k]]
    if G is not None:
        s_arr = _f64(s)
        y += (s_arr[:, None] if s_arr.ndim == 1 else s_arr) * _f64(G)
    return y


# ----------------------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------------------
@dataclass
class LayerSpec:
    """Arguments of one MoE layer, in the pages' notation."""
    N: int
    K: int
    score: int = SOFTMAX
    renorm: bool = True
    alpha: float = 1.0
    s: float = 1.0                    # fixed shared gain when there is no learned gate
    capacity: int = -1                # routes kept per expert (or per destination); < 0 = unlimited
    capacity_group: int = 0           # > 0: destinations of this many experts share `capacity`
    expert_bias: Optional[np.ndarray] = None   # [N] selection-only bias b (p5 Eq. 35)


@dataclass
class Result:
    logits: np.ndarray
    idx: np.ndarray
    r: np.ndarray
    s_tok: Optional[np.ndarray]
    C_req: np.ndarray
    kept: np.ndarray
    perm: Permutation
    H_perm: np.ndarray
    F_perm: np.ndarray
    G: Optional[np.ndarray]
    y: np.ndarray


def forward(spec: LayerSpec, x, w_router, expert_weights: Callable[[int], tuple],
            shared_experts: Sequence = (), logit_bias=None, w_shared_gate=None,
            logits_override=None, selection_override=None) -> Result:
    """The whole layer forward, stage by stage (p5 Section 10 opening paragraph:
    router -> capacity -> dispatch -> grouped expert compute -> combine; p1 Eq. 80).

    `expert_weights(i)` returns (w_gate, w_up, w_down) of routed expert i.
    `logits_override` (e.g. float32 logits) replaces the computed logits for selection
    and coefficients, so that near-ties are decided on identical values.
    `selection_override` ([T, K] expert indices) replaces the top-K selection, for the
    cases where several selections are correct within rounding (the caller checks that
    the one it passes is among them)."""
    x = _f64(x)
    T = x.shape[0]
    z = router_logits(x, w_router, logit_bias)
    zz = z if logits_override is None else np.asarray(logits_override)
    if selection_override is None:
        idx = topk_select(selection_keys(zz, spec.score, spec.expert_bias), spec.K)
    else:
        idx = np.asarray(selection_override).astype(np.int32)
    r = route_coefficients(zz, idx, spec.score, spec.renorm, spec.alpha)
    s_tok = shared_gate(x, w_shared_gate) if w_shared_gate is not None else None
    C_req = requested_counts(idx, spec.N)
    if spec.capacity_group > 0:
        kept = keep_routes_rank_wide(idx, spec.N, spec.capacity_group, spec.capacity,
                                     n_sources=spec.N // spec.capacity_group)
    else:
        kept = keep_routes(idx, spec.N, spec.capacity)
    perm = permutation(idx, kept, spec.N)
    R = int(perm.offsets[-1])
    d = x.shape[1]
    x_perm = x[perm.row_token] if R else np.zeros((0, d))
    H_perm = None
    F_perm = np.zeros((R, d))
    for i in range(spec.N):
        a, b = int(perm.offsets[i]), int(perm.offsets[i + 1])
        if b > a:
            wg, wu, wd = expert_weights(i)
            Hi, Fi = swiglu(x_perm[a:b], wg, wu, wd)
            if H_perm is None:
                H_perm = np.zeros((R, Hi.shape[1]))
            H_perm[a:b] = Hi
            F_perm[a:b] = Fi
    if H_perm is None:
        H_perm = np.zeros((R, 0))
    G = shared_output(x, shared_experts)
    gain = s_tok if s_tok is not None else spec.s
    y = combine(F_perm, perm.dest_row, r, G, gain)
    return Result(z, idx, r, s_tok, C_req, kept, perm, H_perm, F_perm, G, y)


def forward_tokens(spec: LayerSpec, tokens, x, idx, r, kept_or_dest, expert_weights,
                   shared_experts: Sequence = (), s_tok=None) -> np.ndarray:
    """y for a subset of tokens, given each token's routing (selected experts, their
    coefficients and which routes were kept): p1 Eq. 80 evaluated directly, with
    f_i(x) = E_i(x) of p4 Eq. 74, for sampled checks at sizes where the whole layer is
    too slow on the CPU. Each touched expert's weights are fetched once."""
    x = _f64(x)
    kept = np.asarray(kept_or_dest)
    if kept.dtype != bool:
        kept = kept >= 0
    tokens = list(tokens)
    y = np.zeros((len(tokens), x.shape[1]))
    uses = {}
    for j, t in enumerate(tokens):
        for k in range(idx.shape[1]):
            if kept[t, k]:
                uses.setdefault(int(idx[t, k]), []).append((j, t, k))
    for e in sorted(uses):
        wg, wu, wd = expert_weights(e)
        rows = [t for (_, t, _) in uses[e]]
        _, Fe = swiglu(x[rows], wg, wu, wd)
        for n, (j, t, k) in enumerate(uses[e]):
            y[j] += float(r[t, k]) * Fe[n]
    g = shared_output(x[tokens], shared_experts) if tokens else None
    if g is not None:
        gain = np.asarray(s_tok, np.float64)[tokens] if s_tok is not None else spec.s
        y += (gain[:, None] if np.ndim(gain) else gain) * g
    return y
