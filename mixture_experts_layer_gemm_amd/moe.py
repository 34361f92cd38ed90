"""Thin ctypes binding of the C ABI in include/moe.h.

Argument marshalling only: every stage of the layer runs in the HIP kernels of
libmoe_mi355x.so. PyTorch supplies device memory (tensors, workspaces) and the stream
(torch's current stream). Importing this module fails loudly when the library has not
been built; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, c_double, c_float, c_int, c_size_t, c_void_p
from typing import Optional, Sequence

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16 = 0, 1
SCORE_SOFTMAX, SCORE_SIGMOID, SCORE_SOFTMAX_SELECTED = 0, 1, 2


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")
        self.status = status


class ForwardArgs(ctypes.Structure):
    """Mirror of moe_forward_args."""
    _fields_ = [(n, c_int) for n in ("T", "d_model", "N", "K", "d_r", "d_s", "score", "renorm")] + [
        ("alpha", c_float), ("s", c_float), ("capacity", c_int), ("capacity_group", c_int),
        ("dt", c_int),
        ("weights_packed", c_int)] + [
        (n, c_void_p) for n in ("x", "w_router", "logit_bias", "expert_bias", "w_shared_gate",
                                "w_gate", "w_up",
                                "w_down", "ws_gate", "ws_up", "ws_down", "y", "logits", "topk_idx",
                                "topk_r", "s_tok", "C_req", "C_keep", "offsets", "dest_row",
                                "row_token", "x_perm", "h_perm", "f_perm", "g", "balance_P",
                                "balance_stats", "count_accum")]

class BackwardArgs(ctypes.Structure):
    """Mirror of moe_backward_args (include/moe.h)."""
    _fields_ = [(n, c_int) for n in ("T", "d_model", "N", "K", "d_r", "d_s", "dt")] + [
        ("s", c_float), ("max_rows", c_int)] + [
        (n, c_void_p) for n in ("x", "dy", "row_token", "offsets", "dest_row", "topk_r", "s_tok",
                                "w_gate", "w_up", "wt_down", "wt_gate_up", "ws_gate", "ws_up",
                                "wst_down", "wst_gate_up", "dx", "dw_gate", "dw_up", "dw_down",
                                "dws_gate", "dws_up", "dws_down")]


# order of moe_balance_stats' output vector (enum moe_stat)
STAT_NAMES = ["lbl", "imax_req", "imax_keep", "ih_req", "ih_keep", "cv_req", "cv_keep",
              "never_selected", "delta_route", "tokens_lost_any", "tokens_lost_all",
              "weight_removed", "imax_rank_req", "imax_rank_keep"]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"HIP library {LIB_PATH} is not built; run "
                          "`python -m mixture_experts_layer_gemm_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    I, F, P, S = c_int, c_float, c_void_p, c_size_t
    sig = {
        "moe_status_string": (ctypes.c_char_p, [I]),
        "moe_capacity_from_factor": (I, [c_double, I, I, I]),
        "moe_rank_capacity_from_factor": (I, [c_double, I, I]),
        "moe_max_rows": (I, [I, I, I, I, I]),
        "moe_route_workspace_size": (S, [I, I, I, I]),
        "moe_route": (I, [I, I, I, I, I, I, F, I, P, P, P, P, P, P, I, P, P, P, P, P, S, P]),
        "moe_bias_update": (I, [I, F, P, P, I, P]),
        "moe_pack_weights_transposed": (I, [I, I, I, I, I, P, P, P, P]),
        "moe_backward_workspace_size": (S, [P]),
        "moe_backward": (I, [P, P, S, P]),
        "moe_permute_workspace_size": (S, [I, I, I]),
        "moe_permute": (I, [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, I, P, S, P]),
        "moe_permute_noalloc": (I, [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, I, P]),
        "moe_grouped_swiglu": (I, [I, I, I, I, I, P, I, P, P, I, P, P, P, P, P, P]),
        "moe_grouped_gemm": (I, [I, I, I, I, I, I, P, I, P, P, I, P, P, P, P]),
        "moe_pack_weights": (I, [I, I, I, I, P, P, P]),
        "moe_combine": (I, [I, I, I, I, P, P, P, P, F, P, P, P]),
        "moe_experts": (I, [I, I, I, I, I, I, P, I, P, P, I, P, P, P, P, P, P, P, P, P, P, I, P]),
        "moe_balance_stats_workspace_size": (S, [I, I]),
        "moe_balance_stats": (I, [I, I, I, I, I, P, P, P, P, P, P, P, P, S, P]),
        "moe_forward_workspace_size": (S, [POINTER(ForwardArgs)]),
        "moe_forward": (I, [POINTER(ForwardArgs), P, S, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def declared_symbols(header: str = HEADER) -> list:
    """Names of the functions declared in include/moe.h."""
    with open(header) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return lib.moe_status_string(status).decode()


def capacity_from_factor(c: float, K: int, T: int, N: int) -> int:
    return lib.moe_capacity_from_factor(float(c), K, T, N)


def rank_capacity_from_factor(c: float, K: int, T_s: int) -> int:
    return lib.moe_rank_capacity_from_factor(float(c), K, T_s)


def max_rows(T: int, N: int, K: int, capacity: int, capacity_group: int = 0) -> int:
    return lib.moe_max_rows(T, N, K, capacity, capacity_group)


# ---------------------------------------------------------------------------------------
def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _check(fn: str, st: int):
    if st != MOE_OK:
        raise MoEError(fn, st)


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def moe_route(x, w_router, K: int, score: int = SCORE_SOFTMAX, renorm: bool = True,
              alpha: float = 1.0, logit_bias=None, w_shared_gate=None, logits=None,
              logits_mode: int = 0, want_logits: bool = False, want_counts: bool = True,
              expert_bias=None):
    """Router stage. Returns dict(topk_idx, topk_r, s_tok, C_req, logits). expert_bias is
    the selection-only bias of auxiliary-loss-free balancing."""
    if logits_mode == 1:
        T, N = logits.shape
        dev, d, dt = logits.device, 64, MOE_F32
    else:
        T, d = x.shape
        N = w_router.shape[0]
        dev, dt = x.device, _dt(x)
        if want_logits and logits is None:
            logits = torch.empty(T, N, dtype=torch.float32, device=dev)
    out = dict(topk_idx=torch.empty(T, K, dtype=torch.int32, device=dev),
               topk_r=torch.empty(T, K, dtype=torch.float32, device=dev),
               s_tok=(torch.empty(T, dtype=torch.float32, device=dev)
                      if (w_shared_gate is not None and logits_mode == 0) else None),
               C_req=torch.empty(N, dtype=torch.int32, device=dev) if want_counts else None,
               logits=logits)
    ws = _workspace(lib.moe_route_workspace_size(T, d, N, K), dev)
    st = lib.moe_route(T, d, N, K, score, int(renorm), float(alpha), dt,
                       None if logits_mode == 1 else _ptr(x),
                       None if logits_mode == 1 else _ptr(w_router),
                       None if logits_mode == 1 else _ptr(logit_bias), _ptr(expert_bias),
                       None if logits_mode == 1 else _ptr(w_shared_gate),
                       _ptr(logits), logits_mode, _ptr(out["topk_idx"]), _ptr(out["topk_r"]),
                       _ptr(out["s_tok"]), _ptr(out["C_req"]), _ptr(ws), ws.numel(), _stream())
    _check("moe_route", st)
    return out


def moe_bias_update(count_accum, expert_bias, gamma: float, reset: bool = True):
    """b_i += gamma sign(mean(C) - C_i) in place over the accumulated requested counts;
    the accumulator is zeroed when reset."""
    st = lib.moe_bias_update(expert_bias.numel(), float(gamma), _ptr(count_accum),
                             _ptr(expert_bias), int(reset), _stream())
    _check("moe_bias_update", st)


def moe_permute(x, topk_idx, N: int, capacity: int = -1, copy_rows: bool = True,
                capacity_group: int = 0):
    """Counts, capacity admission, offsets, restoration map and (copy_rows) the packed
    rows x_perm; without copy_rows the grouped GEMM gathers rows through row_token.
    capacity_group = g > 0 shares one budget `capacity` among each g consecutive experts."""
    T, d = x.shape
    K = topk_idx.shape[1]
    dev = x.device
    rows = max_rows(T, N, K, capacity, capacity_group)
    out = dict(C_req=torch.empty(N, dtype=torch.int32, device=dev),
               C_keep=torch.empty(N, dtype=torch.int32, device=dev),
               offsets=torch.empty(N + 1, dtype=torch.int32, device=dev),
               dest_row=torch.empty(T, K, dtype=torch.int32, device=dev),
               row_token=torch.empty(max(rows, 1), dtype=torch.int32, device=dev),
               x_perm=(torch.empty(max(rows, 1), d, dtype=x.dtype, device=dev)
                       if copy_rows else None))
    ws = _workspace(lib.moe_permute_workspace_size(T, N, K), dev)
    st = lib.moe_permute(T, d, N, K, capacity, capacity_group, _dt(x), _ptr(x), _ptr(topk_idx),
                         _ptr(out["C_req"]), _ptr(out["C_keep"]), _ptr(out["offsets"]),
                         _ptr(out["dest_row"]), _ptr(out["row_token"]), _ptr(out["x_perm"]),
                         max(rows, 1), _ptr(ws), ws.numel(), _stream())
    _check("moe_permute", st)
    return out


def moe_permute_noalloc(x, topk_idx, N: int, capacity: int = -1, copy_rows: bool = True,
                        capacity_group: int = 0, out=None):
    """moe_permute with its scratch in the library's fixed device array (no workspace).
    `out` (a dict as moe_permute returns) supplies the output buffers; the library
    itself allocates nothing."""
    T, d = x.shape
    K = topk_idx.shape[1]
    dev = x.device
    rows = max_rows(T, N, K, capacity, capacity_group)
    if out is None:
        out = dict(C_req=torch.empty(N, dtype=torch.int32, device=dev),
                   C_keep=torch.empty(N, dtype=torch.int32, device=dev),
                   offsets=torch.empty(N + 1, dtype=torch.int32, device=dev),
                   dest_row=torch.empty(T, K, dtype=torch.int32, device=dev),
                   row_token=torch.empty(max(rows, 1), dtype=torch.int32, device=dev),
                   x_perm=(torch.empty(max(rows, 1), d, dtype=x.dtype, device=dev)
                           if copy_rows else None))
    st = lib.moe_permute_noalloc(T, d, N, K, capacity, capacity_group, _dt(x), _ptr(x),
                                 _ptr(topk_idx), _ptr(out["C_req"]), _ptr(out["C_keep"]),
                                 _ptr(out["offsets"]), _ptr(out["dest_row"]),
                                 _ptr(out["row_token"]), _ptr(out.get("x_perm")),
                                 out["row_token"].numel(), _stream())
    _check("moe_permute_noalloc", st)
    return out


def moe_pack_weights(w):
    """[G][N][K] bf16 weights -> the MFMA-operand layout of moe_pack_weights (same shape
    and dtype; only the element order differs). A one-time weight-load step."""
    G, N, K = w.shape
    p = torch.empty_like(w)
    st = lib.moe_pack_weights(G, N, K, _dt(w), _ptr(w), _ptr(p), _stream())
    _check("moe_pack_weights", st)
    return p


def _rows(a, row_index):
    return a.shape[0] if row_index is None else row_index.shape[0]


def moe_grouped_swiglu(a, offsets, w_gate, w_up, w_down, h=None, out=None, packed=False,
                       row_index=None):
    """Grouped SwiGLU over packed segments (offsets=None: one group over all rows).
    With row_index, packed row r reads a[row_index[r]]."""
    rows, d = _rows(a, row_index), a.shape[1]
    G, d_ff, _ = w_gate.shape
    h = torch.empty(rows, d_ff, dtype=a.dtype, device=a.device) if h is None else h
    out = torch.empty(rows, d, dtype=a.dtype, device=a.device) if out is None else out
    st = lib.moe_grouped_swiglu(G, d, d_ff, _dt(a), int(packed), _ptr(a), a.shape[0],
                                _ptr(row_index), _ptr(offsets), rows,
                                _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(h), _ptr(out),
                                _stream())
    _check("moe_grouped_swiglu", st)
    return h, out


def moe_grouped_gemm(a, offsets, w0, w1=None, out=None, swiglu: bool = True, packed=False,
                     row_index=None):
    """One grouped GEMM pass: SwiGLU(gate, up) when swiglu, else a plain projection."""
    rows, Kd = _rows(a, row_index), a.shape[1]
    G, Nd, _ = w0.shape
    out = torch.empty(rows, Nd, dtype=a.dtype, device=a.device) if out is None else out
    st = lib.moe_grouped_gemm(G, Kd, Nd, _dt(a), int(swiglu), int(packed), _ptr(a), a.shape[0],
                              _ptr(row_index), _ptr(offsets), rows, _ptr(w0), _ptr(w1), _ptr(out), _stream())
    _check("moe_grouped_gemm", st)
    return out


def moe_experts(x, row_token, offsets, max_rows: int, w_gate, w_up, w_down, shared=None,
                out=None, packed=False, pass_: int = 0):
    """The expert stage as moe_forward runs it: routed experts over their segments (rows
    gathered from x through row_token) and the shared MLP `shared` = (ws_gate, ws_up,
    ws_down) or None. Returns dict(h_perm, f_perm, h_shared, g); pass_ 1 = gate/up only,
    2 = down only (reusing the h buffers of `out`), 0 = both."""
    T, d = x.shape
    N, d_r, _ = w_gate.shape
    d_s = 0 if shared is None else shared[0].shape[0]
    dev, dt = x.device, x.dtype
    if out is None:
        rows = max(max_rows, 1)
        out = dict(h_perm=torch.empty(rows, d_r, dtype=dt, device=dev),
                   f_perm=torch.empty(rows, d, dtype=dt, device=dev),
                   h_shared=torch.empty(T, d_s, dtype=dt, device=dev) if d_s else None,
                   g=torch.empty(T, d, dtype=dt, device=dev) if d_s else None)
    ws = (None, None, None) if shared is None else shared
    st = lib.moe_experts(N, d, d_r, d_s, _dt(x), int(packed), _ptr(x), T, _ptr(row_token),
                         _ptr(offsets), max_rows, _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                         _ptr(ws[0]), _ptr(ws[1]), _ptr(ws[2]), _ptr(out["h_perm"]),
                         _ptr(out["f_perm"]), _ptr(out["h_shared"]), _ptr(out["g"]), pass_,
                         _stream())
    _check("moe_experts", st)
    return out


def moe_balance_stats(logits, C_req, C_keep, dest_row, topk_r, score: int = SCORE_SOFTMAX,
                      expert_group: int = 0):
    """Balance statistics and drop diagnostics of one routed batch: returns (P, stats)
    with P the [N] mean normalized scores and stats a dict keyed by STAT_NAMES (device
    tensors; read them after the stream synchronizes)."""
    T, N = logits.shape
    K = dest_row.shape[1]
    dev = logits.device
    P = torch.empty(N, dtype=torch.float32, device=dev)
    st = torch.empty(len(STAT_NAMES), dtype=torch.float32, device=dev)
    ws = _workspace(lib.moe_balance_stats_workspace_size(T, N), dev)
    rc = lib.moe_balance_stats(T, N, K, score, expert_group, _ptr(logits), _ptr(C_req),
                               _ptr(C_keep),
                               _ptr(dest_row), _ptr(topk_r), _ptr(P), _ptr(st), _ptr(ws),
                               ws.numel(), _stream())
    _check("moe_balance_stats", rc)
    return P, st


def stats_dict(st: torch.Tensor) -> dict:
    v = st.cpu().tolist()
    return dict(zip(STAT_NAMES, v))


def moe_combine(f_perm, dest_row, topk_r, g=None, s: float = 1.0, s_tok=None, y=None):
    T, K = dest_row.shape
    d = f_perm.shape[1]
    y = torch.empty(T, d, dtype=f_perm.dtype, device=f_perm.device) if y is None else y
    st = lib.moe_combine(T, d, K, _dt(f_perm), _ptr(f_perm), _ptr(dest_row), _ptr(topk_r),
                         _ptr(g), float(s), _ptr(s_tok), _ptr(y), _stream())
    _check("moe_combine", st)
    return y


def moe_pack_weights_transposed(w_a, w_b=None):
    """[G][Ka][N] (stacked over [G][Kb][N] when w_b is given) bf16 -> the packed transpose
    [G][N][Ka + Kb], the operand of the backward's data-gradient contractions."""
    G, Ka, Nn = w_a.shape
    Kk = Ka + (0 if w_b is None else w_b.shape[1])
    dst = torch.empty(G, Nn, Kk, dtype=w_a.dtype, device=w_a.device)
    st = lib.moe_pack_weights_transposed(G, Nn, Kk, Ka, _dt(w_a), _ptr(w_a.contiguous()),
                                         _ptr(None if w_b is None else w_b.contiguous()),
                                         _ptr(dst), _stream())
    _check("moe_pack_weights_transposed", st)
    return dst


def backward_weights(w_gate, w_up, w_down):
    """Packed transposes used by moe_backward: w_down^T [N][d_r][d] and [w_gate; w_up]^T
    [N][d][2 d_r] (row-major bf16 inputs, as in a Linear layer)."""
    return moe_pack_weights_transposed(w_down), moe_pack_weights_transposed(w_gate, w_up)


def moe_backward(x, dy, routing: dict, max_rows: int, w_gate, w_up, wt_down, wt_gate_up,
                 shared=None, s: float = 1.0):
    """Fixed-router gradients of the layer for upstream dy. `routing` holds the forward's
    row_token, offsets, dest_row, topk_r (and s_tok when the shared gate is learned);
    w_gate/w_up are packed, wt_* the packed transposes (backward_weights); `shared` is
    (ws_gate, ws_up, wst_down, wst_gate_up) of the one shared MLP (packed), or None.
    Returns dict(dx, dw_gate, dw_up, dw_down, dws_gate, dws_up, dws_down)."""
    T, d = x.shape
    N, d_r, _ = w_gate.shape
    K = routing["dest_row"].shape[1]
    dev = x.device
    d_s = 0 if shared is None else shared[0].shape[0]
    f32 = torch.float32
    out = dict(dx=torch.empty_like(x), dw_gate=torch.empty(N, d_r, d, dtype=f32, device=dev),
               dw_up=torch.empty(N, d_r, d, dtype=f32, device=dev),
               dw_down=torch.empty(N, d, d_r, dtype=f32, device=dev),
               dws_gate=torch.empty(d_s, d, dtype=f32, device=dev) if d_s else None,
               dws_up=torch.empty(d_s, d, dtype=f32, device=dev) if d_s else None,
               dws_down=torch.empty(d, d_s, dtype=f32, device=dev) if d_s else None)
    a = BackwardArgs()
    a.T, a.d_model, a.N, a.K, a.d_r, a.d_s, a.dt = T, d, N, K, d_r, d_s, _dt(x)
    a.s, a.max_rows = float(s), int(max_rows)
    a.x, a.dy = _ptr(x), _ptr(dy)
    for name in ("row_token", "offsets", "dest_row", "topk_r", "s_tok"):
        setattr(a, name, _ptr(routing.get(name)))
    a.w_gate, a.w_up, a.wt_down, a.wt_gate_up = (_ptr(w) for w in (w_gate, w_up, wt_down, wt_gate_up))
    if shared is not None:
        a.ws_gate, a.ws_up, a.wst_down, a.wst_gate_up = (_ptr(w) for w in shared)
    for name in ("dx", "dw_gate", "dw_up", "dw_down", "dws_gate", "dws_up", "dws_down"):
        setattr(a, name, _ptr(out[name]))
    ws = _workspace(lib.moe_backward_workspace_size(ctypes.byref(a)), dev)
    st = lib.moe_backward(ctypes.byref(a), _ptr(ws), ws.numel(), _stream())
    _check("moe_backward", st)
    out["_workspace"] = ws          # kept alive until the caller synchronizes
    return out


def pack_shared(shared: Sequence) -> tuple:
    """Several ungated shared experts -> one MLP: gate/up rows concatenated, down columns
    concatenated (Section 20, Eq. 75). A weight-layout step, done once at load time."""
    if not shared:
        return None
    if len(shared) == 1:
        return tuple(w.contiguous() for w in shared[0])
    return (torch.cat([s[0] for s in shared], 0).contiguous(),
            torch.cat([s[1] for s in shared], 0).contiguous(),
            torch.cat([s[2] for s in shared], 1).contiguous())


class MoELayer:
    """Device-resident weights, preallocated outputs and workspace for repeated
    moe_forward calls on torch's current stream."""

    def __init__(self, x, w_router, w_gate, w_up, w_down, K: int, score: int = SCORE_SOFTMAX,
                 renorm: bool = True, alpha: float = 1.0, s: float = 1.0, capacity: int = -1,
                 capacity_group: int = 0, logit_bias=None, w_shared_gate=None, shared=None, keep_intermediates=False,
                 pack_weights=None, keep_x_perm=False, balance_stats=False, expert_bias=None,
                 count_accum=None, trainable=False):
        self.x = x
        T, d = x.shape
        N, d_r, _ = w_gate.shape
        dev = x.device
        shared_mlp = pack_shared(shared) if shared else None
        if pack_weights is None:                      # the fast path whenever it applies
            pack_weights = x.dtype == torch.bfloat16
        self.weights_packed = bool(pack_weights)
        self.bwd = None
        if trainable:           # fixed-router backward: packed transposes, routing kept
            if x.dtype != torch.bfloat16:
                raise MoEError("moe_backward", MOE_ERR_UNSUPPORTED)
            pack_weights, keep_intermediates = True, True
            bwd = dict(zip(("wt_down", "wt_gate_up"), backward_weights(w_gate, w_up, w_down)))
            if shared_mlp:
                sg, su, sd = shared_mlp
                bwd["shared_t"] = (moe_pack_weights_transposed(sd[None])[0],
                                   moe_pack_weights_transposed(sg[None], su[None])[0])
            self.bwd = bwd
        if self.weights_packed:
            w_gate, w_up, w_down = (moe_pack_weights(w) for w in (w_gate, w_up, w_down))
            if shared_mlp:
                shared_mlp = tuple(moe_pack_weights(w[None])[0] for w in shared_mlp)
        self.tensors = dict(w_router=w_router, w_gate=w_gate, w_up=w_up, w_down=w_down,
                            logit_bias=logit_bias, w_shared_gate=w_shared_gate,
                            expert_bias=expert_bias, count_accum=count_accum)  # kept alive
        self.shared_mlp = shared_mlp      # (gate, up, down) of the one shared MLP, or None
        d_s = shared_mlp[0].shape[0] if shared_mlp else 0
        self.y = torch.empty(T, d, dtype=x.dtype, device=dev)
        self.rows = max_rows(T, N, K, capacity, capacity_group)
        self.out = {}
        a = ForwardArgs()
        a.T, a.d_model, a.N, a.K, a.d_r, a.d_s = T, d, N, K, d_r, d_s
        a.score, a.renorm, a.alpha, a.s, a.capacity, a.dt = score, int(renorm), alpha, s, capacity, _dt(x)
        a.capacity_group = capacity_group
        a.weights_packed = int(self.weights_packed)
        a.x, a.w_router, a.w_gate, a.w_up, a.w_down = (_ptr(x), _ptr(w_router), _ptr(w_gate),
                                                       _ptr(w_up), _ptr(w_down))
        a.logit_bias, a.w_shared_gate = _ptr(logit_bias), _ptr(w_shared_gate)
        a.expert_bias, a.count_accum = _ptr(expert_bias), _ptr(count_accum)
        if shared_mlp:
            a.ws_gate, a.ws_up, a.ws_down = (_ptr(p) for p in shared_mlp)
        a.y = _ptr(self.y)
        if keep_intermediates:
            rows = max(self.rows, 1)
            i32, f32 = torch.int32, torch.float32
            spec = dict(logits=((T, N), f32), topk_idx=((T, K), i32), topk_r=((T, K), f32),
                        C_req=((N,), i32), C_keep=((N,), i32), offsets=((N + 1,), i32),
                        dest_row=((T, K), i32), row_token=((rows,), i32),
                        h_perm=((rows, d_r), x.dtype), f_perm=((rows, d), x.dtype))
            if keep_x_perm:     # an extra copy: the gate/up pass itself gathers from x
                spec["x_perm"] = ((rows, d), x.dtype)
            if w_shared_gate is not None:
                spec["s_tok"] = ((T,), f32)
            if d_s:
                spec["g"] = ((T, d), x.dtype)
            for name, (shape, dtype) in spec.items():
                t = torch.empty(*shape, dtype=dtype, device=dev)
                self.out[name] = t
                setattr(a, name, t.data_ptr())
        if balance_stats:       # f and drop diagnostics of every forward (moe_balance_stats)
            self.out["balance_P"] = torch.empty(N, dtype=torch.float32, device=dev)
            self.out["balance_stats"] = torch.empty(len(STAT_NAMES), dtype=torch.float32, device=dev)
            a.balance_P = self.out["balance_P"].data_ptr()
            a.balance_stats = self.out["balance_stats"].data_ptr()
        self.args = a
        self.ws = _workspace(lib.moe_forward_workspace_size(ctypes.byref(a)), dev)

    def forward(self, stream=None):
        st = lib.moe_forward(ctypes.byref(self.args), self.ws.data_ptr(), self.ws.numel(),
                             _stream() if stream is None else stream)
        _check("moe_forward", st)
        return self.y

    def backward(self, dy):
        """Fixed-router gradients for the last forward (needs trainable=True)."""
        if self.bwd is None:
            raise MoEError("moe_backward", MOE_ERR_INVALID_ARG)
        t = self.tensors
        shared = None
        if self.shared_mlp:
            shared = (self.shared_mlp[0], self.shared_mlp[1]) + self.bwd["shared_t"]
        return moe_backward(self.x, dy, self.out, self.rows, t["w_gate"], t["w_up"],
                            self.bwd["wt_down"], self.bwd["wt_gate_up"], shared=shared,
                            s=self.args.s)


def moe_forward(x, w_router, w_gate, w_up, w_down, K: int, **kw):
    """One whole-layer forward. Returns y, or (y, intermediates) with
    keep_intermediates=True."""
    keep = kw.pop("keep_intermediates", False)
    layer = MoELayer(x, w_router, w_gate, w_up, w_down, K, keep_intermediates=keep, **kw)
    y = layer.forward()
    return (y, layer.out) if keep else y
