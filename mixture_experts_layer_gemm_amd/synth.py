"""Seeded synthetic inputs for the MoE layer forward.

This module only draws and stores inputs; it holds none of the layer's arithmetic. Both
the HIP path and the CPU oracle consume what it produces, which is why it lives apart
from both of them.

Every tensor comes from its own counter-keyed NumPy PCG64 stream,
``np.random.default_rng([seed, cfg_id, tensor_id, index])``, drawn as float32 standard
normals times the workload's standard deviation and, for bf16 workloads, rounded to
bfloat16 with round-to-nearest-even on the float32 bit pattern. The device receives the
exact bf16 bit patterns, and the oracle widens the same bits to float, so both sides
read identical values. Tensor ids: x=0, router=1, routed gate/up/down=2/3/4 (index =
expert), shared gate/up/down=5/6/7 (index = shared expert), shared-gate vector=8.

The workloads follow the layer shapes of the source pages' studies and the public model
families they tabulate: the tiny fp32 layer, the Olmo-style 64-expert top-4 layer, a
fine-grained 256-expert sigmoid layer, a coarse 8-expert routed-only layer, and a
capacity-limited layer whose router is skewed by a Zipf(1.1) per-expert logit bias.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np

SCORE_SOFTMAX, SCORE_SIGMOID, SCORE_SOFTMAX_SELECTED = 0, 1, 2

T_X, T_ROUTER, T_GATE, T_UP, T_DOWN, T_SGATE, T_SUP, T_SDOWN, T_GATEVEC = range(9)


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    T: int
    d_model: int
    N: int
    K: int
    d_r: int
    shared_widths: Tuple[int, ...] = ()
    score: int = SCORE_SOFTMAX
    renorm: bool = True
    alpha: float = 1.0
    s: float = 1.0
    capacity_factor: Optional[float] = None      # None = unlimited (dropless)
    capacity_group: int = 0                      # > 0: rank-wide budget per group of experts
    dtype: str = "bf16"                          # "bf16" or "f32"
    std_x: float = 1.0
    std_w: float = 0.02
    zipf_bias: bool = False                      # b_i = 2 ln(Zipf(1.1) weight of rank i+1)
    shared_gate: bool = False                    # learned sigmoid gate s(x) = sigma(x w_s)
    router_zero: bool = False                    # all router weights zero (every logit ties)
    seed: int = 0

    @property
    def d_s(self) -> int:
        return int(sum(self.shared_widths))

    @property
    def flops_routed_per_route(self) -> int:
        return 6 * self.d_model * self.d_r


CONFIGS = {
    # tiny fp32 layer; the CPU oracle finishes it in well under a second
    "C0": Config("tiny-fp32", 0, T=256, d_model=256, N=8, K=2, d_r=512, shared_widths=(256,),
                 alpha=2.0, dtype="f32", std_w=0.02),
    # Olmo-style: 64 experts, top-4, alpha = K, unit shared gain
    "C1": Config("olmo-64e-top4", 1, T=4096, d_model=2048, N=64, K=4, d_r=2560,
                 shared_widths=(1280,), alpha=4.0, std_w=0.02),
    # fine-grained DeepSeek-V3-like: sigmoid affinities, alpha = 2.5
    "C2": Config("deepseek-v3-like-256e-top8", 2, T=8192, d_model=7168, N=256, K=8, d_r=2048,
                 shared_widths=(2048,), score=SCORE_SIGMOID, alpha=2.5, std_w=0.006),
    # coarse Mixtral-like: softmax over the selected logits, no shared expert
    "C3": Config("mixtral-like-8e-top2", 3, T=16384, d_model=4096, N=8, K=2, d_r=14336,
                 shared_widths=(), score=SCORE_SOFTMAX_SELECTED, alpha=1.0, std_w=0.01),
    # capacity-limited, Zipf-skewed; A: full softmax without renorm + learned shared gate
    "C4A": Config("skewed-capacity-qwen-gate", 4, T=4096, d_model=2048, N=64, K=4, d_r=2560,
                  shared_widths=(1280,), renorm=False, alpha=1.0, capacity_factor=1.0,
                  zipf_bias=True, shared_gate=True, std_w=0.02),
    # B: Olmo rule with three ungated shared experts 640/384/256 (one 1280-wide MLP)
    "C4B": Config("skewed-capacity-3shared", 4, T=4096, d_model=2048, N=64, K=4, d_r=2560,
                  shared_widths=(640, 384, 256), alpha=4.0, capacity_factor=1.0,
                  zipf_bias=True, std_w=0.02),
}

# Small workloads for element-by-element parity: several tiles in every dimension,
# ragged token counts and ragged expert segments, every router mode.
SMALL = {
    "S_softmax": Config("small-softmax", 10, T=1000, d_model=512, N=16, K=4, d_r=320,
                        shared_widths=(192,), alpha=4.0, std_w=0.05),
    "S_sigmoid": Config("small-sigmoid", 11, T=517, d_model=384, N=32, K=8, d_r=256,
                        shared_widths=(128,), score=SCORE_SIGMOID, alpha=2.5, std_w=0.05),
    "S_selected": Config("small-selected", 12, T=700, d_model=256, N=8, K=2, d_r=576,
                         score=SCORE_SOFTMAX_SELECTED, alpha=1.0, std_w=0.05),
    "S_capgate": Config("small-capacity-gate", 13, T=600, d_model=256, N=16, K=4, d_r=192,
                        shared_widths=(128,), renorm=False, alpha=1.0, capacity_factor=1.0,
                        zipf_bias=True, shared_gate=True, std_w=0.05),
    "S_cap3shared": Config("small-capacity-3shared", 14, T=600, d_model=256, N=16, K=4,
                           d_r=192, shared_widths=(64, 128, 64), alpha=4.0,
                           capacity_factor=0.5, zipf_bias=True, std_w=0.05),
    "S_f32": Config("small-fp32", 15, T=333, d_model=192, N=8, K=3, d_r=320,
                    shared_widths=(128,), alpha=3.0, dtype="f32", std_w=0.05),
    "S_tied": Config("small-all-tied", 16, T=300, d_model=256, N=8, K=2, d_r=128,
                     shared_widths=(128,), alpha=2.0, router_zero=True, capacity_factor=1.0,
                     std_w=0.05),
    "S_KeqN": Config("small-k-equals-n", 17, T=129, d_model=128, N=4, K=4, d_r=128,
                     shared_widths=(64,), alpha=4.0, std_w=0.05),
    "S_N1": Config("small-one-expert", 18, T=77, d_model=64, N=1, K=1, d_r=64,
                   alpha=1.0, std_w=0.05),
    # shapes of the persistent GEMM (widths multiples of 256, >= 512), with more tiles
    # than compute units so that tiles follow one another in a workgroup
    "S_stream": Config("small-stream", 19, T=2048, d_model=1024, N=8, K=4, d_r=1024,
                       shared_widths=(512,), alpha=4.0, std_w=0.03),
    "S_stream_cap": Config("small-stream-capacity-gate", 20, T=2048, d_model=512, N=16, K=4,
                           d_r=512, shared_widths=(256, 256), renorm=False, alpha=1.0,
                           capacity_factor=1.0, zipf_bias=True, shared_gate=True, std_w=0.04),
    # rank-wide capacity: four destinations of four experts share one budget each
    "S_rankcap": Config("small-rank-capacity", 21, T=600, d_model=256, N=16, K=4, d_r=192,
                        shared_widths=(128,), alpha=4.0, capacity_factor=1.0, capacity_group=4,
                        zipf_bias=True, std_w=0.05),
    # tighter rank-wide budget on the persistent-GEMM shapes, sigmoid routing
    "S_rankcap_stream": Config("small-stream-rank-capacity", 22, T=2048, d_model=512, N=16,
                               K=4, d_r=512, shared_widths=(256,), score=SCORE_SIGMOID,
                               alpha=2.5, capacity_factor=0.75, capacity_group=2,
                               zipf_bias=True, std_w=0.04),
    # fine-grained routing at a small size: 256 experts, top-8 of sigmoid affinities, a
    # ragged last token tile (the split-K router logits of many experts)
    # many tokens, Zipf-skewed and at capacity: the router's 16-token histogram rows
    # (1025 x 64 counts) exceed what one placement workgroup re-reads, so the forward
    # places with a scan, then the map
    "S_longT": Config("small-many-tokens", 25, T=16400, d_model=256, N=64, K=4, d_r=128,
                      shared_widths=(64,), capacity_factor=1.0, zipf_bias=True, std_w=0.05),
    # router shapes between the small and the many-expert ones: 40 experts + a gate column
    # (three 16-column blocks) over a ragged last token tile; 100 experts (seven blocks,
    # a three-stage LDS ring); 200 experts (not a multiple of 64: the register-direct
    # 32-token router) with a gate and a d_model that is not a multiple of 128
    "S_mid40": Config("small-40-experts-gate", 26, T=1001, d_model=384, N=40, K=5, d_r=128,
                      shared_widths=(64,), shared_gate=True, capacity_factor=1.25, std_w=0.05),
    "S_mid100": Config("small-100-experts", 27, T=555, d_model=640, N=100, K=6, d_r=192,
                       score=SCORE_SIGMOID, alpha=2.0, std_w=0.04),
    "S_mid200": Config("small-200-experts-gate", 28, T=300, d_model=320, N=200, K=8, d_r=128,
                       shared_widths=(64,), shared_gate=True, std_w=0.04),
    "S_wide": Config("small-256-experts", 23, T=1000, d_model=1024, N=256, K=8, d_r=256,
                     shared_widths=(128,), score=SCORE_SIGMOID, alpha=2.5, std_w=0.03),
    # 192 experts (three groups of 64) under the Olmo rule, d_model in two slices
    "S_wide192": Config("small-192-experts", 24, T=300, d_model=768, N=192, K=6, d_r=128,
                        shared_widths=(64,), alpha=6.0, std_w=0.04),
}


def get_config(name: str) -> Config:
    if name in CONFIGS:
        return CONFIGS[name]
    if name in SMALL:
        return SMALL[name]
    raise KeyError(name)


# ---------------------------------------------------------------------------------------
# bfloat16 storage
# ---------------------------------------------------------------------------------------
def bf16_bits(f32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
            ).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit pattern -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def stream(cfg: Config, tensor_id: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([cfg.seed, cfg.cfg_id, tensor_id, index])


def _draw(cfg: Config, tensor_id: int, index: int, shape, std: float, out=None):
    """One tensor from its own stream: float32 normals * std, stored in the workload's
    dtype (uint16 bit patterns for bf16). Writes into `out` when given."""
    v = stream(cfg, tensor_id, index).standard_normal(size=shape, dtype=np.float32)
    v *= np.float32(std)
    if cfg.dtype != "bf16":
        if out is not None:
            out[...] = v
            return out
        return v
    # round to nearest even in place: u += 0x7FFF + ((u >> 16) & 1); keep the top half
    u = v.view(np.uint32)
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    u += t
    u >>= np.uint32(16)
    if out is None:
        out = np.empty(shape, dtype=np.uint16)
    np.copyto(out, u, casting="unsafe")
    return out


def zipf_logit_bias(N: int, a: float = 1.1) -> np.ndarray:
    """Per-expert logit bias b_i = 2 ln(w_{i+1}), w_k = k^-a / sum_{j<=N} j^-a: expert i
    is given Zipf rank i+1, so expert 0 is the most favoured. Returned as float32."""
    k = np.arange(1, N + 1, dtype=np.float64)
    w = k ** (-a)
    w = w / w.sum()
    return (2.0 * np.log(w)).astype(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


@dataclass
class LayerInputs:
    """Stored inputs of one layer (uint16 bf16 bits or float32 values)."""
    cfg: Config
    x: np.ndarray                 # [T, d_model]
    w_router: np.ndarray          # [N, d_model]
    w_gate: np.ndarray            # [N, d_r, d_model]
    w_up: np.ndarray              # [N, d_r, d_model]
    w_down: np.ndarray            # [N, d_model, d_r]
    shared: list = field(default_factory=list)   # [(w_gate [m_j, d], w_up [m_j, d], w_down [d, m_j])]
    logit_bias: Optional[np.ndarray] = None       # [N] float32
    w_shared_gate: Optional[np.ndarray] = None    # [d_model]

    def as_float(self, a: np.ndarray) -> np.ndarray:
        """Stored values widened to float32 (exact for bf16)."""
        return bf16_to_f32(a) if self.cfg.dtype == "bf16" else np.asarray(a, np.float32)

    def expert_f32(self, i: int):
        return (self.as_float(self.w_gate[i]), self.as_float(self.w_up[i]),
                self.as_float(self.w_down[i]))

    def shared_f32(self):
        return [tuple(self.as_float(w) for w in ws) for ws in self.shared]


def make_inputs(cfg: Config, T: Optional[int] = None, progress=None) -> LayerInputs:
    """Draw every input of `cfg` (optionally with a different token count T, which
    keeps the same streams, so a smaller T gives a prefix of the same tokens).
    `progress(done, total)` is called as expert weights are drawn."""
    T = cfg.T if T is None else T
    d, N, dr = cfg.d_model, cfg.N, cfg.d_r
    sdt = np.uint16 if cfg.dtype == "bf16" else np.float32
    x = _draw(cfg, T_X, 0, (cfg.T, d), cfg.std_x)[:T].copy() if T <= cfg.T else None
    if x is None:
        x = _draw(replace(cfg, T=T), T_X, 0, (T, d), cfg.std_x)
    if cfg.router_zero:
        w_router = np.zeros((N, d), dtype=sdt)
    else:
        w_router = _draw(cfg, T_ROUTER, 0, (N, d), cfg.std_w)
    w_gate = np.empty((N, dr, d), dtype=sdt)
    w_up = np.empty((N, dr, d), dtype=sdt)
    w_down = np.empty((N, d, dr), dtype=sdt)

    def one(i):
        _draw(cfg, T_GATE, i, (dr, d), cfg.std_w, out=w_gate[i])
        _draw(cfg, T_UP, i, (dr, d), cfg.std_w, out=w_up[i])
        _draw(cfg, T_DOWN, i, (d, dr), cfg.std_w, out=w_down[i])

    with ThreadPoolExecutor(_threads()) as ex:
        for i, _ in enumerate(ex.map(one, range(N))):
            if progress is not None and (i + 1) % 16 == 0:
                progress(i + 1, N)
    shared = []
    for j, m in enumerate(cfg.shared_widths):
        shared.append((_draw(cfg, T_SGATE, j, (m, d), cfg.std_w),
                       _draw(cfg, T_SUP, j, (m, d), cfg.std_w),
                       _draw(cfg, T_SDOWN, j, (d, m), cfg.std_w)))
    bias = zipf_logit_bias(N) if cfg.zipf_bias else None
    gate = _draw(cfg, T_GATEVEC, 0, (d,), cfg.std_w) if cfg.shared_gate else None
    return LayerInputs(cfg, x, w_router, w_gate, w_up, w_down, shared, bias, gate)
