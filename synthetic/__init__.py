"""Seeded synthetic inputs for the routed-MoE expert layer.

This module only draws random numbers and arranges them into the shapes of
the workloads; it holds none of the layer's arithmetic (no quantization, no
routing, no FFN).  Both the oracle side and the GPU side take their inputs
from here.

Workloads (shapes of a DeepSeek-V3-class MoE layer; the pages name the
quantization mix -- "DwarfStar" README, section on model weights -- but give
no shapes, so the shapes are the stated workload definitions):

  tiny         H=256  I=128  E=8   k=2  T=4     x fp32, no shared expert
  decode1      H=7168 I=2048 E=256 k=8  T=1     x bf16, + bf16 shared expert
  decode32     same layer                 T=32    Zipf(1.1)-skewed logits
  prefill2048  same layer                 T=2048  unskewed logits
  prefill8192  same layer                 T=8192  Zipf-skewed logits
  prefill8192_q4k  as prefill8192 with all three routed projections in Q4_K
  decode32_q4k     as decode32 with all three routed projections in Q4_K
  prefill2048_cb2s, decode32_cb2s  as prefill2048 / decode32 with gate/up in
                   the signed codebook format (66 B per 256 weights)

Every tensor comes from its own child stream of one layer seed
(``numpy.random.default_rng([seed, tag, index])``), so one expert can be
regenerated without materialising the whole 11.3 G-weight layer.
"""
from __future__ import annotations

import json
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

LAYER_SEED = 0
WEIGHT_STD = 0.02

# stream tags
_TAG_GATE, _TAG_UP, _TAG_DOWN = 1, 2, 3
_TAG_SHARED = 4
_TAG_ROUTER = 5
_TAG_CODEBOOK = 6
_TAG_TOKENS = 7
_TAG_GRID = 8

FMT_CB2, FMT_Q2K, FMT_Q4K, FMT_BF16, FMT_Q5K, FMT_Q6K, FMT_CB2S = 1, 2, 3, 4, 5, 6, 7

_BIG = dict(hidden=7168, inter=2048, n_experts=256, top_k=8, sh_inter=2048)

CONFIGS = {
    "tiny": dict(hidden=256, inter=128, n_experts=8, top_k=2, sh_inter=0,
                 T=4, x_dtype="f32", skew=False,
                 fmt_gate_up=FMT_CB2, fmt_down=FMT_Q2K, index=0),
    "decode1": dict(_BIG, T=1, x_dtype="bf16", skew=False,
                    fmt_gate_up=FMT_CB2, fmt_down=FMT_Q2K, index=1),
    "decode32": dict(_BIG, T=32, x_dtype="bf16", skew=True,
                     fmt_gate_up=FMT_CB2, fmt_down=FMT_Q2K, index=2),
    "prefill2048": dict(_BIG, T=2048, x_dtype="bf16", skew=False,
                        fmt_gate_up=FMT_CB2, fmt_down=FMT_Q2K, index=3),
    "prefill8192": dict(_BIG, T=8192, x_dtype="bf16", skew=True,
                        fmt_gate_up=FMT_CB2, fmt_down=FMT_Q2K, index=4),
    "prefill8192_q4k": dict(_BIG, T=8192, x_dtype="bf16", skew=True,
                            fmt_gate_up=FMT_Q4K, fmt_down=FMT_Q4K, index=4),
    "decode32_q4k": dict(_BIG, T=32, x_dtype="bf16", skew=True,
                         fmt_gate_up=FMT_Q4K, fmt_down=FMT_Q4K, index=4),
    "prefill2048_cb2s": dict(_BIG, T=2048, x_dtype="bf16", skew=False,
                             fmt_gate_up=FMT_CB2S, fmt_down=FMT_Q2K, index=3),
    "decode32_cb2s": dict(_BIG, T=32, x_dtype="bf16", skew=True,
                          fmt_gate_up=FMT_CB2S, fmt_down=FMT_Q2K, index=2),
}

_GOLDEN = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "tests", "golden")


# Per-layer quantization recipes: (gate/up format, down format) of layer l of
# an n-layer stack.  "q2" is the pages' 2-bit recipe for every layer; "q2-q4"
# keeps the last 6 layers in Q4_K ("DwarfStar" README and "ds4" README
# mirror, section on model weights: q2 with the last six layers in q4; a stack
# shorter than 12 layers keeps its last half in Q4_K); "q4" is Q4_K throughout;
# "q5-q6" is the wider routed mix the "ds4" mirror lists for other models
# (gate/up Q5_K, down Q6_K); "q2s" is "q2" with gate/up in the signed codebook
# format, the byte budget of the pages' 2-bit gate/up type.
RECIPES = ("q2", "q2-q4", "q4", "q5-q6", "q2s")


def layer_formats(recipe: str, layer: int, n_layers: int) -> tuple:
    if recipe == "q2":
        return FMT_CB2, FMT_Q2K
    if recipe == "q2-q4":
        return (FMT_Q4K, FMT_Q4K) if layer >= n_layers - min(6, n_layers // 2) else (FMT_CB2, FMT_Q2K)
    if recipe == "q4":
        return FMT_Q4K, FMT_Q4K
    if recipe == "q5-q6":
        return FMT_Q5K, FMT_Q6K
    if recipe == "q2s":
        return FMT_CB2S, FMT_Q2K
    raise ValueError("unknown recipe %r" % recipe)


def config(name: str, **override) -> dict:
    c = dict(CONFIGS[name])
    c["name"] = name
    c.update(override)
    return c


# ----------------------------------------------------------------- codebook
def codebook(seed: int = LAYER_SEED) -> np.ndarray:
    """256 distinct 8-vectors with entries drawn uniformly from {-3,-1,1,3}.

    Duplicates are redrawn (in index order) so that every index names a
    distinct vector.  Returned as int8 [256, 8].
    """
    rng = np.random.default_rng([seed, _TAG_CODEBOOK])
    levels = np.array([-3, -1, 1, 3], dtype=np.int8)
    out = np.empty((256, 8), dtype=np.int8)
    seen = set()
    i = 0
    while i < 256:
        row = levels[rng.integers(0, 4, size=8)]
        key = row.tobytes()
        if key in seen:
            continue
        seen.add(key)
        out[i] = row
        i += 1
    return out


def grid_cb2s(seed: int = LAYER_SEED) -> np.ndarray:
    """The magnitude grid of the signed codebook format: 256 distinct 8-vectors
    with entries drawn from {1, 3, 5} with probabilities 1/2, 1/3, 1/6 (small
    magnitudes are the common ones for bell-shaped weights).  Duplicates are
    redrawn in index order.  Returned as uint8 [256, 8]."""
    rng = np.random.default_rng([seed, _TAG_GRID])
    levels = np.array([1, 3, 5], dtype=np.uint8)
    out = np.empty((256, 8), dtype=np.uint8)
    seen = set()
    i = 0
    while i < 256:
        row = levels[rng.choice(3, size=8, p=[0.5, 1.0 / 3.0, 1.0 / 6.0])]
        key = row.tobytes()
        if key in seen:
            continue
        seen.add(key)
        out[i] = row
        i += 1
    return out


def codebook_for(fmt: int, seed: int = LAYER_SEED) -> np.ndarray:
    """The table a gate/up format reads: the signed grid for FMT_CB2S, else the
    CB2 codebook (ignored by the formats that have none)."""
    return grid_cb2s(seed) if fmt == FMT_CB2S else codebook(seed)


# ------------------------------------------------------------------ weights
def _normal(stream, shape, std=WEIGHT_STD) -> np.ndarray:
    rng = np.random.default_rng(stream)
    a = rng.standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(std)
    return a


def router_weight(cfg: dict, seed: int = LAYER_SEED) -> np.ndarray:
    """W_r [E, H] fp32, N(0, 0.02)."""
    return _normal([seed, _TAG_ROUTER], (cfg["n_experts"], cfg["hidden"]))


def expert_weight(cfg: dict, which: str, e: int, seed: int = LAYER_SEED) -> np.ndarray:
    """fp32 weight of routed expert e before quantization, N(0, 0.02).

    gate/up: [I, H] (rows = intermediate features, K = hidden);
    down:    [H, I] (rows = hidden features,      K = intermediate).
    """
    H, I = cfg["hidden"], cfg["inter"]
    tag = {"gate": _TAG_GATE, "up": _TAG_UP, "down": _TAG_DOWN}[which]
    shape = (H, I) if which == "down" else (I, H)
    return _normal([seed, tag, e], shape)


def shared_weight_f32(cfg: dict, which: str, seed: int = LAYER_SEED) -> np.ndarray:
    """fp32 draw of the shared expert; callers round it to bf16 (shared_weight_bf16)."""
    H, I = cfg["hidden"], cfg["sh_inter"]
    j = {"gate": 0, "up": 1, "down": 2}[which]
    shape = (H, I) if which == "down" else (I, H)
    return _normal([seed, _TAG_SHARED, j], shape)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even) and return the uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def shared_weight_bf16(cfg: dict, which: str, seed: int = LAYER_SEED) -> np.ndarray:
    """Shared-expert weight as bf16 bit patterns (uint16), row-major."""
    return bf16_bits(shared_weight_f32(cfg, which, seed))


# ------------------------------------------------------------------- tokens
def tokens_f32(cfg: dict, T: int | None = None, seed: int = LAYER_SEED) -> np.ndarray:
    """x [T, H] fp32 N(0,1); one stream per workload index."""
    T = cfg["T"] if T is None else T
    rng = np.random.default_rng([seed, _TAG_TOKENS, cfg["index"]])
    return rng.standard_normal(size=(T, cfg["hidden"]), dtype=np.float32)


def tokens(cfg: dict, T: int | None = None, seed: int = LAYER_SEED):
    """Activations as the workload feeds them.

    Returns (array, kind): kind 'f32' -> float32 [T,H]; kind 'bf16' -> uint16
    bf16 bit patterns [T,H] (round-to-nearest-even of the fp32 draw).
    """
    x = tokens_f32(cfg, T, seed)
    if cfg["x_dtype"] == "bf16":
        return bf16_bits(x), "bf16"
    return x, "f32"


# --------------------------------------------------------------- logit bias
def zipf_log_p(E: int, s: float = 1.1) -> np.ndarray:
    """ln p_e for p_e proportional to (e+1)^-s, normalised over the E experts."""
    r = np.arange(1, E + 1, dtype=np.float64)
    lp = -s * np.log(r)
    lp -= np.log(np.exp(lp).sum())
    return lp


def zipf_beta() -> float:
    """Bias strength beta, stored by tests/golden/make_zipf_beta.py."""
    with open(os.path.join(_GOLDEN, "zipf_beta.json")) as f:
        return float(json.load(f)["beta"])


def logit_bias(cfg: dict, beta: float | None = None):
    """Router logit bias b[E] (fp32) or None for unskewed workloads.

    b_e = beta * ln p_e with Zipf(1.1) p_e.  beta is fixed once so that the 8
    most-assigned experts take about 30% of the prefill8192 assignments.
    """
    if not cfg.get("skew"):
        return None
    beta = zipf_beta() if beta is None else beta
    return (beta * zipf_log_p(cfg["n_experts"])).astype(np.float32)


# ------------------------------------------------------ whole-layer helpers
def for_each_expert(cfg: dict, fn, experts=None, threads: int | None = None, seed: int = LAYER_SEED):
    """Call fn(e, gate, up, down) for each expert, generating in parallel threads.

    numpy's generators release the GIL while filling, so threads overlap the
    draws.  fn runs in the worker threads too.
    """
    experts = range(cfg["n_experts"]) if experts is None else list(experts)
    threads = threads or min(16, os.cpu_count() or 1)

    def job(e):
        fn(e, expert_weight(cfg, "gate", e, seed), expert_weight(cfg, "up", e, seed),
           expert_weight(cfg, "down", e, seed))

    with ThreadPoolExecutor(threads) as ex:
        for _ in ex.map(job, experts):
            pass
