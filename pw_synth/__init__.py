"""Seeded synthetic MoE-layer inputs, shared by the oracle and the HIP path.

This module only draws random numbers; it holds none of the method's
arithmetic (no decode, no routing, no contraction).  Both the CPU oracle and
the HIP library consume exactly the arrays produced here.

Workload shapes follow the models the PagedWeight pages evaluate on
(Qwen1.5-MoE-A2.7B, Mixtral-8x7B; page "Technical summary: PagedWeight",
"Core contributions" item 4).  The pages give no weights, so every array is
synthetic:

* activations x: fp16 from N(0, 1);
* router logits: fp32 from N(0, 1), optionally plus a Zipf(1.1) per-expert bias
  (bias_e = -1.1 * ln(rank_e), rank a seeded permutation of 1..E);
* parent codes: uint8 uniform over 0..255 (p = 8 bits);
* per-row LUTs: for every child width k in 3..8, 2**k draws of N(0, 0.02**2),
  sorted ascending, rounded to fp16 (round-to-nearest-even, subnormals kept);
* committed width q per linear block: uniform in 3..8, or tiered by Zipf rank
  (top 10% of experts at 8, next 30% in {5, 6}, the rest in {3, 4}).

Every stream is keyed by numpy SeedSequence([seed, stream, layer, ...]) so any
piece can be regenerated on its own, in any order, on any machine.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

SEED_BASE = 20260720
QMIN, QMAX = 3, 8
PARENT_BITS = 8
LUT_SIGMA = 0.02

# stream ids inside a config's SeedSequence
_S_WEIGHTS, _S_ACT, _S_Q, _S_RANK = 0, 1, 2, 3


@dataclass
class LayerShape:
    """One MoE layer: hidden H, expert intermediate I, E routed experts,
    top_k routing, optional shared expert with intermediate I_shared."""
    H: int
    I: int
    E: int
    top_k: int
    I_shared: int = 0


@dataclass
class Block:
    """One per-expert linear block in parent-code form.

    code8: uint8 [R][K] parent codes; luts[k]: fp16 [R][2**k] for k in 3..8;
    q: committed width.  For gate_up R = 2*I (rows [0, I) gate, [I, 2I) up),
    K = H; for down R = H, K = I.
    """
    code8: np.ndarray
    luts: Dict[int, np.ndarray]
    q: int

    @property
    def R(self) -> int:
        return int(self.code8.shape[0])

    @property
    def K(self) -> int:
        return int(self.code8.shape[1])


@dataclass
class LayerWeights:
    shape: LayerShape
    gate_up: List[Block]
    down: List[Block]
    shared_gate_up: Optional[Block] = None
    shared_down: Optional[Block] = None
    rank: Optional[np.ndarray] = None  # Zipf rank (1 = hottest) per expert


@dataclass
class Activations:
    x: np.ndarray       # fp16 [T][H]
    logits: np.ndarray  # fp32 [T][E]


@dataclass
class ConfigSpec:
    name: str
    shape: LayerShape
    tokens: Sequence[int]
    logits: str = "normal"      # "normal" | "zipf"
    q_policy: str = "uniform"   # "uniform" | "zipf_tiers"
    layers: int = 1
    steps: int = 1
    extra: dict = field(default_factory=dict)


CONFIGS: Dict[int, ConfigSpec] = {
    0: ConfigSpec("toy", LayerShape(H=256, I=512, E=4, top_k=2), tokens=[16]),
    1: ConfigSpec("qwen1.5-moe-a2.7b-layer-decode",
                  LayerShape(H=2048, I=1408, E=60, top_k=4, I_shared=5632),
                  tokens=[4], logits="zipf", q_policy="zipf_tiers"),
    2: ConfigSpec("mixtral-8x7b-layer-decode",
                  LayerShape(H=4096, I=14336, E=8, top_k=2), tokens=[1, 4, 16, 64]),
    3: ConfigSpec("mixtral-8x7b-layer-prefill",
                  LayerShape(H=4096, I=14336, E=8, top_k=2), tokens=[4096]),
    4: ConfigSpec("qwen1.5-moe-24-layer-stack-decode",
                  LayerShape(H=2048, I=1408, E=60, top_k=4, I_shared=5632),
                  tokens=[4], logits="zipf", q_policy="zipf_tiers",
                  layers=24, steps=64,
                  extra=dict(commit_every=8, commit_fraction=0.2)),
}


def config_seed(cfg: int) -> int:
    return SEED_BASE + int(cfg)


# Seed of every workload built from a user-supplied model config.
USER_CONFIG_SEED = SEED_BASE + 100

# Model-config keys read for each layer dimension, in order of preference
# (the names common Hugging Face MoE configs use; H/I/E/top_k/I_shared
# themselves are accepted too).
_SHAPE_KEYS = {
    "H": ("H", "hidden_size", "d_model"),
    "I": ("I", "moe_intermediate_size", "expert_intermediate_size", "moe_ffn_hidden_size",
          "intermediate_size"),
    "E": ("E", "num_experts", "num_local_experts", "n_routed_experts", "moe_num_experts"),
    "top_k": ("top_k", "num_experts_per_tok", "top_k_experts", "moe_top_k", "num_selected_experts"),
}


def _first(cfg: dict, keys):
    for key in keys:
        if cfg.get(key) is not None:
            return key, cfg[key]
    return None, None


def shape_from_model_config(cfg) -> "tuple[LayerShape, int, str]":
    """(LayerShape, layers, name) of a MoE model described by a config dict or
    a JSON file path.  A nested "text_config" dict (multimodal configs) is
    read first.  The shared expert's width is shared_expert_intermediate_size,
    else n_shared_experts (or num_shared_experts) times the routed I, else 0.
    Raises ValueError naming a missing key or a dimension the bit-plane
    layout cannot hold (H, I and I_shared must be multiples of 32)."""
    import json
    import os
    name = None
    if not isinstance(cfg, dict):
        path = os.fspath(cfg)
        with open(path) as f:
            cfg = json.load(f)
        name = os.path.splitext(os.path.basename(path))[0]
    flat = dict(cfg)
    if isinstance(cfg.get("text_config"), dict):
        flat.update({k: v for k, v in cfg["text_config"].items() if v is not None})
    dims = {}
    for dim, keys in _SHAPE_KEYS.items():
        key, val = _first(flat, keys)
        if key is None:
            raise ValueError("model config has no %s (looked for %s)" % (dim, ", ".join(keys)))
        dims[dim] = int(val)
    _, shared = _first(flat, ("I_shared", "shared_expert_intermediate_size"))
    if shared is None:
        _, n_shared = _first(flat, ("n_shared_experts", "num_shared_experts"))
        shared = int(n_shared or 0) * dims["I"]
    dims["I_shared"] = int(shared)
    for dim in ("H", "I", "I_shared"):
        if dims[dim] < 0 or dims[dim] % 32:
            raise ValueError("%s = %d: hidden and intermediate sizes must be multiples of 32" % (dim, dims[dim]))
    if dims["H"] == 0 or dims["I"] == 0:
        raise ValueError("H and I must be positive")
    if not 1 <= dims["top_k"] <= dims["E"]:
        raise ValueError("top_k = %d must lie in 1..E = %d" % (dims["top_k"], dims["E"]))
    _, layers = _first(flat, ("num_hidden_layers", "n_layers", "num_layers"))
    name = str(flat.get("name") or flat.get("_name_or_path") or name or flat.get("model_type") or "user-model")
    return LayerShape(**dims), int(layers or 1), name


def model_config_spec(cfg, tokens: Sequence[int] = (4,)) -> ConfigSpec:
    """Decode workload of one layer of a user-supplied MoE model config
    (shape_from_model_config): Zipf-biased routing and widths tiered by
    routing rank, as for the Qwen-shaped layer; seed USER_CONFIG_SEED."""
    shape, layers, name = shape_from_model_config(cfg)
    return ConfigSpec("%s-layer-decode" % name, shape, tokens=list(tokens), logits="zipf",
                      q_policy="zipf_tiers", extra=dict(model_layers=layers, user_config=True))


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, key)])))


def draw_codes(rng: np.random.Generator, R: int, K: int) -> np.ndarray:
    return rng.integers(0, 1 << PARENT_BITS, size=(R, K), dtype=np.uint8)


def draw_luts(rng: np.random.Generator, R: int) -> Dict[int, np.ndarray]:
    luts = {}
    for k in range(QMIN, QMAX + 1):
        v = rng.normal(0.0, LUT_SIGMA, size=(R, 1 << k))
        v.sort(axis=1)
        luts[k] = v.astype(np.float16)
    return luts


def draw_block(rng: np.random.Generator, R: int, K: int, q: int) -> Block:
    code8 = draw_codes(rng, R, K)
    luts = draw_luts(rng, R)
    return Block(code8=code8, luts=luts, q=int(q))


def zipf_rank(seed: int, layer: int, E: int) -> np.ndarray:
    """Seeded permutation giving each expert a rank in 1..E (1 = hottest)."""
    perm = _rng(seed, _S_RANK, layer).permutation(E)
    rank = np.empty(E, dtype=np.int64)
    rank[perm] = np.arange(1, E + 1)
    return rank


def zipf_bias(rank: np.ndarray, s: float = 1.1) -> np.ndarray:
    return (-s * np.log(rank.astype(np.float64))).astype(np.float32)


def draw_q(seed: int, layer: int, E: int, policy: str,
           rank: Optional[np.ndarray] = None) -> np.ndarray:
    """Committed widths q[e][m] (m = 0 gate_up, 1 down) for the routed blocks."""
    rng = _rng(seed, _S_Q, layer)
    if policy == "uniform":
        return rng.integers(QMIN, QMAX + 1, size=(E, 2)).astype(np.int32)
    if policy == "zipf_tiers":
        assert rank is not None
        q = np.empty((E, 2), dtype=np.int32)
        hot = int(round(0.1 * E))
        warm = int(round(0.3 * E))
        lo_draw = rng.integers(0, 2, size=(E, 2))
        for e in range(E):
            r = int(rank[e])
            if r <= hot:
                q[e] = 8
            elif r <= hot + warm:
                q[e] = 5 + lo_draw[e]
            else:
                q[e] = 3 + lo_draw[e]
        return q
    raise ValueError(policy)


def make_weights(shape: LayerShape, seed: int, layer: int = 0, q_policy: str = "uniform",
                 logits: str = "normal", experts: Optional[Sequence[int]] = None) -> LayerWeights:
    """Draw every block of one layer (or only `experts`; others are None)."""
    rank = zipf_rank(seed, layer, shape.E) if (logits == "zipf" or q_policy == "zipf_tiers") else None
    q = draw_q(seed, layer, shape.E, q_policy, rank)
    want = set(range(shape.E)) if experts is None else set(int(e) for e in experts)
    gu: List[Optional[Block]] = []
    dn: List[Optional[Block]] = []
    for e in range(shape.E):
        if e not in want:
            gu.append(None)
            dn.append(None)
            continue
        rng = _rng(seed, _S_WEIGHTS, layer, e)
        gu.append(draw_block(rng, 2 * shape.I, shape.H, q[e, 0]))
        dn.append(draw_block(rng, shape.H, shape.I, q[e, 1]))
    sgu = sdn = None
    if shape.I_shared:
        rng = _rng(seed, _S_WEIGHTS, layer, 1 << 20)
        sgu = draw_block(rng, 2 * shape.I_shared, shape.H, QMAX)
        sdn = draw_block(rng, shape.H, shape.I_shared, QMAX)
    return LayerWeights(shape=shape, gate_up=gu, down=dn, shared_gate_up=sgu,
                        shared_down=sdn, rank=rank)


def make_activations(shape: LayerShape, T: int, seed: int, layer: int = 0, step: int = 0,
                     logits: str = "normal", rank: Optional[np.ndarray] = None) -> Activations:
    rng = _rng(seed, _S_ACT, layer, step, T)
    lg = rng.normal(0.0, 1.0, size=(T, shape.E)).astype(np.float32)
    if logits == "zipf":
        if rank is None:
            rank = zipf_rank(seed, layer, shape.E)
        lg = (lg + zipf_bias(rank)[None, :]).astype(np.float32)
    x = rng.normal(0.0, 1.0, size=(T, shape.H)).astype(np.float16)
    return Activations(x=x, logits=lg)


def make_config(cfg: int, T: Optional[int] = None, layer: int = 0, step: int = 0,
                experts: Optional[Sequence[int]] = None):
    """Weights + activations of one layer of configuration `cfg` (0..4)."""
    spec = CONFIGS[cfg]
    seed = config_seed(cfg)
    T = spec.tokens[0] if T is None else int(T)
    w = make_weights(spec.shape, seed, layer, spec.q_policy, spec.logits, experts)
    a = make_activations(spec.shape, T, seed, layer, step, spec.logits, w.rank)
    return w, a


def make_small(H: int, I: int, E: int, top_k: int, T: int, I_shared: int = 0,
               seed: int = 12345, q_policy: str = "uniform", logits: str = "normal",
               q_fixed: Optional[int] = None):
    """A small seeded layer for parity tests (same distributions as the configs)."""
    shape = LayerShape(H=H, I=I, E=E, top_k=top_k, I_shared=I_shared)
    w = make_weights(shape, seed, 0, q_policy, logits)
    if q_fixed is not None:
        for b in w.gate_up + w.down:
            b.q = int(q_fixed)
    a = make_activations(shape, T, seed, 0, 0, logits, w.rank)
    return w, a
