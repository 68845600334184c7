"""Seeded synthetic workloads for the folded multi-branch verify layer.

This module only draws inputs: draft graphs, per-branch hidden states, layer
weights and a shared-prefix KV cache.  It holds none of the layer's arithmetic
(no gate, no attention, no GEMM), so both the CPU oracle's tests and the HIP
path can consume the same inputs without sharing method code.

Workload model (SpecFold explainer, blog.ontle.kr/blog/358, sections on the
parent/child candidates and the "residual ripple" of section 4.4): a child
branch equals its parent block state except at one or a few newly revealed
positions, whose change spreads to nearby positions through bidirectional
attention.  A child is therefore drawn as parent + N(0,1) at its revealed
positions + a ripple whose standard deviation decays exponentially with the
distance to the nearest revealed position.  Draft graphs are trees or
multi-parent DAGs (Spiffy explainer, lifetechia.com/?p=5403, section on the
directed draft graph); the first parent of a node is its fold source.

All values are drawn in fp32 from numpy PCG64 streams (seed 1000 + config id,
sub-streams via SeedSequence.spawn).  For bf16 configurations every tensor is
rounded to bf16 (round-to-nearest-even) and returned as the exactly
representable fp32 values, so both consumers see bit-identical inputs.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = [
    "Config", "CONFIGS", "Workload", "make_workload", "make_layer_weights",
    "round_bf16", "bf16_bits", "draft_graph", "hidden_states", "prefix_cache",
    "custom_config", "budget_config", "BUDGETS", "graph_depth", "layer_weights_of",
    "lm_head_weights", "VOCAB_7B",
    "layer_cache_of", "iter_layers",
]


@dataclasses.dataclass(frozen=True)
class Config:
    """Shape and workload recipe of one verify-layer configuration."""
    name: str
    num_nodes: int          # root + children (N)
    block: int              # block length (B)
    hidden: int             # d
    n_q: int
    n_kv: int
    head_dim: int
    ffn: int
    prefix: int             # shared prefix length (P)
    dtype: str              # "f32" or "bf16"
    tau: float
    graph: str              # "chain2", "tree3", "dag", "dag_deep"
    reveal: Tuple[int, int]  # inclusive range of revealed positions per child
    ripple_len: float = 3.0
    ripple_amp: float = 0.1
    layers: int = 1
    seed: int = 1000
    taus: Tuple[float, ...] = ()
    rms_eps: float = 1e-6
    max_depth: int = 0      # dag_deep only
    weight_std: float = 0.02  # std of the linear weights
    rope_theta: float = 0.0   # rotary embedding base (0: none)
    qkv_bias: bool = False    # QKV projection bias ~ N(0, 0.1^2)

    @property
    def slots(self) -> int:
        return self.num_nodes * self.block

    @property
    def qkv_dim(self) -> int:
        return (self.n_q + 2 * self.n_kv) * self.head_dim

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


# The five workloads of this method's benchmark plan.
CONFIGS: Dict[int, Config] = {
    0: Config("tiny-fp32", num_nodes=4, block=32, hidden=256, n_q=4, n_kv=2, head_dim=64,
              ffn=1024, prefix=64, dtype="f32", tau=0.05, graph="chain2", reveal=(1, 1),
              seed=1000),
    1: Config("7b-layer-1+15", num_nodes=16, block=32, hidden=3584, n_q=28, n_kv=4,
              head_dim=128, ffn=18944, prefix=512, dtype="bf16", tau=0.05, graph="tree3",
              reveal=(1, 2), seed=1001),
    2: Config("3b-layer-dag-1+31", num_nodes=32, block=32, hidden=3072, n_q=24, n_kv=8,
              head_dim=128, ffn=8192, prefix=2048, dtype="bf16", tau=0.05, graph="dag",
              reveal=(1, 2), ripple_len=5.0, seed=1002, taus=(0.0, 0.02, 0.05, 0.1)),
    3: Config("7b-stack28-1+31", num_nodes=32, block=32, hidden=3584, n_q=28, n_kv=4,
              head_dim=128, ffn=18944, prefix=4096, dtype="bf16", tau=0.05, graph="tree3",
              reveal=(1, 2), layers=28, seed=1003),
    4: Config("stress-1+63", num_nodes=64, block=64, hidden=4096, n_q=32, n_kv=4,
              head_dim=128, ffn=14336, prefix=16384, dtype="bf16", tau=0.02,
              graph="dag_deep", reveal=(1, 4), seed=1004, max_depth=6),
}


# Draft budgets of the budget sweep (SpecFold explainer, Fig. 3 and the draft-budget
# appendix: per-verify latency against the number of draft branches): the 7B-shaped layer
# with 1 + {3, 7, 15, 31, 63} branches of the same 3-ary level-order tree.
BUDGETS: Tuple[int, ...] = (4, 8, 16, 32, 64)


def budget_config(num_nodes: int) -> Config:
    """The 7B-shaped layer with `num_nodes` nodes (root + children); same seed, weights and
    prefix as the 1 + 15 layer, so only the draft graph and the hidden states change."""
    return CONFIGS[1].with_(num_nodes=num_nodes, name=f"7b-layer-1+{num_nodes - 1}")


# Vocabulary of the 7B-shaped model family (Qwen2-style tokenizer size) for the LM head
# that follows the layer stack.
VOCAB_7B = 152064


def lm_head_weights(cfg: Config, vocab: int) -> Tuple[np.ndarray, np.ndarray]:
    """Final RMSNorm gain (ones, like the layers' gains) and LM-head weight [vocab, d]
    ~ N(0, weight_std^2), rounded to the configuration's storage format.  Seeded from the
    configuration's seed on a stream of its own, so the layer inputs do not change."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, 0x1B, vocab])))
    w = rng.standard_normal((vocab, cfg.hidden), dtype=np.float32)
    w *= np.float32(cfg.weight_std)
    g = np.ones(cfg.hidden, dtype=np.float32)
    return _storage(cfg, g), _storage(cfg, w)


def custom_config(**kw) -> Config:
    """A small configuration for tests (defaults: a tiny fp32 layer)."""
    base = dict(name="custom", num_nodes=4, block=8, hidden=64, n_q=2, n_kv=1, head_dim=64,
                ffn=128, prefix=16, dtype="f32", tau=0.05, graph="tree3", reveal=(1, 1),
                seed=7)
    base.update(kw)
    return Config(**base)


# ----------------------------------------------------------------------------------------
# bf16 storage format (round-to-nearest-even); a data-format conversion, not layer math.
# ----------------------------------------------------------------------------------------
def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); return them as fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32).reshape(x.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bf16 encodings of values that are already exactly representable in bf16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bf16-representable; call round_bf16 first")
    return (u >> 16).astype(np.uint16).reshape(x.shape)


def _storage(cfg: Config, x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return round_bf16(x) if cfg.dtype == "bf16" else np.ascontiguousarray(x)


# ----------------------------------------------------------------------------------------
# Draft graphs.  Nodes are numbered topologically: node 0 is the root, and the fold source
# (first parent) of node n is a node m < n.
# ----------------------------------------------------------------------------------------
def draft_graph(cfg: Config, rng: np.random.Generator) -> Tuple[np.ndarray, List[List[int]]]:
    """Return (fold_src[int32, N] with fold_src[0] = -1, parents list per node)."""
    n = cfg.num_nodes
    parents: List[List[int]] = [[] for _ in range(n)]
    if cfg.graph == "chain2":
        # 1 parent + 3 children "in a chain of depth 2": 0 -> 1 -> {2, 3}
        table = [-1, 0, 1, 1, 2, 2, 3, 3]
        if n > len(table):
            raise ValueError("chain2 graph defined for at most 8 nodes")
        for m in range(1, n):
            parents[m] = [table[m]]
    elif cfg.graph == "tree3":
        # 3-ary tree filled in level order: node m's parent is (m-1)//3.
        for m in range(1, n):
            parents[m] = [(m - 1) // 3]
    elif cfg.graph == "chain":
        for m in range(1, n):
            parents[m] = [m - 1]
    elif cfg.graph == "star":
        for m in range(1, n):
            parents[m] = [0]
    elif cfg.graph == "dag":
        # each node draws U{1,2,3} distinct parents among earlier nodes; the first one is
        # the fold source.
        for m in range(1, n):
            k = min(int(rng.integers(1, 4)), m)
            parents[m] = [int(p) for p in rng.choice(m, size=k, replace=False)]
    elif cfg.graph == "dag_deep":
        depth = np.zeros(n, dtype=np.int64)
        dmax = cfg.max_depth or 6
        for m in range(1, n):
            if m <= dmax:
                first = m - 1                     # one chain of full depth
            else:
                cand = np.flatnonzero(depth[:m] < dmax)
                first = int(rng.choice(cand))
            depth[m] = depth[first] + 1
            extra = int(rng.integers(0, 3))
            others = [p for p in range(m) if p != first]
            more = []
            if extra and others:
                more = [int(p) for p in rng.choice(others, size=min(extra, len(others)),
                                                   replace=False)]
            parents[m] = [first] + more
    else:
        raise ValueError(f"unknown graph kind {cfg.graph!r}")
    fold_src = np.array([-1] + [parents[m][0] for m in range(1, n)], dtype=np.int32)[:n]
    return fold_src, parents


def graph_depth(fold_src: np.ndarray) -> np.ndarray:
    """Depth of every node along first-parent edges."""
    depth = np.zeros(len(fold_src), dtype=np.int64)
    for m in range(1, len(fold_src)):
        depth[m] = depth[fold_src[m]] + 1
    return depth


# ----------------------------------------------------------------------------------------
# Hidden states at the layer input.
# ----------------------------------------------------------------------------------------
def hidden_states(cfg: Config, fold_src: np.ndarray, rng: np.random.Generator
                  ) -> Tuple[np.ndarray, List[np.ndarray]]:
    """Root ~ N(0,1); child = its fold source + N(0,1) at the revealed positions + ripple.

    Returns (H [N, B, d] fp32 before storage rounding, reveal sets)."""
    n, b, d = cfg.num_nodes, cfg.block, cfg.hidden
    H = np.empty((n, b, d), dtype=np.float32)
    H[0] = rng.standard_normal((b, d), dtype=np.float32)
    reveals: List[np.ndarray] = [np.zeros(0, dtype=np.int64)]
    pos = np.arange(b)
    lo, hi = cfg.reveal
    for m in range(1, n):
        k = min(int(rng.integers(lo, hi + 1)), b)
        rev = np.sort(rng.choice(b, size=k, replace=False))
        dist = np.min(np.abs(pos[:, None] - rev[None, :]), axis=1)
        sigma = (cfg.ripple_amp * np.exp(-dist / cfg.ripple_len)).astype(np.float32)
        sigma[rev] = 1.0
        noise = rng.standard_normal((b, d), dtype=np.float32) * sigma[:, None]
        H[m] = H[fold_src[m]] + noise
        reveals.append(rev)
    return H, reveals


# ----------------------------------------------------------------------------------------
# Weights and the shared prefix cache.
# ----------------------------------------------------------------------------------------
def make_layer_weights(cfg: Config, rng: np.random.Generator) -> Dict[str, np.ndarray]:
    """Row-major [out, in] linear weights ~ N(0, weight_std^2) (0.02 in the benchmark
    configurations); RMSNorm gains = 1.

    w_qkv rows are the Q heads, then the K heads, then the V heads; w_gate_up rows are
    the gate projection then the up projection."""
    d, f, dh = cfg.hidden, cfg.ffn, cfg.head_dim
    std = np.float32(cfg.weight_std)

    def lin(o, i):
        return _storage(cfg, rng.standard_normal((o, i), dtype=np.float32) * std)

    out = {
        "rms1": np.ones(d, dtype=np.float32),
        "w_qkv": lin(cfg.qkv_dim, d),
        "w_o": lin(d, cfg.n_q * dh),
        "rms2": np.ones(d, dtype=np.float32),
        "w_gate_up": lin(2 * f, d),
        "w_down": lin(d, f),
    }
    if cfg.qkv_bias:          # drawn last, so the other weights do not change
        out["b_qkv"] = _storage(cfg, rng.standard_normal(cfg.qkv_dim, dtype=np.float32) *
                                np.float32(0.1))
    return out


def prefix_cache(cfg: Config, rng: np.random.Generator, pad_tokens: int = 64) -> np.ndarray:
    """K|V-interleaved cache [P + pad, 2, n_kv, dh] ~ N(0, (0.02*sqrt(d))^2).

    The prefix is handed to the layer as a strided view of this cache (token stride
    2*n_kv*dh elements, head stride dh), never as per-branch copies."""
    p = cfg.prefix
    shape = (p + pad_tokens, 2, cfg.n_kv, cfg.head_dim)
    std = np.float32(0.02 * math.sqrt(cfg.hidden))
    return _storage(cfg, rng.standard_normal(shape, dtype=np.float32) * std)


@dataclasses.dataclass
class Workload:
    cfg: Config
    fold_src: np.ndarray              # int32 [N]
    parents: List[List[int]]
    reveals: List[np.ndarray]
    H: np.ndarray                     # fp32 [N, B, d] (bf16-exact for bf16 configs)
    weights: List[Dict[str, np.ndarray]]
    caches: List[np.ndarray]          # per layer: [P+pad, 2, n_kv, dh]

    @property
    def cache(self) -> np.ndarray:
        return self.caches[0]

    def prefix_kv(self, layer: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """(K, V) prefix views [P, n_kv, dh] of one layer's interleaved cache."""
        c = self.caches[layer]
        return c[: self.cfg.prefix, 0], c[: self.cfg.prefix, 1]


def _streams(cfg: Config):
    ss = np.random.SeedSequence(cfg.seed)
    return ss.spawn(4)          # graph, hidden, prefix caches, weights


def make_workload(cfg: Config, layers: Optional[int] = None, weights: bool = True
                  ) -> Workload:
    """Draw the whole workload of a configuration from its seed.

    `layers` (default cfg.layers) limits how many layers' weights and caches are drawn;
    layer l always gets the same values whatever the limit."""
    nl = cfg.layers if layers is None else layers
    s_graph, s_hidden, s_prefix, s_weights = _streams(cfg)
    fold_src, parents = draft_graph(cfg, np.random.Generator(np.random.PCG64(s_graph)))
    H, reveals = hidden_states(cfg, fold_src, np.random.Generator(np.random.PCG64(s_hidden)))
    H = _storage(cfg, H)
    caches = [prefix_cache(cfg, np.random.Generator(np.random.PCG64(c)))
              for c in s_prefix.spawn(nl)]
    ws: List[Dict[str, np.ndarray]] = []
    if weights:
        for ls in s_weights.spawn(nl):
            ws.append(make_layer_weights(cfg, np.random.Generator(np.random.PCG64(ls))))
    return Workload(cfg, fold_src, parents, reveals, H, ws, caches)


def layer_weights_of(cfg: Config, layer: int) -> Dict[str, np.ndarray]:
    """Weights of one layer, regenerated from the seed (keeps host memory bounded)."""
    ls = _streams(cfg)[3].spawn(layer + 1)[layer]
    return make_layer_weights(cfg, np.random.Generator(np.random.PCG64(ls)))


def layer_cache_of(cfg: Config, layer: int) -> np.ndarray:
    """Prefix cache of one layer, regenerated from the seed."""
    cs = _streams(cfg)[2].spawn(layer + 1)[layer]
    return prefix_cache(cfg, np.random.Generator(np.random.PCG64(cs)))


def iter_layers(cfg: Config, layers: Optional[int] = None, workers: int = 4):
    """Yield (layer, weights, prefix cache) for layers 0, 1, ... in order, drawing up to
    `workers` layers ahead on threads (numpy's generators release the GIL).  Every layer
    has its own sub-stream, so the values equal layer_weights_of / layer_cache_of."""
    nl = cfg.layers if layers is None else layers
    s_prefix, s_weights = _streams(cfg)[2:4]
    c_seeds, w_seeds = s_prefix.spawn(nl), s_weights.spawn(nl)

    def draw(l):
        w = make_layer_weights(cfg, np.random.Generator(np.random.PCG64(w_seeds[l])))
        c = prefix_cache(cfg, np.random.Generator(np.random.PCG64(c_seeds[l])))
        return l, w, c

    with concurrent.futures.ThreadPoolExecutor(max(1, workers)) as ex:
        pending = [ex.submit(draw, l) for l in range(min(nl, workers))]
        nxt = len(pending)
        while pending:
            res = pending.pop(0).result()
            if nxt < nl:
                pending.append(ex.submit(draw, nxt))
                nxt += 1
            yield res
