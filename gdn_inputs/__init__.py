"""Seeded synthetic inputs for one Gated DeltaNet layer.

Both sides of every parity check (the HIP library and the CPU oracle) draw
their inputs from here, so this module holds none of the method's
arithmetic: only random draws, rounding of draws to their storage type, and
draft-tree sampling.

Random numbers come from NumPy's Philox-4x64 counter-based generator.  A
tensor is drawn in fixed blocks of rows; block ``j`` of tensor ``stream``
under ``seed`` uses the key ``(seed, stream << 32 | j)`` with the counter
starting at zero, so any block can be regenerated on its own and the result
does not depend on how many threads draw it.

Shapes and distributions follow the workloads the serving-engine pages
describe for the 27B-class hybrid model: 48 value heads and 16 query/key
heads of width 128 ("Architecture", section 8.1 table: an fp32 state of 48
heads of 128 by 128 plus a 4-wide convolution tail of 80 KB), draft trees of
up to 32 nodes (repository "Architecture" page, decode-loop sequence
diagram), and long prompts.
"""
from __future__ import annotations

import concurrent.futures as _fut
import os
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "LayerShape", "TINY", "QWEN27B_LAYER", "normal_rows", "f32_to_bf16_bits",
    "bf16_bits_to_f32", "random_tree", "random_leaf_path", "tree_depths",
    "decode_inputs", "tree_inputs", "tree_batch_inputs", "prefill_inputs", "kda_inputs", "channel_gates", "Inputs",
    "GATE_REGIMES",
]

BF16 = "bf16"
F32 = "f32"


@dataclass(frozen=True)
class LayerShape:
    """Head counts and widths of one recurrent layer."""
    num_k_heads: int
    num_v_heads: int
    head_k_dim: int
    head_v_dim: int
    conv_width: int = 4
    act: str = BF16  # storage type of raw activations, conv tail and conv weights

    @property
    def conv_channels(self) -> int:
        return 2 * self.num_k_heads * self.head_k_dim + self.num_v_heads * self.head_v_dim

    @property
    def group(self) -> int:
        return self.num_v_heads // self.num_k_heads


# The tiny layer: 4 q/k heads and 4 v heads of width 32, fp32 activations.
TINY = LayerShape(4, 4, 32, 32, 4, F32)
# The 27B-class layer: 16 q/k heads shared 3:1 by 48 v heads, all of width 128.
QWEN27B_LAYER = LayerShape(16, 48, 128, 128, 4, BF16)

# Stream identifiers: one per tensor role, fixed forever.
S_X, S_A, S_B, S_W, S_STATE, S_TAIL, S_TREE, S_A_CHANNEL = 1, 2, 3, 4, 5, 6, 7, 8

_ROWS_PER_BLOCK = 64
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        _POOL = _fut.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))
    return _POOL


def _gen(seed: int, stream: int, block: int) -> np.random.Generator:
    key = np.array([seed & (2**64 - 1), ((stream << 32) | block) & (2**64 - 1)], dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key))


def normal_rows(seed: int, stream: int, nrows: int, rowlen: int, sigma: float = 1.0) -> np.ndarray:
    """float32 [nrows][rowlen] of N(0, sigma^2) draws (sigma is the standard deviation)."""
    out = np.empty((nrows, rowlen), dtype=np.float32)
    nblk = (nrows + _ROWS_PER_BLOCK - 1) // _ROWS_PER_BLOCK

    def fill(j):
        r0 = j * _ROWS_PER_BLOCK
        r1 = min(nrows, r0 + _ROWS_PER_BLOCK)
        g = _gen(seed, stream, j)
        out[r0:r1] = g.standard_normal((r1 - r0, rowlen), dtype=np.float32)
        if sigma != 1.0:
            out[r0:r1] *= np.float32(sigma)

    if nblk * rowlen * _ROWS_PER_BLOCK > 4_000_000:
        list(_pool().map(fill, range(nblk)))
    else:
        for j in range(nblk):
            fill(j)
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + r) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return out


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _act(x32: np.ndarray, act: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if act == BF16 else x32


# --------------------------------------------------------------------------- trees

def random_tree(rng: np.random.Generator, n: int, max_depth: int = 8) -> np.ndarray:
    """Draft tree as a parent array: node 0 is the root (parent -1); node i > 0 takes
    its parent uniformly among the earlier nodes whose depth (root = 1) is below
    max_depth, which is rejection sampling of a uniform parent in [0, i)."""
    parent = np.full(n, -1, dtype=np.int32)
    depth = np.ones(n, dtype=np.int32)
    for i in range(1, n):
        eligible = np.nonzero(depth[:i] < max_depth)[0]
        j = int(eligible[rng.integers(len(eligible))])
        parent[i] = j
        depth[i] = depth[j] + 1
    return parent


def tree_depths(parent: np.ndarray) -> np.ndarray:
    d = np.ones(len(parent), dtype=np.int32)
    for i in range(1, len(parent)):
        d[i] = d[parent[i]] + 1
    return d


def path_to(parent: np.ndarray, node: int) -> np.ndarray:
    p = []
    while node >= 0:
        p.append(node)
        node = int(parent[node])
    return np.array(p[::-1], dtype=np.int32)


def random_leaf_path(rng: np.random.Generator, parent: np.ndarray) -> np.ndarray:
    """Root-first path to a leaf chosen uniformly among the leaves."""
    n = len(parent)
    has_child = np.zeros(n, dtype=bool)
    has_child[parent[parent >= 0]] = True
    leaves = np.nonzero(~has_child)[0]
    return path_to(parent, int(leaves[rng.integers(len(leaves))]))


# --------------------------------------------------------------------------- workloads

@dataclass
class Inputs:
    shape: LayerShape
    batch: int
    steps: int
    x: np.ndarray          # [steps][batch][C] act storage (uint16 bf16 bits or float32)
    a: np.ndarray          # [steps][batch][Hv] float32
    b: np.ndarray          # [steps][batch][Hv] float32
    w: np.ndarray          # [C][W] act storage
    state: np.ndarray      # [batch][Hv][dv][dk] float32
    tail: np.ndarray       # [batch][C][W] act storage, oldest to newest
    extra: dict = field(default_factory=dict)


# Gate regimes: the means of the gate inputs a and b (each drawn as mean + N(0,1)).
# The pages' workloads draw both from N(0,1) ("normal": median alpha = beta = 1/2,
# so the state forgets within a few tokens); the others push each gate to an end
# of its range, where chunked and tree forms round differently from token order:
#   long_memory   a ~ N(-6,1): alpha close to 1, the state remembers for thousands of tokens
#   strong_decay  a ~ N(+6,1): alpha close to 0, products of gates underflow within a chunk
#   beta_one      b ~ N(+6,1): beta close to 1, each key's old value is fully replaced
#   beta_zero     b ~ N(-6,1): beta close to 0, writes almost vanish
#   long_beta_one long memory and beta close to 1 together
GATE_REGIMES = {
    "normal": (0.0, 0.0),
    "long_memory": (-6.0, 0.0),
    "strong_decay": (6.0, 0.0),
    "beta_one": (0.0, 6.0),
    "beta_zero": (0.0, -6.0),
    "long_beta_one": (-6.0, 6.0),
}


def _common(seed, shape, batch, steps, state_sigma, tail_random, gates="normal"):
    C, W = shape.conv_channels, shape.conv_width
    Hv, dk, dv = shape.num_v_heads, shape.head_k_dim, shape.head_v_dim
    a_mean, b_mean = GATE_REGIMES[gates]
    x = _act(normal_rows(seed, S_X, steps * batch, C), shape.act).reshape(steps, batch, C)
    a = normal_rows(seed, S_A, steps * batch, Hv).reshape(steps, batch, Hv)
    b = normal_rows(seed, S_B, steps * batch, Hv).reshape(steps, batch, Hv)
    if a_mean:
        a += np.float32(a_mean)
    if b_mean:
        b += np.float32(b_mean)
    w = _act(normal_rows(seed, S_W, C, W, sigma=0.5), shape.act)
    if state_sigma:
        state = normal_rows(seed, S_STATE, batch * Hv * dv, dk, sigma=state_sigma).reshape(batch, Hv, dv, dk)
    else:
        state = np.zeros((batch, Hv, dv, dk), dtype=np.float32)
    if tail_random:
        tail = _act(normal_rows(seed, S_TAIL, batch * C, W), shape.act).reshape(batch, C, W)
    else:
        tail = _act(np.zeros((batch * C, W), dtype=np.float32), shape.act).reshape(batch, C, W)
    return x, a, b, w, state, tail


def decode_inputs(seed: int, shape: LayerShape, batch: int, steps: int,
                  state_sigma: float = 0.1, tail_random: bool = True, gates: str = "normal") -> Inputs:
    """Chained decode: `steps` tokens per sequence, q|k|v raw activations ~ N(0,1),
    gate inputs a, b ~ N(0,1) shifted per the gate regime, conv weights ~ N(0, 0.5^2),
    state ~ N(0, state_sigma^2)."""
    x, a, b, w, state, tail = _common(seed, shape, batch, steps, state_sigma, tail_random, gates)
    return Inputs(shape, batch, steps, x, a, b, w, state, tail)


def tree_inputs(seed: int, shape: LayerShape, n_nodes: int = 32, max_depth: int = 8,
                state_sigma: float = 0.1, tail_random: bool = True, gates: str = "normal") -> Inputs:
    """One draft tree of n_nodes over a batch-1 checkpoint; x/a/b hold one row per node."""
    x, a, b, w, state, tail = _common(seed, shape, 1, n_nodes, state_sigma, tail_random, gates)
    rng = _gen(seed, S_TREE, 0)
    parent = random_tree(rng, n_nodes, max_depth)
    path = random_leaf_path(rng, parent)
    return Inputs(shape, 1, n_nodes, x, a, b, w, state, tail,
                  extra={"parent": parent, "path": path, "max_depth": max_depth})


def tree_batch_inputs(seed: int, shape: LayerShape, batch: int, n_nodes: int = 32, max_depth: int = 8,
                      state_sigma: float = 0.1, tail_random: bool = True, gates: str = "normal") -> Inputs:
    """One draft tree of n_nodes per sequence over `batch` checkpoints; x/a/b hold one row
    per (node, sequence), [n_nodes][batch][...].  extra["parent"] is [batch][n_nodes] (an
    independent tree per sequence); extra["path"] is [batch][max_depth]: per row a
    root-first prefix of the path to a uniformly chosen leaf, of uniform length between 1
    and that path's length, padded with -1."""
    x, a, b, w, state, tail = _common(seed, shape, batch, n_nodes, state_sigma, tail_random, gates)
    parent = np.empty((batch, n_nodes), dtype=np.int32)
    path = np.full((batch, max_depth), -1, dtype=np.int32)
    for s in range(batch):
        rng = _gen(seed, S_TREE, 1 + s)
        parent[s] = random_tree(rng, n_nodes, max_depth)
        full = random_leaf_path(rng, parent[s])
        keep = 1 + int(rng.integers(len(full)))
        path[s, :keep] = full[:keep]
    return Inputs(shape, batch, n_nodes, x, a, b, w, state, tail,
                  extra={"parent": parent, "path": path, "max_depth": max_depth})


def prefill_inputs(seed: int, shape: LayerShape, T: int, batch: int = 1,
                   state_sigma: float = 0.0, tail_random: bool = False, gates: str = "normal") -> Inputs:
    """A prompt of T tokens; by default from a fresh (zero) state and zero conv tail."""
    x, a, b, w, state, tail = _common(seed, shape, batch, T, state_sigma, tail_random, gates)
    return Inputs(shape, batch, T, x, a, b, w, state, tail)


def kda_inputs(seed: int, shape: LayerShape, batch: int, steps: int, state_sigma: float = 0.1,
               tail_random: bool = True, gates: str = "normal") -> Inputs:
    """Chained decode with a per-channel forget gate: as decode_inputs, except that a is
    [steps][batch][Hv][dk], one gate input per (value head, key channel), each drawn
    from N(0,1) shifted by the regime's mean (its own stream, so a and b keep their
    meaning in every regime)."""
    x, _, b, w, state, tail = _common(seed, shape, batch, steps, state_sigma, tail_random, gates)
    a = channel_gates(seed, shape, batch, steps, gates)
    return Inputs(shape, batch, steps, x, a, b, w, state, tail)


def channel_gates(seed: int, shape: LayerShape, batch: int, steps: int, gates: str = "normal") -> np.ndarray:
    """The per-channel gate inputs of kda_inputs alone: [steps][batch][Hv][dk] float32."""
    Hv, dk = shape.num_v_heads, shape.head_k_dim
    a_mean, _ = GATE_REGIMES[gates]
    a = normal_rows(seed, S_A_CHANNEL, steps * batch * Hv, dk).reshape(steps, batch, Hv, dk)
    if a_mean:
        a += np.float32(a_mean)
    return a
