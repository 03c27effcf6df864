"""Pins of the CPU oracle to things other than itself.

The pages print no worked values for this recurrence, so the pins are: a
hand-derived example, closed forms, invariants, library routines for the
pieces that have one, and an independent brute-force formulation (explicit
products of transition matrices).  A plausible slip in the oracle (a dropped
term, a sign, decay on the wrong side of the correction, a transposed state,
a wrong q/k head for a value head, an off-by-one conv window) fails at least
one test here.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import expit

import gdn_inputs as gi
import oracle
from gdn_inputs import LayerShape
from tests.conftest import normwise

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ independent pieces

def np_conv_silu(tail0, w, x):
    """Causal depthwise conv by np.convolve over the whole sequence (history = tail0)
    followed by SiLU written as z * expit(z)."""
    tail0 = oracle.f64(tail0)
    w = oracle.f64(w)
    x = oracle.f64(x)
    Cc, W = tail0.shape
    T = x.shape[0]
    y = np.empty((T, Cc))
    for c in range(Cc):
        seq = np.concatenate([tail0[c, 1:], x[:, c]])  # the newest W-1 of the old window, then x
        z = np.convolve(seq, w[c, ::-1], mode="valid")
        y[:, c] = z * expit(z)
    return y


def brute_force(shape, S0, y, a, b):
    """o_t for all t from the unrolled recurrence with explicit transition matrices:
    S_t = S_0 M_1...M_t + sum_{j<=t} beta_j v_j k_j^T M_{j+1}...M_t,
    M_j = alpha_j (I - beta_j k_j k_j^T).  Heads are split by reshape; value head h
    uses q/k head h // G (np.repeat)."""
    Hk, Hv, dk, dv = shape.num_k_heads, shape.num_v_heads, shape.head_k_dim, shape.head_v_dim
    G = Hv // Hk
    T = y.shape[0]
    q = y[:, : Hk * dk].reshape(T, Hk, dk)
    k = y[:, Hk * dk: 2 * Hk * dk].reshape(T, Hk, dk)
    v = y[:, 2 * Hk * dk:].reshape(T, Hv, dv)
    qn = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + 1e-6)
    kn = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + 1e-6)
    qn = np.repeat(qn, G, axis=1)
    kn = np.repeat(kn, G, axis=1)
    alpha = np.exp(-np.logaddexp(0.0, a.astype(np.float64)))
    beta = expit(b.astype(np.float64))
    o = np.zeros((T, Hv, dv))
    S_end = np.zeros((Hv, dv, dk))
    I = np.eye(dk)
    for h in range(Hv):
        M = [alpha[t, h] * (I - beta[t, h] * np.outer(kn[t, h], kn[t, h])) for t in range(T)]
        for t in range(T):
            P = np.eye(dk)
            for j in range(t + 1):
                P = P @ M[j]
            St = S0[h] @ P
            for j in range(t + 1):
                Pj = np.eye(dk)
                for m in range(j + 1, t + 1):
                    Pj = Pj @ M[m]
                St = St + beta[j, h] * np.outer(v[j, h], kn[j, h]) @ Pj
            o[t, h] = St @ qn[t, h] / np.sqrt(dk)
            if t == T - 1:
                S_end[h] = St
    return o, S_end


# ------------------------------------------------------------------ storage

def test_bf16_widening_exhaustive(oracle_lib):
    """All 65,536 bf16 patterns widen exactly (the CPU page checks its 16-bit convert
    exhaustively; here the independent routine is NumPy's float32 bit view)."""
    h = np.arange(65536, dtype=np.uint16)
    got = oracle.widen(h)
    ref = (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint64), ref[~nan].view(np.uint64))


def test_batched_tree_draws_are_valid():
    """Every sequence of a batched draw has its own valid tree (parents earlier, depth at
    most 8, checked by the oracle's tree tables), and each path row is a root-first chain
    of that tree followed by -1 only; the draw mixes path lengths."""
    inp = gi.tree_batch_inputs(11, gi.TINY, 16, n_nodes=32, max_depth=8)
    parent, path = inp.extra["parent"], inp.extra["path"]
    assert parent.shape == (16, 32) and path.shape == (16, 8)
    assert inp.x.shape == (32, 16, gi.TINY.conv_channels)
    lens = []
    for s in range(16):
        st, depth, _ = oracle.tree_tables(parent[s], 8)
        assert st == 0 and depth.max() <= 8
        row = path[s]
        L = int(np.argmax(row == -1)) if (row == -1).any() else len(row)
        assert L >= 1 and (row[L:] == -1).all() and row[0] == 0
        assert all(parent[s][row[j]] == row[j - 1] for j in range(1, L))
        lens.append(L)
    assert len(set(lens)) > 2
    assert len({tuple(p) for p in parent}) == 16


def test_input_bf16_rounding_ties_and_sample():
    """The generator's fp32 -> bf16 rounding against an independent round-half-even
    written with integer division, on edge patterns and a large random sample."""
    rng = np.random.default_rng(5)
    u = np.concatenate([
        rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32),
        np.array([0x3F808000, 0x3F818000, 0x3F80_7FFF, 0x3F80_8001, 0x7F7F_FFFF, 0x0000_8000,
                  0x0001_8000, 0x8000_8000, 0x7F80_0000, 0xFF80_0000], dtype=np.uint32),
    ])
    u = u[((u & 0x7FFFFFFF) <= 0x7F800000)]  # drop NaN payloads
    got = gi.f32_to_bf16_bits(u.view(np.float32))
    q, r = np.divmod(u.astype(np.uint64), np.uint64(65536))
    up = (r > 32768) | ((r == 32768) & (q % 2 == 1))
    ref = (q + up.astype(np.uint64)).astype(np.uint16)
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------ conv

@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_conv_matches_direct_convolution(act, oracle_lib):
    shape = LayerShape(2, 2, 8, 8, 4, act)
    inp = gi.decode_inputs(11, shape, 1, 20)
    y, tail = oracle.conv(inp.tail[0], inp.w, inp.x[:, 0])
    ref = np_conv_silu(inp.tail[0], inp.w, inp.x[:, 0])
    assert normwise(y, ref) < 1e-14
    # the tail is the last W raw inputs, oldest first: pure data movement, exact
    assert np.array_equal(tail, oracle.f64(inp.x[-4:, 0]).T)


def test_conv_identity_tap_is_silu(oracle_lib):
    Cc, W, T = 16, 4, 5
    w = np.zeros((Cc, W), dtype=np.float32)
    w[:, W - 1] = 1.0
    x = gi.normal_rows(3, 1, T, Cc) * 3
    y, _ = oracle.conv(np.zeros((Cc, W), np.float32), w, x)
    xd = x.astype(np.float64)
    assert normwise(y, xd * expit(xd)) < 1e-15


def test_conv_window_is_causal_with_history(oracle_lib):
    """A single unit impulse at token 0 in tap position j reaches y at token W-1-j only."""
    Cc, W, T = 4, 4, 8
    for j in range(W):
        w = np.zeros((Cc, W), np.float32)
        w[:, j] = 1.0
        x = np.zeros((T, Cc), np.float32)
        x[0] = 2.0
        y, _ = oracle.conv(np.zeros((Cc, W), np.float32), w, x)
        hit = np.nonzero(np.abs(y[:, 0]) > 0)[0]
        assert list(hit) == [W - 1 - j]


# ------------------------------------------------------------------ the recurrence

def test_hand_worked_2x2():
    d = json.load(open(os.path.join(GOLDEN, "recurrence_2x2_hand.json")))
    shape = LayerShape(1, 1, 2, 2, 1, "f32")
    S0 = np.array(d["inputs"]["S0_rows_value_major"], dtype=np.float64)[None]
    y = np.array(d["inputs"]["y_q_then_k_then_v"])
    o, S = oracle.recur(shape, S0, y, np.array(d["inputs"]["a"]), np.array(d["inputs"]["b"]))
    tol = d["tolerance_rel"]
    np.testing.assert_allclose(S[0], np.array(d["expected"]["S_rows_value_major"]), rtol=tol, atol=0)
    np.testing.assert_allclose(o[0], np.array(d["expected"]["o"]), rtol=tol, atol=0)


@pytest.mark.parametrize("shape,T,seed", [
    (LayerShape(4, 4, 32, 32, 4, "f32"), 12, 0),      # the tiny layer's dims
    (LayerShape(2, 6, 16, 8, 4, "bf16"), 10, 1),      # grouped 3:1, dk != dv
    (LayerShape(1, 2, 8, 12, 4, "bf16"), 9, 2),
])
def test_against_brute_force_transition_products(shape, T, seed, oracle_lib):
    inp = gi.decode_inputs(seed, shape, 1, T, state_sigma=0.5)
    o, S, _ = oracle.run(shape, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0], inp.a[:, 0], inp.b[:, 0])
    y = np_conv_silu(inp.tail[0], inp.w, inp.x[:, 0])
    o_ref, S_ref = brute_force(shape, inp.state[0].astype(np.float64), y, inp.a[:, 0], inp.b[:, 0])
    assert normwise(o, o_ref) < 1e-11
    assert normwise(S, S_ref) < 1e-11


def test_beta_zero_decays_by_product_of_alphas(oracle_lib):
    """beta = 0 (b = -1000): S_T = (prod alpha) S_0 and o_t = s (prod_{m<=t} alpha) S_0 q^_t."""
    shape = LayerShape(2, 4, 16, 16, 4, "f32")
    T = 40
    inp = gi.decode_inputs(7, shape, 1, T, state_sigma=1.0)
    b = np.full((T, shape.num_v_heads), -1000.0, np.float32)
    o, S, _ = oracle.run(shape, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0], inp.a[:, 0], b)
    loga = -np.logaddexp(0.0, inp.a[:, 0].astype(np.float64))         # [T][Hv]
    cum = np.exp(np.cumsum(loga, axis=0))
    S0 = inp.state[0].astype(np.float64)
    ref = cum[-1][:, None, None] * S0
    assert np.max(np.abs(S - ref) / np.abs(ref)) < 4 * T * 2.0**-52
    y = np_conv_silu(inp.tail[0], inp.w, inp.x[:, 0])
    Hk, dk = shape.num_k_heads, shape.head_k_dim
    q = y[:, : Hk * dk].reshape(T, Hk, dk)
    qn = np.repeat(q / np.sqrt((q * q).sum(-1, keepdims=True) + 1e-6), shape.group, axis=1)
    o_ref = cum[:, :, None] * np.einsum("hik,thk->thi", S0, qn) / np.sqrt(dk)
    assert normwise(o, o_ref) < 1e-13


def test_alpha_one_beta_one_retrieves_value(oracle_lib):
    """alpha = beta = 1: after the update S k^ = v up to the eps in the norm; a
    one-hot key changes only its own column, the other columns stay bit for bit."""
    shape = LayerShape(1, 1, 8, 8, 1, "f32")
    rng = np.random.default_rng(1)
    S0 = rng.standard_normal((1, 8, 8))
    for t in range(3):
        q = rng.standard_normal(8)
        k = 30.0 * rng.standard_normal(8)
        v = rng.standard_normal(8)
        o, S = oracle.recur(shape, S0, np.concatenate([q, k, v]), np.array([-1000.0]), np.array([1000.0]))
        kn = k / np.linalg.norm(k)
        assert np.max(np.abs(S[0] @ kn - v)) < 1e-8
        S0 = S
    k = np.zeros(8)
    k[3] = 50.0
    o, S = oracle.recur(shape, S0, np.concatenate([q, k, v]), np.array([-1000.0]), np.array([1000.0]))
    other = [c for c in range(8) if c != 3]
    assert np.array_equal(S[0][:, other], S0[0][:, other])
    assert np.max(np.abs(S[0][:, 3] - v)) < 1e-8


def test_first_token_from_zero_state_closed_form(oracle_lib):
    """T = 1 from S = 0: o = s * beta * v * (k^ . q^)."""
    shape = LayerShape(2, 4, 16, 16, 1, "f32")
    rng = np.random.default_rng(2)
    y = rng.standard_normal(shape.conv_channels)
    a = rng.standard_normal(4)
    b = rng.standard_normal(4)
    o, _ = oracle.recur(shape, np.zeros((4, 16, 16)), y, a, b)
    for h in range(4):
        g = h // 2
        q = y[g * 16:(g + 1) * 16]
        k = y[32 + g * 16: 32 + (g + 1) * 16]
        v = y[64 + h * 16: 64 + (h + 1) * 16]
        kq = (q @ k) / np.sqrt((q @ q + 1e-6) * (k @ k + 1e-6))
        np.testing.assert_allclose(o[h], expit(b[h]) * v * kq / 4.0, rtol=1e-13, atol=1e-15)


def test_value_head_reads_its_own_qk_group(oracle_lib):
    """Value heads h use q/k head h // (Hv/Hk): changing q/k of head 1 moves value
    heads 2 and 3 only, and changing v of head 2 moves head 2 only."""
    shape = LayerShape(2, 4, 8, 8, 1, "f32")
    rng = np.random.default_rng(3)
    S0 = rng.standard_normal((4, 8, 8))
    y = rng.standard_normal(shape.conv_channels)
    a, b = rng.standard_normal(4), rng.standard_normal(4)
    o0, S0n = oracle.recur(shape, S0, y, a, b)
    y1 = y.copy()
    y1[8:16] += 1.0       # q of q/k head 1
    y1[16 + 8:32] -= 0.5  # k of q/k head 1
    o1, S1n = oracle.recur(shape, S0, y1, a, b)
    assert np.array_equal(o0[:2], o1[:2]) and np.array_equal(S0n[:2], S1n[:2])
    assert not np.any(o0[2:] == o1[2:])
    y2 = y.copy()
    y2[32 + 2 * 8 + 5] += 1.0  # v row 5 of value head 2
    o2, S2n = oracle.recur(shape, S0, y2, a, b)
    for h in (0, 1, 3):
        assert np.array_equal(S2n[h], S0n[h])
    assert not np.array_equal(S2n[2][5], S0n[2][5])
    assert np.array_equal(np.delete(S2n[2], 5, axis=0), np.delete(S0n[2], 5, axis=0))


def test_state_size_is_independent_of_T(oracle_lib):
    shape = LayerShape(2, 2, 8, 8, 4, "f32")
    for T in (1, 7, 64):
        inp = gi.decode_inputs(1, shape, 1, T)
        _, S, tail = oracle.run(shape, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0], inp.a[:, 0], inp.b[:, 0])
        assert S.shape == (2, 8, 8) and tail.shape == (shape.conv_channels, 4)


def test_head_range_matches_full_run(oracle_lib):
    """Running a subset of value heads gives those heads' full-run values exactly,
    and the tail advances on every channel either way."""
    shape = LayerShape(2, 6, 16, 16, 4, "bf16")
    inp = gi.decode_inputs(4, shape, 1, 6)
    o, S, t = oracle.run(shape, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0], inp.a[:, 0], inp.b[:, 0])
    o2, S2, t2 = oracle.run(shape, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0], inp.a[:, 0], inp.b[:, 0],
                            h_range=(3, 5))
    assert np.array_equal(o[:, 3:5], o2[:, 3:5]) and np.array_equal(S[3:5], S2[3:5])
    assert np.array_equal(t, t2)


# ------------------------------------------------------------------ trees and paths

def _py_preorder(parent):
    """Pre-order by sorting root-first ancestor paths lexicographically."""
    def key(i):
        p = []
        while i >= 0:
            p.append(i)
            i = parent[i]
        return p[::-1]
    return sorted(range(len(parent)), key=key)


def test_tree_tables_against_brute_force(oracle_lib):
    rng = np.random.default_rng(9)
    for n in (1, 2, 5, 17, 32):
        for _ in range(20):
            parent = gi.random_tree(rng, n, 8)
            rc, depth, order = oracle.tree_tables(parent)
            assert rc == oracle.OK
            assert np.array_equal(depth, gi.tree_depths(parent))
            assert list(order) == _py_preorder(list(parent))
            assert depth.max() <= 8


@pytest.mark.parametrize("parent", [
    [0, 0],            # root must have parent -1
    [-1, 1],           # parent must be earlier
    [-1, 0, 3, 1],     # forward reference
    [-1, -1],          # two roots
    list(range(-1, 8)),  # chain of 9 nodes: depth 9 > 8
])
def test_tree_tables_reject_invalid(parent, oracle_lib):
    rc, _, _ = oracle.tree_tables(np.array(parent, np.int32), 8)
    assert rc == oracle.ERR_TREE


@pytest.fixture(scope="module")
def small_tree_case():
    shape = LayerShape(2, 4, 16, 16, 4, "bf16")
    inp = gi.tree_inputs(21, shape, n_nodes=12, max_depth=8)
    return shape, inp


def test_chain_tree_equals_sequential(oracle_lib):
    shape = LayerShape(2, 4, 16, 16, 4, "bf16")
    inp = gi.tree_inputs(22, shape, n_nodes=8)
    parent = np.arange(-1, 7, dtype=np.int32)
    o_tree = oracle.tree_verify(shape, inp.state[0], inp.tail[0], inp.w, parent, inp.x[:, 0], inp.a[:, 0], inp.b[:, 0])
    o_seq, _, _ = oracle.run(shape, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0], inp.a[:, 0], inp.b[:, 0])
    assert np.array_equal(o_tree, o_seq)


def test_star_tree_children_are_one_step_from_root(oracle_lib):
    shape = LayerShape(2, 4, 16, 16, 4, "bf16")
    inp = gi.tree_inputs(23, shape, n_nodes=6)
    parent = np.array([-1, 0, 0, 0, 0, 0], np.int32)
    o_tree = oracle.tree_verify(shape, inp.state[0], inp.tail[0], inp.w, parent, inp.x[:, 0], inp.a[:, 0], inp.b[:, 0])
    _, S_root, t_root = oracle.run(shape, inp.state[0], inp.tail[0], inp.w, inp.x[:1, 0], inp.a[:1, 0], inp.b[:1, 0])
    for n in range(1, 6):
        o1, _, _ = oracle.run(shape, S_root, t_root, inp.w, inp.x[n:n + 1, 0], inp.a[n:n + 1, 0], inp.b[n:n + 1, 0])
        assert np.array_equal(o_tree[n], o1[0])


def test_identical_siblings_give_identical_outputs(oracle_lib):
    shape = LayerShape(2, 4, 16, 16, 4, "bf16")
    inp = gi.tree_inputs(24, shape, n_nodes=5)
    parent = np.array([-1, 0, 1, 1, 0], np.int32)
    x = inp.x[:, 0].copy(); a = inp.a[:, 0].copy(); b = inp.b[:, 0].copy()
    x[3], a[3], b[3] = x[2], a[2], b[2]
    o = oracle.tree_verify(shape, inp.state[0], inp.tail[0], inp.w, parent, x, a, b)
    assert np.array_equal(o[2], o[3])
    assert not np.array_equal(o[2], o[4])


def test_tree_equals_commit_on_every_path(small_tree_case, oracle_lib):
    """Replaying a root-first path from the checkpoint (commit) gives, at its last
    node, the output the tree pass gives for that node."""
    shape, inp = small_tree_case
    parent = inp.extra["parent"]
    o_tree = oracle.tree_verify(shape, inp.state[0], inp.tail[0], inp.w, parent, inp.x[:, 0], inp.a[:, 0], inp.b[:, 0])
    for node in range(len(parent)):
        path = gi.path_to(parent, node)
        o_c, _, _ = oracle.commit_path(shape, inp.state[0], inp.tail[0], inp.w, parent, inp.x[:, 0],
                                       inp.a[:, 0], inp.b[:, 0], path)
        assert np.array_equal(o_c[-1], o_tree[node])


def test_commit_equals_sequential_decode_of_path(small_tree_case, oracle_lib):
    shape, inp = small_tree_case
    parent, path = inp.extra["parent"], inp.extra["path"]
    o_c, S_c, t_c = oracle.commit_path(shape, inp.state[0], inp.tail[0], inp.w, parent, inp.x[:, 0],
                                       inp.a[:, 0], inp.b[:, 0], path)
    o_s, S_s, t_s = oracle.run(shape, inp.state[0], inp.tail[0], inp.w, inp.x[path, 0], inp.a[path, 0], inp.b[path, 0])
    assert np.array_equal(S_c, S_s) and np.array_equal(t_c, t_s) and np.array_equal(o_c, o_s)
    # the tail after a commit is the last four raw inputs of (old tail ++ path)
    hist = np.concatenate([oracle.f64(inp.tail[0]).T, oracle.f64(inp.x[path, 0])])
    assert np.array_equal(t_c, hist[-4:].T)


@pytest.mark.parametrize("kind", ["not_from_root", "repeated_node", "skips_a_level", "past_the_tree"])
def test_commit_rejects_non_paths(kind, small_tree_case, oracle_lib):
    shape, inp = small_tree_case
    parent = inp.extra["parent"].copy()
    n = len(parent)
    if kind == "not_from_root":
        bad = [1]
    elif kind == "repeated_node":
        bad = [0, 0]
    elif kind == "skips_a_level":
        k = next(i for i in range(1, n) if parent[i] != 0)   # a node that is not a child of the root
        bad = [0, k]
    else:
        bad = [0, n]
    bad = np.array(bad, np.int32)
    with pytest.raises(oracle.OracleError) as e:
        oracle.commit_path(shape, inp.state[0], inp.tail[0], inp.w, parent, inp.x[:, 0], inp.a[:, 0],
                           inp.b[:, 0], bad)
    assert e.value.rc == oracle.ERR_TREE
