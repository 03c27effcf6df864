"""The UT form of tree verify, in fp64 NumPy, against the oracle's per-node
path replay.

This is the algebra the HIP UT-form verify follows, checked before any GPU
rounding enters.  It is the chunked form (test_chunk_algebra.py) with "j is i
or an ancestor of i" in place of "j <= i in the chunk".  Per value head, with
rho(i, j) the product of the gates alpha over the path (j, i], gamma_i the
product over the whole root-first path to i, and j <= i the ancestor order:
    A[j][l] = beta_j rho(j, l) k_j.k_l        (l a strict ancestor of j)
    M[i][j] = rho(i, j) q_i.k_j               (j <= i)
    R = M (I + A)^-1 diag(beta)
    e_i = gamma_i q_i - sum_l R[i][l] gamma_l k_l
    o_i = s (S_c e_i + sum_l R[i][l] v_l)
Nodes are in index order, every parent before its children, so A is strictly
lower triangular.  The gate products are formed by multiplication along each
path, never by division, so a gate that underflows to 0 gives 0, not NaN.
"""
import numpy as np
import pytest
from scipy.special import expit

import gdn_inputs as gi
import oracle
from gdn_inputs import LayerShape
from tests.conftest import normwise
from tests.test_oracle_pins import np_conv_silu


def node_conv(tail, w, x, parent):
    """y [n][C]: node i's conv output over the tail and its root-first path."""
    n = len(parent)
    return np.stack([np_conv_silu(tail, w, x[gi.path_to(parent, i)])[-1] for i in range(n)])


def tree_ut(shape, S0, y, a, b, parent):
    Hk, Hv, dk, dv = shape.num_k_heads, shape.num_v_heads, shape.head_k_dim, shape.head_v_dim
    G = Hv // Hk
    n = len(parent)
    q = y[:, : Hk * dk].reshape(n, Hk, dk)
    k = y[:, Hk * dk: 2 * Hk * dk].reshape(n, Hk, dk)
    v = y[:, 2 * Hk * dk:].reshape(n, Hv, dv)
    q = q / np.sqrt((q * q).sum(-1, keepdims=True) + 1e-6)
    k = k / np.sqrt((k * k).sum(-1, keepdims=True) + 1e-6)
    alpha = expit(-a.astype(np.float64))        # exp(-softplus(a))
    beta = expit(b.astype(np.float64))
    s = 1.0 / np.sqrt(dk)
    O = np.zeros((n, Hv, dv))
    for h in range(Hv):
        g = h // G
        rho = np.zeros((n, n))
        gam = np.zeros(n)
        for i in range(n):
            prod, cur = 1.0, i
            while cur >= 0:
                rho[i, cur] = prod
                prod *= alpha[cur, h]
                cur = parent[cur]
            gam[i] = prod
        Q, K, V = q[:, g], k[:, g], v[:, h]
        A = beta[:, h][:, None] * rho * (K @ K.T)
        np.fill_diagonal(A, 0.0)
        M = rho * (Q @ K.T)
        R = M @ np.linalg.inv(np.eye(n) + A) * beta[:, h][None, :]
        E = gam[:, None] * Q - R @ (gam[:, None] * K)
        O[:, h] = s * (E @ S0[h].T + R @ V)
    return O


def chain(n):
    return np.arange(-1, n - 1, dtype=np.int32)


@pytest.mark.parametrize("n,max_depth,chainlike", [(32, 8, False), (17, 8, False), (32, 3, False), (1, 8, False),
                                                   (32, 32, True), (5, 5, True)])
def test_tree_ut_form_equals_path_replay(n, max_depth, chainlike, oracle_lib):
    shape = LayerShape(2, 6, 16, 16, 4, "bf16")
    inp = gi.tree_inputs(41 + n + max_depth, shape, n, max_depth=max_depth, state_sigma=0.3)
    parent = chain(n) if chainlike else inp.extra["parent"]
    md = n if chainlike else max_depth
    x, a, b = inp.x[:, 0], inp.a[:, 0], inp.b[:, 0]
    o = oracle.tree_verify(shape, inp.state[0], inp.tail[0], inp.w, parent, x, a, b, max_depth=md)
    O2 = tree_ut(shape, oracle.f64(inp.state[0]), node_conv(inp.tail[0], inp.w, x, parent), a, b, parent)
    assert normwise(O2, o) < 1e-12


def test_tree_ut_form_gates_that_underflow(oracle_lib):
    """Gate inputs near 800 give alpha = exp(-800), which is 0 in fp64: a path through
    such a node forgets everything above it, and no ratio of gate products is formed, so
    the form gives exactly what the replay gives, with no 0/0."""
    shape = LayerShape(1, 2, 16, 16, 4, "f32")
    inp = gi.tree_inputs(47, shape, 24, max_depth=8, state_sigma=0.3)
    parent = inp.extra["parent"]
    a = inp.a[:, 0].astype(np.float64)
    a[::3] = 800.0
    a = a.astype(np.float32)
    x, b = inp.x[:, 0], inp.b[:, 0]
    o = oracle.tree_verify(shape, inp.state[0], inp.tail[0], inp.w, parent, x, a, b)
    with np.errstate(invalid="raise"):
        O2 = tree_ut(shape, oracle.f64(inp.state[0]), node_conv(inp.tail[0], inp.w, x, parent), a, b, parent)
    assert np.all(np.isfinite(O2))
    assert normwise(O2, o) < 1e-12
