"""The chunked (WY / UT) form of the recurrence, in fp64 NumPy, against the
sequential oracle.

The CPU page ("Serving a research architecture on CPU", exactness section)
notes that the recurrence is computed in parallel over chunks at training time
and one token at a time at decode time, and that the two are algebraically the
same while rounding differently.  The HIP prefill uses the chunk form; this
test checks that algebra in fp64 before any GPU rounding enters, with chunk
sizes that do and do not divide T.

Derivation (per value head; S is [dv][dk], rows over values).  Write the
recurrence as S_t = alpha_t S_{t-1} + u_t k_t^T with
u_t = beta_t (v_t - alpha_t S_{t-1} k_t).  Inside a chunk that starts from S0,
with gamma_t = prod_{m<=t} alpha_m,
    S_t = gamma_t S0 + sum_{j<=t} (gamma_t / gamma_j) u_j k_j^T.
Substituting into u_t gives (I + A) U = diag(beta) V - diag(beta gamma) K S0^T
with A_tj = beta_t (gamma_t / gamma_j) k_t.k_j for j < t.  With
Tm = (I + A)^-1:  U = Tm diag(beta) V - Tm diag(beta gamma) K S0^T,
    O  = s [diag(gamma) Q S0^T + (P (.) mask_incl) U],  P_tj = (gamma_t/gamma_j) q_t.k_j,
    S_n = gamma_n S0 + U^T diag(gamma_n / gamma_j) K.
Only gamma ratios with t >= j are ever formed (as exp of differences of the
cumulative log-decay), so nothing overflows.
"""
import numpy as np
import pytest
from scipy.special import expit

import gdn_inputs as gi
import oracle
from gdn_inputs import LayerShape
from tests.conftest import normwise
from tests.test_oracle_pins import np_conv_silu


def chunked(shape, S0, y, a, b, chunk):
    Hk, Hv, dk, dv = shape.num_k_heads, shape.num_v_heads, shape.head_k_dim, shape.head_v_dim
    G = Hv // Hk
    T = y.shape[0]
    q = y[:, : Hk * dk].reshape(T, Hk, dk)
    k = y[:, Hk * dk: 2 * Hk * dk].reshape(T, Hk, dk)
    v = y[:, 2 * Hk * dk:].reshape(T, Hv, dv)
    q = q / np.sqrt((q * q).sum(-1, keepdims=True) + 1e-6)
    k = k / np.sqrt((k * k).sum(-1, keepdims=True) + 1e-6)
    loga = -np.logaddexp(0.0, a.astype(np.float64))
    beta = expit(b.astype(np.float64))
    s = 1.0 / np.sqrt(dk)
    S = S0.astype(np.float64).copy()
    O = np.zeros((T, Hv, dv))
    for h in range(Hv):
        g = h // G
        for c0 in range(0, T, chunk):
            c1 = min(T, c0 + chunk)
            n = c1 - c0
            Q, K, V = q[c0:c1, g], k[c0:c1, g], v[c0:c1, h]
            Gc = np.cumsum(loga[c0:c1, h])
            be = beta[c0:c1, h]
            diff = Gc[:, None] - Gc[None, :]
            lower = np.tril(np.ones((n, n), bool), -1)
            incl = np.tril(np.ones((n, n), bool), 0)
            ratio = np.where(incl, np.exp(np.where(incl, diff, 0.0)), 0.0)
            A = np.where(lower, be[:, None] * ratio * (K @ K.T), 0.0)
            Tm = np.linalg.solve(np.eye(n) + A, np.eye(n))
            Ut = Tm @ (be[:, None] * V)
            Wt = Tm @ ((be * np.exp(Gc))[:, None] * K)
            U = Ut - Wt @ S[h].T
            P = np.where(incl, ratio * (Q @ K.T), 0.0)
            O[c0:c1, h] = s * (np.exp(Gc)[:, None] * (Q @ S[h].T) + P @ U)
            S[h] = np.exp(Gc[-1]) * S[h] + U.T @ (np.exp(Gc[-1] - Gc)[:, None] * K)
    return O, S


@pytest.mark.parametrize("T,chunk", [(37, 8), (64, 16), (50, 64), (130, 64), (1, 64)])
def test_chunk_form_equals_sequential(T, chunk, oracle_lib):
    shape = LayerShape(2, 6, 16, 16, 4, "bf16")
    inp = gi.prefill_inputs(31, shape, T, state_sigma=0.3, tail_random=True)
    o, S, _ = oracle.run(shape, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0], inp.a[:, 0], inp.b[:, 0])
    y = np_conv_silu(inp.tail[0], inp.w, inp.x[:, 0])
    O2, S2 = chunked(shape, inp.state[0], y, inp.a[:, 0], inp.b[:, 0], chunk)
    assert normwise(O2, o) < 1e-12
    assert normwise(S2, S) < 1e-12


def test_chunk_form_strong_decay_does_not_overflow(oracle_lib):
    """Gate inputs a ~ 6: log alpha ~ -6 per token, about -380 over a chunk of 64,
    so exp(-G_j) alone would overflow; ratios with t >= j stay in range."""
    shape = LayerShape(1, 1, 16, 16, 4, "f32")
    T = 128
    inp = gi.prefill_inputs(32, shape, T, state_sigma=0.3)
    a = inp.a[:, 0] * 0.1 + 6.0
    o, S, _ = oracle.run(shape, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0], a, inp.b[:, 0])
    y = np_conv_silu(inp.tail[0], inp.w, inp.x[:, 0])
    with np.errstate(over="raise"):
        O2, S2 = chunked(shape, inp.state[0], y, a, inp.b[:, 0], 64)
    assert normwise(O2, o) < 1e-12
    assert np.all(np.isfinite(S2))
