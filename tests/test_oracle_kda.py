"""Pins of the oracle's per-channel-decay variant (oracle_run_kda, oracle_recur_kda).

The model-arch page names a Kimi Delta Attention mixer but does not define it;
the reading pinned here is the gated delta rule with its forget gate made one
value per key channel, applied to the state's key columns before the delta
correction.  The pins reach the oracle from outside: the scalar case against the
gated-delta-rule oracle (itself pinned in test_oracle_pins.py), a hand-worked
2x2 step, the beta = 0 closed form, a one-hot key, and an independent
brute-force formulation with explicit transition matrices
M_t = diag(alpha_t) (I - beta_t k_t k_t^T).
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
from tests.test_oracle_pins import np_conv_silu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_force_kda(shape, S0, y, a, b):
    """o_t and S_T from S_t = S_0 M_1...M_t + sum_{j<=t} beta_j v_j k_j^T M_{j+1}...M_t
    with M_j = diag(alpha_j) (I - beta_j k_j k_j^T), alpha_j a vector over key channels."""
    Hk, Hv, dk, dv = shape.num_k_heads, shape.num_v_heads, shape.head_k_dim, shape.head_v_dim
    G = Hv // Hk
    T = y.shape[0]
    q = y[:, : Hk * dk].reshape(T, Hk, dk)
    k = y[:, Hk * dk: 2 * Hk * dk].reshape(T, Hk, dk)
    v = y[:, 2 * Hk * dk:].reshape(T, Hv, dv)
    qn = np.repeat(q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + 1e-6), G, axis=1)
    kn = np.repeat(k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + 1e-6), G, axis=1)
    alpha = np.exp(-np.logaddexp(0.0, a.astype(np.float64)))     # [T][Hv][dk]
    beta = expit(b.astype(np.float64))
    o = np.zeros((T, Hv, dv))
    S_end = np.zeros((Hv, dv, dk))
    I = np.eye(dk)
    for h in range(Hv):
        M = [np.diag(alpha[t, h]) @ (I - beta[t, h] * np.outer(kn[t, h], kn[t, h])) for t in range(T)]
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


def test_hand_worked_2x2(oracle_lib):
    d = json.load(open(os.path.join(GOLDEN, "kda_2x2_hand.json")))
    shape = LayerShape(1, 1, 2, 2, 1, "f32")
    S0 = np.array(d["inputs"]["S0_rows_value_major"], dtype=np.float64)[None]
    y = np.array(d["inputs"]["y_q_then_k_then_v"])
    o, S = oracle.recur_kda(shape, S0, y, np.array(d["inputs"]["a_per_key_channel"]), np.array(d["inputs"]["b"]))
    tol = d["tolerance_rel"]
    np.testing.assert_allclose(S[0], np.array(d["expected"]["S_rows_value_major"]), rtol=tol, atol=0)
    np.testing.assert_allclose(o[0], np.array(d["expected"]["o"]), rtol=tol, atol=0)


@pytest.mark.parametrize("shape,T,seed", [(gi.TINY, 7, 0), (LayerShape(2, 6, 16, 8, 4, "bf16"), 5, 1)],
                         ids=["tiny", "grouped"])
def test_scalar_gates_equal_the_gated_delta_rule_bitwise(shape, T, seed, oracle_lib):
    """With every channel's gate input equal to the head's, the variant is the gated
    delta rule, operation for operation: outputs, state and tail agree bit for bit."""
    inp = gi.decode_inputs(seed, shape, 1, T, state_sigma=0.5)
    a_vec = np.repeat(inp.a[:, 0, :, None], shape.head_k_dim, axis=2)
    o_k, S_k, t_k = oracle.run_kda(shape, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0], a_vec, inp.b[:, 0])
    o_g, S_g, t_g = oracle.run(shape, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0], inp.a[:, 0], inp.b[:, 0])
    assert np.array_equal(o_k, o_g) and np.array_equal(S_k, S_g) and np.array_equal(t_k, t_g)


def test_beta_zero_decays_each_key_column_by_its_product(oracle_lib):
    """beta = 0 (b = -inf): S_T = S_0 diag(prod_t alpha_t), column by column, and
    o_t = S_0 diag(prod_{m<=t} alpha_m) q^_t / sqrt(dk)."""
    shape = LayerShape(2, 4, 16, 16, 4, "f32")
    T = 30
    inp = gi.kda_inputs(3, shape, 1, T, state_sigma=1.0)
    b = np.full((T, shape.num_v_heads), -np.inf, np.float32)
    o, S, _ = oracle.run_kda(shape, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0], inp.a[:, 0], b)
    loga = -np.logaddexp(0.0, inp.a[:, 0].astype(np.float64))        # [T][Hv][dk]
    cum = np.exp(np.cumsum(loga, axis=0))
    S0 = inp.state[0].astype(np.float64)
    ref = S0 * cum[-1][:, None, :]
    assert np.max(np.abs(S - ref) / np.abs(ref)) < 4 * T * 2.0**-52
    y = np_conv_silu(inp.tail[0], inp.w, inp.x[:, 0])
    Hk, dk = shape.num_k_heads, shape.head_k_dim
    q = y[:, : Hk * dk].reshape(T, Hk, dk)
    qn = np.repeat(q / np.sqrt((q * q).sum(-1, keepdims=True) + 1e-6), shape.group, axis=1)
    o_ref = np.stack([np.einsum("hik,hk->hi", S0 * cum[t][:, None, :], qn[t]) for t in range(T)]) / np.sqrt(dk)
    assert normwise(o, o_ref) < 1e-13


def test_one_hot_key_with_beta_one_writes_its_column_and_decays_the_rest(oracle_lib):
    """beta = 1 and k^ = e_j: column j becomes v (up to the norm's eps), whatever
    alpha_j is, and every other column c is alpha_c times its old value."""
    shape = LayerShape(1, 1, 8, 8, 1, "f32")
    rng = np.random.default_rng(5)
    S0 = rng.standard_normal((1, 8, 8))
    q = rng.standard_normal(8)
    v = rng.standard_normal(8)
    k = np.zeros(8)
    k[5] = 40.0
    a = rng.standard_normal((1, 8))
    o, S = oracle.recur_kda(shape, S0, np.concatenate([q, k, v]), a, np.array([np.inf]))
    alpha = 1.0 / (1.0 + np.exp(a[0]))
    other = [c for c in range(8) if c != 5]
    np.testing.assert_allclose(S[0][:, other], S0[0][:, other] * alpha[other], rtol=4e-16, atol=0)
    assert np.max(np.abs(S[0][:, 5] - v)) < 1e-8


@pytest.mark.parametrize("shape,T,seed", [
    (LayerShape(4, 4, 32, 32, 4, "f32"), 8, 0),
    (LayerShape(2, 6, 16, 8, 4, "bf16"), 9, 1),       # grouped 3:1, dk != dv
    (LayerShape(1, 2, 8, 12, 4, "bf16"), 10, 2),
])
@pytest.mark.parametrize("gates", ["normal", "long_memory", "beta_one"])
def test_against_brute_force_transition_products(shape, T, seed, gates, oracle_lib):
    inp = gi.kda_inputs(seed, shape, 1, T, state_sigma=0.5, gates=gates)
    o, S, _ = oracle.run_kda(shape, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0], inp.a[:, 0], inp.b[:, 0])
    y = np_conv_silu(inp.tail[0], inp.w, inp.x[:, 0])
    o_ref, S_ref = brute_force_kda(shape, inp.state[0].astype(np.float64), y, inp.a[:, 0], inp.b[:, 0])
    assert normwise(o, o_ref) < 1e-11
    assert normwise(S, S_ref) < 1e-11


def test_channels_are_not_interchangeable(oracle_lib):
    """Reversing the gate vector over key channels changes the result (the gate is
    tied to its key channel, not pooled over the head)."""
    shape = LayerShape(1, 1, 8, 8, 4, "f32")
    inp = gi.kda_inputs(9, shape, 1, 4, state_sigma=1.0)
    args = (shape, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0])
    o1, _, _ = oracle.run_kda(*args, inp.a[:, 0], inp.b[:, 0])
    o2, _, _ = oracle.run_kda(*args, inp.a[:, 0, :, ::-1], inp.b[:, 0])
    assert normwise(o1, o2) > 1e-3
