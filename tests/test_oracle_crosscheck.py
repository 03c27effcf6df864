"""The oracle against an independent implementation of the gated delta rule.

transformers ships plain PyTorch versions of the recurrence for its Qwen3-Next
model, token by token and chunked (torch_recurrent_gated_delta_rule,
torch_chunk_gated_delta_rule).  They are written by other people, against the
published method, in fp32: agreement to fp32 rounding pins the readings the
pages leave open (decay before the delta correction, the output read from the
updated state, the q/k L2 norm with eps 1e-6 after the conv, the 1/sqrt(dk)
output scale, value head h reading q/k head h // (Hv/Hk)) to something other
than this repository.  Their conventions are mapped here: log-decay
g = -softplus(a), beta = sigmoid(b), state [dk][dv] per head (ours [dv][dk]).
The conv is taken from np.convolve (test_oracle_pins.np_conv_silu), not from
the oracle.  Test infrastructure only; transformers never enters the library.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from gdn_inputs import LayerShape
from tests.conftest import normwise
from tests.test_oracle_pins import np_conv_silu

qwen3_next = pytest.importorskip("transformers.models.qwen3_next.modeling_qwen3_next")

TOL = 2e-6   # fp32 arithmetic on their side (measured 0.9-4.1e-7), T up to 130 steps


def their_inputs(inp, seq=0):
    shape = inp.shape
    Hk, Hv, dk, dv = shape.num_k_heads, shape.num_v_heads, shape.head_k_dim, shape.head_v_dim
    G = Hv // Hk
    y = np_conv_silu(inp.tail[seq], inp.w, inp.x[:, seq])            # [T][C] fp64
    T = y.shape[0]
    q = np.repeat(y[:, : Hk * dk].reshape(T, Hk, dk), G, axis=1)
    k = np.repeat(y[:, Hk * dk: 2 * Hk * dk].reshape(T, Hk, dk), G, axis=1)
    v = y[:, 2 * Hk * dk:].reshape(T, Hv, dv)
    a = inp.a[:, seq].astype(np.float64)
    b = inp.b[:, seq].astype(np.float64)
    g = -np.logaddexp(0.0, a)                                        # log alpha = -softplus(a)
    beta = 1.0 / (1.0 + np.exp(-b))
    t = lambda arr: torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))[None]
    S0 = torch.from_numpy(np.ascontiguousarray(np.swapaxes(inp.state[seq], 1, 2), dtype=np.float32))[None]
    return t(q), t(k), t(v), t(g), t(beta), S0


@pytest.mark.parametrize("shape,T,seed", [
    (gi.TINY, 40, 0),
    (LayerShape(2, 6, 16, 8, 4, "bf16"), 33, 1),          # grouped 3:1, dk != dv
    (LayerShape(4, 12, 128, 128, 4, "bf16"), 12, 2),      # the 27B layer's head width and grouping
])
@pytest.mark.parametrize("gates", ["normal", "long_memory", "beta_one"])
def test_oracle_matches_the_recurrent_form(shape, T, seed, gates):
    inp = gi.decode_inputs(seed, shape, 1, T, state_sigma=0.3, gates=gates)
    o, S, _ = oracle.run(shape, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0], inp.a[:, 0], inp.b[:, 0])
    q, k, v, g, beta, S0 = their_inputs(inp)
    o_t, S_t = qwen3_next.torch_recurrent_gated_delta_rule(q, k, v, g, beta, S0, True, use_qk_l2norm_in_kernel=True)
    assert normwise(o, o_t[0].double().numpy()) < TOL
    assert normwise(S, np.swapaxes(S_t[0].double().numpy(), 1, 2)) < TOL


@pytest.mark.parametrize("T", [1, 64, 130])
def test_oracle_matches_the_chunked_form(T):
    """Their chunked (WY) form, 64-token chunks, a ragged last chunk."""
    shape = LayerShape(2, 6, 32, 32, 4, "bf16")
    inp = gi.decode_inputs(7, shape, 1, T, state_sigma=0.3)
    o, S, _ = oracle.run(shape, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0], inp.a[:, 0], inp.b[:, 0])
    q, k, v, g, beta, S0 = their_inputs(inp)
    o_t, S_t = qwen3_next.torch_chunk_gated_delta_rule(q, k, v, g, beta, chunk_size=64, initial_state=S0,
                                                       output_final_state=True, use_qk_l2norm_in_kernel=True)
    assert normwise(o, o_t[0].double().numpy()) < TOL
    assert normwise(S, np.swapaxes(S_t[0].double().numpy(), 1, 2)) < TOL


def test_a_misread_convention_is_detected():
    """Decay applied after the correction (the other plausible reading) disagrees
    with their form far beyond the tolerance: the comparison can tell readings apart."""
    shape = gi.TINY
    inp = gi.decode_inputs(3, shape, 1, 16, state_sigma=0.3)
    q, k, v, g, beta, S0 = their_inputs(inp)
    o_t, _ = qwen3_next.torch_recurrent_gated_delta_rule(q, k, v, g, beta, S0, True, use_qk_l2norm_in_kernel=True)
    # the other reading, S <- alpha (S + beta (v - S k) k^T), written out here in fp64
    qn = q[0].double() / torch.sqrt((q[0].double() ** 2).sum(-1, keepdim=True) + 1e-6)
    kn = k[0].double() / torch.sqrt((k[0].double() ** 2).sum(-1, keepdim=True) + 1e-6)
    S = S0[0].double().clone()                                         # [H][dk][dv]
    outs = []
    for t in range(16):
        al = torch.exp(g[0, t].double())[:, None, None]
        kv = torch.einsum("hkv,hk->hv", S, kn[t])
        S = al * (S + kn[t][:, :, None] * ((v[0, t].double() - kv) * beta[0, t].double()[:, None])[:, None, :])
        outs.append(torch.einsum("hkv,hk->hv", S, qn[t]) / np.sqrt(shape.head_k_dim))
    other = torch.stack(outs).numpy()
    assert normwise(other, o_t[0].double().numpy()) > 100 * TOL
