"""GPU: the per-channel-decay step (gdn_kda_decode_step, gdn_kda_decode_token)
against the oracle's oracle_run_kda.

Chained decode over several tokens, held to the decode bound (1e-4 normwise per
step's o and for the final state; the conv tail exactly), in the gate regimes
that push alpha to 1 or 0 and beta to 1 or 0; the fused token call equal bit
for bit to conv_update + kda_decode_step; equal per-channel gates against the
gated-delta-rule kernel (same math, products ordered differently); the
27B-class layer at batch 64, the launch with two row-quads per wave, every
sequence against the oracle; ragged shapes (d = 32, a 3:1 and an 8:1 group).
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from gdn_inputs import QWEN27B_LAYER, TINY, LayerShape
from tests.conftest import normwise

pytestmark = pytest.mark.gpu
TOL = 1e-4


def run_kda(inp, fused=False):
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import act_to_dev, act_to_host, dims_of, f32_to_dev, host
    shape, B, T = inp.shape, inp.batch, inp.steps
    assert inp.a.shape == (T, B, shape.num_v_heads, shape.head_k_dim)
    d = dims_of(shape, B)
    S = f32_to_dev(inp.state)
    w = act_to_dev(inp.w)
    x, a, b = act_to_dev(inp.x), f32_to_dev(inp.a), f32_to_dev(inp.b)
    o = torch.empty(T, B, shape.num_v_heads, shape.head_v_dim, device="cuda")
    if fused:
        tails = [act_to_dev(inp.tail), act_to_dev(inp.tail).fill_(0)]
        for t in range(T):
            gdn.kda_decode_token(d, S, tails[t % 2], tails[(t + 1) % 2], w, x[t], a[t], b[t], o[t])
        tail = tails[T % 2]
    else:
        tail = act_to_dev(inp.tail)
        y = torch.empty(B, shape.conv_channels, device="cuda")
        for t in range(T):
            gdn.conv_update(d, x[t], tail, w, y)
            gdn.kda_decode_step(d, S, y, a[t], b[t], o[t])
    torch.cuda.synchronize()
    return host(o), host(S), act_to_host(tail)


def check_against_oracle(inp, o, S, tail, seqs, what):
    for s in seqs:
        o_r, S_r, t_r = oracle.run_kda(inp.shape, inp.state[s], inp.tail[s], inp.w, inp.x[:, s], inp.a[:, s],
                                       inp.b[:, s])
        for t in range(inp.steps):
            err = normwise(o[t, s], o_r[t])
            assert err < TOL, f"{what} seq {s} step {t}: o error {err:.3e}"
        err = normwise(S[s], S_r)
        assert err < TOL, f"{what} seq {s}: state error {err:.3e}"
        assert np.array_equal(oracle.f64(tail[s]), t_r), f"{what} seq {s}: tail differs"


CASES = [
    ("tiny_f32", TINY, 3, 16),
    ("27b_b1", QWEN27B_LAYER, 1, 8),
    ("27b_b3", QWEN27B_LAYER, 3, 4),
    ("g8_b1", LayerShape(2, 16, 128, 128, 4, "bf16"), 1, 4),
    ("d32_bf16_b2", LayerShape(2, 6, 32, 32, 4, "bf16"), 2, 12),
]


@pytest.mark.parametrize("name,shape,batch,steps", CASES, ids=[c[0] for c in CASES])
def test_kda_step_matches_oracle(name, shape, batch, steps):
    inp = gi.kda_inputs(300, shape, batch, steps)
    o, S, tail = run_kda(inp)
    check_against_oracle(inp, o, S, tail, range(batch), name)


@pytest.mark.parametrize("gates", ["long_memory", "strong_decay", "beta_one", "beta_zero", "long_beta_one"])
def test_kda_gate_regimes(gates):
    inp = gi.kda_inputs(301, QWEN27B_LAYER, 2, 6, gates=gates)
    o, S, tail = run_kda(inp, fused=True)
    check_against_oracle(inp, o, S, tail, range(2), gates)


@pytest.mark.parametrize("name,shape,batch,steps", CASES + [("27b_b64", QWEN27B_LAYER, 64, 2)],
                         ids=[c[0] for c in CASES] + ["27b_b64"])
def test_kda_fused_equals_two_calls_bitwise(name, shape, batch, steps):
    inp = gi.kda_inputs(302, shape, batch, steps)
    o1, S1, t1 = run_kda(inp)
    o2, S2, t2 = run_kda(inp, fused=True)
    assert np.array_equal(o1.view(np.int32), o2.view(np.int32)), f"{name}: o differs"
    assert np.array_equal(S1.view(np.int32), S2.view(np.int32)), f"{name}: state differs"
    assert np.array_equal(t1, t2), f"{name}: tail differs"


def test_kda_batch64_full_size_every_sequence():
    """The 27B-class layer at batch 64 (two row-quads per wave), fused call, two tokens."""
    inp = gi.kda_inputs(303, QWEN27B_LAYER, 64, 2)
    o, S, tail = run_kda(inp, fused=True)
    check_against_oracle(inp, o, S, tail, range(64), "b64")


def test_equal_channel_gates_match_the_gated_delta_rule():
    """a[h][c] = a[h] for every channel: the variant's kernel and the gated-delta-rule
    kernel compute the same recurrence (to rounding)."""
    from tests.test_gpu_decode import run_gpu_decode
    inp = gi.decode_inputs(304, QWEN27B_LAYER, 2, 6)
    o_g, S_g, t_g = run_gpu_decode(inp)
    kda = gi.Inputs(inp.shape, inp.batch, inp.steps, inp.x,
                    np.repeat(inp.a[..., None], QWEN27B_LAYER.head_k_dim, axis=3), inp.b, inp.w, inp.state, inp.tail)
    o_k, S_k, t_k = run_kda(kda)
    assert normwise(o_k, o_g) < 1e-6 and normwise(S_k, S_g) < 1e-6
    assert np.array_equal(t_k, t_g)


def test_kda_rejects_aliased_tails():
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import act_to_dev, dims_of, f32_to_dev
    inp = gi.kda_inputs(305, QWEN27B_LAYER, 1, 1)
    d = dims_of(QWEN27B_LAYER, 1)
    S, tail, w = f32_to_dev(inp.state), act_to_dev(inp.tail), act_to_dev(inp.w)
    o = torch.empty(1, QWEN27B_LAYER.num_v_heads, QWEN27B_LAYER.head_v_dim, device="cuda")
    with pytest.raises(gdn.GdnError):
        gdn.kda_decode_token(d, S, tail, tail, w, act_to_dev(inp.x[0]), f32_to_dev(inp.a[0]), f32_to_dev(inp.b[0]),
                             o)
