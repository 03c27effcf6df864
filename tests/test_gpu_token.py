"""GPU: the fused token call (gdn_decode_token) against the two-call path and the
oracle.

The fused call must give, bit for bit, what gdn_conv_update + gdn_decode_step
give (state, per-step o, conv tail), with the tail ping-ponging between two
buffers; against the CPU oracle it is held to the decode bound (1e-4
normwise), and the tail exactly.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from gdn_inputs import QWEN27B_LAYER, TINY, LayerShape
from tests.conftest import normwise
from tests.test_gpu_decode import run_gpu_decode

pytestmark = pytest.mark.gpu
TOL = 1e-4


def run_gpu_token(inp, steps=None):
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import act_to_dev, act_to_host, dims_of, f32_to_dev, host
    shape, B = inp.shape, inp.batch
    T = inp.steps if steps is None else steps
    d = dims_of(shape, B)
    S = f32_to_dev(inp.state)
    tails = [act_to_dev(inp.tail), act_to_dev(inp.tail).fill_(0)]
    w = act_to_dev(inp.w)
    x, a, b = act_to_dev(inp.x[:T]), f32_to_dev(inp.a[:T]), f32_to_dev(inp.b[:T])
    o = torch.empty(T, B, shape.num_v_heads, shape.head_v_dim, device="cuda")
    for t in range(T):
        gdn.decode_token(d, S, tails[t % 2], tails[(t + 1) % 2], w, x[t], a[t], b[t], o[t])
    torch.cuda.synchronize()
    return host(o), host(S), act_to_host(tails[T % 2])


CASES = [
    ("tiny_f32", TINY, 1, 64),
    ("27b_b1", QWEN27B_LAYER, 1, 24),
    ("27b_b5", QWEN27B_LAYER, 5, 6),
    ("27b_b64", QWEN27B_LAYER, 64, 4),          # two row-quads per wave
    ("tiny_bf16_b3", LayerShape(4, 8, 32, 32, 4, "bf16"), 3, 12),
    ("27b_f32_b2", LayerShape(16, 48, 128, 128, 4, "f32"), 2, 5),
    ("g8_b1", LayerShape(2, 16, 128, 128, 4, "bf16"), 1, 5),
]


@pytest.mark.parametrize("name,shape,batch,steps", CASES, ids=[c[0] for c in CASES])
def test_fused_equals_two_calls_bitwise(name, shape, batch, steps):
    inp = gi.decode_inputs(70, shape, batch, steps)
    o1, S1, t1 = run_gpu_decode(inp)
    o2, S2, t2 = run_gpu_token(inp)
    assert np.array_equal(o1.view(np.int32), o2.view(np.int32)), f"{name}: o differs"
    assert np.array_equal(S1.view(np.int32), S2.view(np.int32)), f"{name}: state differs"
    assert np.array_equal(t1, t2), f"{name}: tail differs"


def test_fused_matches_oracle_27b_all_heads():
    inp = gi.decode_inputs(71, QWEN27B_LAYER, 2, 16)
    o, S, tail = run_gpu_token(inp)
    for s in range(2):
        o_r, S_r, t_r = oracle.run(QWEN27B_LAYER, inp.state[s], inp.tail[s], inp.w, inp.x[:, s], inp.a[:, s],
                                   inp.b[:, s])
        for t in range(16):
            err = normwise(o[t, s], o_r[t])
            assert err < TOL, f"seq {s} step {t}: o error {err:.3e}"
        assert normwise(S[s], S_r) < TOL
        assert np.array_equal(oracle.f64(tail[s]), t_r)


def test_fused_leaves_tail_in_untouched():
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import act_to_dev, dims_of, f32_to_dev
    inp = gi.decode_inputs(72, QWEN27B_LAYER, 3, 1)
    d = dims_of(QWEN27B_LAYER, 3)
    S, tin, w = f32_to_dev(inp.state), act_to_dev(inp.tail), act_to_dev(inp.w)
    tout = torch.zeros_like(tin)
    keep = tin.clone()
    o = torch.empty(3, 48, 128, device="cuda")
    gdn.decode_token(d, S, tin, tout, w, act_to_dev(inp.x[0]), f32_to_dev(inp.a[0]), f32_to_dev(inp.b[0]), o)
    torch.cuda.synchronize()
    assert torch.equal(tin, keep)
    with pytest.raises(gdn.GdnError):
        gdn.decode_token(d, S, tin, tin, w, act_to_dev(inp.x[0]), f32_to_dev(inp.a[0]), f32_to_dev(inp.b[0]), o)


def test_fused_4096_chained_steps_sampled_heads():
    """The timed workload's launch configuration: 4,096 chained fused steps at
    batch 1; the oracle follows q/k heads 0 and 15 (value heads 0-2, 45-47)."""
    inp = gi.decode_inputs(73, QWEN27B_LAYER, 1, 4096)
    o, S, tail = run_gpu_token(inp)
    for lo, hi in ((0, 3), (45, 48)):
        o_r, S_r, t_r = oracle.run(QWEN27B_LAYER, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0], inp.a[:, 0],
                                   inp.b[:, 0], h_range=(lo, hi))
        for t in range(4096):
            err = normwise(o[t, 0, lo:hi], o_r[t, lo:hi])
            assert err < TOL, f"heads {lo}-{hi} step {t}: o error {err:.3e}"
        assert normwise(S[0, lo:hi], S_r[lo:hi]) < TOL
        assert np.array_equal(oracle.f64(tail[0]), t_r)


def test_fused_batch64_256_steps_sampled():
    """Batch 64, the two-row-quad launch, 256 chained fused steps; sampled
    sequences and q/k heads against the oracle."""
    inp = gi.decode_inputs(74, QWEN27B_LAYER, 64, 256)
    o, S, tail = run_gpu_token(inp)
    for s in (0, 29, 63):
        for lo, hi in ((0, 3), (24, 27)):
            o_r, S_r, t_r = oracle.run(QWEN27B_LAYER, inp.state[s], inp.tail[s], inp.w, inp.x[:, s], inp.a[:, s],
                                       inp.b[:, s], h_range=(lo, hi))
            for t in range(256):
                err = normwise(o[t, s, lo:hi], o_r[t, lo:hi])
                assert err < TOL, f"seq {s} heads {lo}-{hi} step {t}: o error {err:.3e}"
            assert normwise(S[s, lo:hi], S_r[lo:hi]) < TOL
            assert np.array_equal(oracle.f64(tail[s]), t_r)
