"""GPU parity of gdn_conv_update + gdn_decode_step against the CPU oracle.

Tolerance: the benchmark spec's bound for decode, max relative error 1e-4, taken
normwise per tensor (max |x - r| / max |r|) for each step's o and for the
state; the conv tail is data movement and must match exactly.
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


def run_gpu_decode(inp, steps=None, keep_o=True):
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import act_to_dev, act_to_host, dims_of, f32_to_dev, host
    shape, B = inp.shape, inp.batch
    T = inp.steps if steps is None else steps
    d = dims_of(shape, B)
    S = f32_to_dev(inp.state)
    tail = act_to_dev(inp.tail)
    w = act_to_dev(inp.w)
    x = act_to_dev(inp.x[:T])
    a = f32_to_dev(inp.a[:T])
    b = f32_to_dev(inp.b[:T])
    y = torch.empty(B, shape.conv_channels, device="cuda")
    o = torch.empty(T, B, shape.num_v_heads, shape.head_v_dim, device="cuda")
    for t in range(T):
        gdn.conv_update(d, x[t], tail, w, y)
        gdn.decode_step(d, S, y, a[t], b[t], o[t])
    torch.cuda.synchronize()
    return (host(o) if keep_o else None), host(S), act_to_host(tail)


def oracle_decode(inp, seqs, steps=None, h_range=None):
    T = inp.steps if steps is None else steps
    res = []
    for s in seqs:
        res.append(oracle.run(inp.shape, inp.state[s], inp.tail[s], inp.w, inp.x[:T, s], inp.a[:T, s],
                              inp.b[:T, s], h_range=h_range))
    return res


def check(o_gpu, S_gpu, tail_gpu, ref, seqs, h_range=None, shape=None):
    lo, hi = (0, shape.num_v_heads) if h_range is None else h_range
    for i, s in enumerate(seqs):
        o_r, S_r, t_r = ref[i]
        for t in range(o_r.shape[0]):
            err = normwise(o_gpu[t, s, lo:hi], o_r[t, lo:hi])
            assert err < TOL, f"seq {s} step {t}: o error {err:.3e}"
        err = normwise(S_gpu[s, lo:hi], S_r[lo:hi])
        assert err < TOL, f"seq {s}: state error {err:.3e}"
        assert np.array_equal(oracle.f64(tail_gpu[s]), t_r), f"seq {s}: conv tail differs"


def test_tiny_layer_64_steps():
    """The tiny layer: 4+4 heads of 32, fp32, 64 steps from a zero state and tail."""
    inp = gi.decode_inputs(0, TINY, 1, 64, state_sigma=0.0, tail_random=False)
    o, S, tail = run_gpu_decode(inp)
    check(o, S, tail, oracle_decode(inp, [0]), [0], shape=TINY)


def test_27b_layer_all_heads_64_steps():
    inp = gi.decode_inputs(1, QWEN27B_LAYER, 1, 64)
    o, S, tail = run_gpu_decode(inp)
    check(o, S, tail, oracle_decode(inp, [0]), [0], shape=QWEN27B_LAYER)


def test_27b_layer_4096_chained_steps_sampled_heads():
    """The full 4,096 chained steps; the oracle follows q/k head 0 and 15 (value
    heads 0-2 and 45-47) through every step."""
    inp = gi.decode_inputs(1, QWEN27B_LAYER, 1, 4096)
    o, S, tail = run_gpu_decode(inp)
    for hr in ((0, 3), (45, 48)):
        check(o, S, tail, oracle_decode(inp, [0], h_range=hr), [0], h_range=hr, shape=QWEN27B_LAYER)


@pytest.mark.parametrize("batch", [2, 5, 11])
def test_batched_ragged(batch):
    """Batch sizes that do and do not fill a launch evenly, both kernel variants."""
    inp = gi.decode_inputs(2 + batch, QWEN27B_LAYER, batch, 6)
    o, S, tail = run_gpu_decode(inp)
    check(o, S, tail, oracle_decode(inp, range(batch)), range(batch), shape=QWEN27B_LAYER)


def test_batch64_warmup_then_256_steps_sampled():
    """The batched workload: 64 sequences, 512 warm-up tokens then 256 steps, all
    through the library; the oracle replays all 768 tokens for sampled sequences
    and q/k heads from the same seeded start."""
    inp = gi.decode_inputs(2, QWEN27B_LAYER, 64, 768)
    o, S, tail = run_gpu_decode(inp)
    seqs = [0, 37, 63]
    for hr in ((0, 3), (24, 27)):
        check(o, S, tail, oracle_decode(inp, seqs, h_range=hr), seqs, h_range=hr, shape=QWEN27B_LAYER)


def test_tiny_layer_batched_bf16():
    shape = LayerShape(4, 8, 32, 32, 4, "bf16")
    inp = gi.decode_inputs(3, shape, 3, 20)
    o, S, tail = run_gpu_decode(inp)
    check(o, S, tail, oracle_decode(inp, range(3)), range(3), shape=shape)


def test_beta_zero_gpu_decays_state():
    """b = -100 gives beta = 0 in fp32; the state then only decays: S_T = (prod alpha) S_0."""
    inp = gi.decode_inputs(4, QWEN27B_LAYER, 1, 8)
    inp.b[:] = -100.0
    o, S, tail = run_gpu_decode(inp)
    loga = -np.logaddexp(0.0, inp.a[:, 0].astype(np.float64))
    ref = np.exp(loga.sum(0))[:, None, None] * inp.state[0]
    assert normwise(S[0], ref) < 4e-6


def test_deterministic_repeat():
    inp = gi.decode_inputs(5, QWEN27B_LAYER, 4, 8)
    r1 = run_gpu_decode(inp)
    r2 = run_gpu_decode(inp)
    for u, v in zip(r1, r2):
        assert np.array_equal(u, v)


def test_decode_allocates_nothing():
    """The state size is fixed: after warm-up, further steps allocate no device memory."""
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import act_to_dev, dims_of, f32_to_dev
    inp = gi.decode_inputs(6, QWEN27B_LAYER, 2, 4)
    d = dims_of(QWEN27B_LAYER, 2)
    S, tail, w = f32_to_dev(inp.state), act_to_dev(inp.tail), act_to_dev(inp.w)
    x, a, b = act_to_dev(inp.x), f32_to_dev(inp.a), f32_to_dev(inp.b)
    y = torch.empty(2, QWEN27B_LAYER.conv_channels, device="cuda")
    o = torch.empty(2, 48, 128, device="cuda")
    gdn.conv_update(d, x[0], tail, w, y)
    gdn.decode_step(d, S, y, a[0], b[0], o)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    for t in range(1, 4):
        for _ in range(50):
            gdn.conv_update(d, x[t], tail, w, y)
            gdn.decode_step(d, S, y, a[t], b[t], o)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == alloc0
    assert free1 == free0
