"""The oracle split over host threads by q/k head group equals the oracle run
on all heads at once, bit for bit: each value head keeps its own token order,
so the split only changes which thread runs it."""
import numpy as np

import gdn_inputs as gi
import oracle
from gdn_inputs import LayerShape


def test_run_parallel_equals_run_bitwise(oracle_lib):
    shape = LayerShape(4, 12, 32, 32, 4, "bf16")
    inp = gi.prefill_inputs(31, shape, 50, state_sigma=0.1, tail_random=True, gates="long_memory")
    o1, S1, t1 = oracle.run(shape, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0], inp.a[:, 0], inp.b[:, 0])
    for threads in (1, 3, 4):
        o2, S2, t2 = oracle.run_parallel(shape, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0], inp.a[:, 0],
                                         inp.b[:, 0], threads=threads)
        assert np.array_equal(o1, o2) and np.array_equal(S1, S2) and np.array_equal(t1, t2)
    _, S3, t3 = oracle.run_parallel(shape, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0], inp.a[:, 0], inp.b[:, 0],
                                    want_o=False, threads=2)
    assert np.array_equal(S1, S3) and np.array_equal(t1, t3)


def test_gate_regimes_shift_only_the_gate_inputs():
    """A regime moves the mean of a or b and nothing else: the other tensors are the
    same draws, and the shift is exact in float32."""
    shape = LayerShape(2, 4, 32, 32, 4, "f32")
    base = gi.decode_inputs(5, shape, 2, 7)
    for name, (ma, mb) in gi.GATE_REGIMES.items():
        r = gi.decode_inputs(5, shape, 2, 7, gates=name)
        assert np.array_equal(r.x, base.x) and np.array_equal(r.state, base.state)
        assert np.array_equal(r.a, base.a + np.float32(ma))
        assert np.array_equal(r.b, base.b + np.float32(mb))
