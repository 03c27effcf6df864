"""GPU snapshot and restore of sequences' recurrent state (state and conv tail).

Byte work, so everything is bit-exact: a restored sequence equals the saved
one, decode continues from a restored state exactly as it would have without
the round trip, and refused restores write nothing.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_inputs import QWEN27B_LAYER, TINY

pytestmark = pytest.mark.gpu

OK, ERR_SIGNATURE, ERR_INDEX = 0, 9, 10


def same_bits(u, v):
    return torch.equal(u.contiguous().view(torch.int32), v.contiguous().view(torch.int32))


def case(shape, B, seed):
    from tests.gpu_util import act_to_dev, dims_of, f32_to_dev
    inp = gi.decode_inputs(seed, shape, B, 6, state_sigma=0.1, tail_random=True)
    return inp, dims_of(shape, B), f32_to_dev(inp.state), act_to_dev(inp.tail)


def snap(d, S, T, seqs):
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import i32_to_dev
    blob = torch.zeros(gdn.snapshot_bytes(d, len(seqs)), dtype=torch.uint8, device="cuda")
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    gdn.snapshot(d, S, T, i32_to_dev(np.array(seqs, np.int32)), blob, st)
    torch.cuda.synchronize()
    return blob, int(st.item())


def rest(d, S, T, seqs, blob):
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import i32_to_dev
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    gdn.restore(d, S, T, i32_to_dev(np.array(seqs, np.int32)), blob, st)
    torch.cuda.synchronize()
    return int(st.item())


@pytest.mark.parametrize("shape", [QWEN27B_LAYER, TINY], ids=["27b", "tiny"])
def test_round_trip_moves_each_sequence_bitwise(shape):
    import gated_deltanet_decode_amd as gdn
    inp, d, S, T = case(shape, 5, 90)
    blob, st = snap(d, S, T, [3, 0, 4, 3])
    assert st == OK
    # header: magic, version, signature, count, per-sequence section sizes, zeros
    h = blob[:256].cpu().numpy()
    u32, u64 = h.view(np.uint32), h.view(np.uint64)
    sb = shape.num_v_heads * shape.head_v_dim * shape.head_k_dim * 4
    tb = shape.conv_channels * 4 * (2 if shape.act == "bf16" else 4)
    assert u32[0] == 0x534E4447 and u32[1] == 1 and u64[1] == gdn.state_signature(d)
    assert u32[4] == 4 and u32[5] == 0 and u64[3] == sb and u64[4] == tb
    assert not h[40:].any()
    # the sections: states of slots 0..3, then their tails
    body = blob[256:]
    st_sec = body[:4 * sb].view(torch.float32).view(4, *S.shape[1:])
    tl_sec = body[4 * sb:4 * sb + 4 * tb].view(T.dtype).view(4, *T.shape[1:])
    for slot, q in enumerate([3, 0, 4, 3]):
        assert same_bits(st_sec[slot], S[q]) and torch.equal(tl_sec[slot].view(torch.int16), T[q].view(torch.int16))
    # restore slots 0..2 into other positions of a zeroed batch
    S2, T2 = torch.zeros_like(S), torch.zeros_like(T)
    blob3, st = snap(d, S, T, [3, 0, 4])
    assert st == OK
    assert rest(d, S2, T2, [1, 2, 0], blob3) == OK
    for dst, src in ((1, 3), (2, 0), (0, 4)):
        assert same_bits(S2[dst], S[src]) and torch.equal(T2[dst].view(torch.int16), T[src].view(torch.int16))
    assert not S2[3:].any() and not T2[3:].view(torch.int16).any()


def test_restore_then_decode_equals_uninterrupted_decode():
    """Save, run other tokens over the state (another request), restore, decode: the result
    is bit-identical to decoding straight from the saved state."""
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import act_to_dev, f32_to_dev
    inp, d, S0, T0 = case(QWEN27B_LAYER, 2, 91)
    x, a, b, w = act_to_dev(inp.x), f32_to_dev(inp.a), f32_to_dev(inp.b), act_to_dev(inp.w)
    o = torch.empty(2, 48, 128, device="cuda")

    def run(S, T, t0, t1):
        bufs = [T, torch.empty_like(T)]
        outs = []
        for i, t in enumerate(range(t0, t1)):
            gdn.decode_token(d, S, bufs[i % 2], bufs[1 - i % 2], w, x[t], a[t], b[t], o)
            outs.append(o.clone())
        torch.cuda.synchronize()
        return bufs[(t1 - t0) % 2], outs

    Sa, Ta = S0.clone(), T0.clone()
    Ta, outs_a = run(Sa, Ta, 3, 6)
    Sb, Tb = S0.clone(), T0.clone()
    blob, st = snap(d, Sb, Tb, [0, 1])
    assert st == OK
    Tb, _ = run(Sb, Tb, 0, 3)            # the state moves on
    assert not same_bits(Sb, S0)
    assert rest(d, Sb, Tb, [0, 1], blob) == OK
    assert same_bits(Sb, S0) and torch.equal(Tb, T0)
    Tb, outs_b = run(Sb, Tb, 3, 6)
    assert same_bits(Sb, Sa) and torch.equal(Tb, Ta)
    assert all(same_bits(p, q) for p, q in zip(outs_a, outs_b))


def test_restore_refuses_another_layer_shape_and_count():
    """A snapshot of the 27B-class layer restored as the tiny layer (the blob is large enough,
    so only the signature can refuse it), a count that differs from the saved one, and a
    corrupted header: each sets the status and writes nothing."""
    inp, d, S, T = case(QWEN27B_LAYER, 3, 92)
    blob, st = snap(d, S, T, [0, 1, 2])
    assert st == OK
    _, dt, St, Tt = case(TINY, 3, 93)
    St0, Tt0 = St.clone(), Tt.clone()
    assert rest(dt, St, Tt, [0, 1, 2], blob) == ERR_SIGNATURE
    assert same_bits(St, St0) and torch.equal(Tt, Tt0)
    S2, T2 = torch.zeros_like(S), torch.zeros_like(T)
    assert rest(d, S2, T2, [0, 1], blob) == ERR_SIGNATURE          # saved 3, restoring 2
    bad = blob.clone()
    bad[8] ^= 1                                                     # one bit of the signature
    assert rest(d, S2, T2, [0, 1, 2], bad) == ERR_SIGNATURE
    assert not S2.any() and not T2.view(torch.int16).any()
    assert rest(d, S2, T2, [0, 1, 2], blob) == OK and same_bits(S2, S)


def test_bad_sequence_lists():
    inp, d, S, T = case(TINY, 4, 94)
    blob, st = snap(d, S, T, [0, 4])                               # 4 is past the batch
    assert st == ERR_INDEX
    assert blob[:4].view(torch.int32).item() == 0                   # a refused snapshot has magic 0
    S2, T2 = torch.zeros_like(S), torch.zeros_like(T)
    assert rest(d, S2, T2, [0, 1], blob) == ERR_SIGNATURE
    good, st = snap(d, S, T, [1, 2])
    assert st == OK
    assert rest(d, S2, T2, [3, 3], good) == ERR_INDEX               # repeated target
    assert rest(d, S2, T2, [-1, 0], good) == ERR_INDEX
    assert not S2.any()


def test_batch64_full_size():
    """The 27B-class layer at 64 sequences (the launch the snapshot row times): all 64 saved
    and restored in reverse order."""
    inp, d, S, T = case(QWEN27B_LAYER, 64, 95)
    blob, st = snap(d, S, T, list(range(64)))
    assert st == OK
    S2, T2 = torch.empty_like(S), torch.empty_like(T)
    assert rest(d, S2, T2, list(range(63, -1, -1)), blob) == OK
    assert same_bits(S2, S.flip(0)) and torch.equal(T2.view(torch.int16), T.flip(0).view(torch.int16))
