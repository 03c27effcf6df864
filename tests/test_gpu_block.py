"""GPU block verify and block commit: a chain of k drafted tokens per sequence.

Against token-by-token decode on the GPU, bit for bit: every position's
output, and the committed state, tail and outputs.  Against the CPU oracle's
chained decode: within 1e-4 normwise.  Also: accepted counts of 0 and k, out
of range counts refused per sequence, the checkpoint left untouched by verify,
blocks of 1 and 32, and the full-size batch of 64.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from gdn_inputs import QWEN27B_LAYER, TINY
from tests.conftest import normwise

pytestmark = pytest.mark.gpu
TOL = 1e-4


def seq_major(arr):
    """[k][B][...] -> [B][k][...] (the calls' layout)."""
    return np.ascontiguousarray(np.swapaxes(arr, 0, 1))


def same_bits(u, v):
    return torch.equal(u.contiguous().view(torch.int32), v.contiguous().view(torch.int32))


def dev(inp):
    from tests.gpu_util import act_to_dev, dims_of, f32_to_dev
    return dict(d=dims_of(inp.shape, inp.batch), S=f32_to_dev(inp.state), T=act_to_dev(inp.tail),
                w=act_to_dev(inp.w), x=act_to_dev(seq_major(inp.x)), a=f32_to_dev(seq_major(inp.a)),
                b=f32_to_dev(seq_major(inp.b)), xs=act_to_dev(inp.x), as_=f32_to_dev(inp.a),
                bs=f32_to_dev(inp.b))


def verify(c, k):
    import gated_deltanet_decode_amd as gdn
    d = c["d"]
    o = torch.full((d.batch, k, d.num_v_heads, d.head_v_dim), float("nan"), device="cuda")
    ws = torch.empty(gdn.block_workspace_bytes(d, k), dtype=torch.uint8, device="cuda")
    gdn.block_verify(d, c["S"], c["T"], c["w"], c["x"], c["a"], c["b"], o, ws)
    torch.cuda.synchronize()
    return o


def commit(c, k, accepted, want_o=True):
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import i32_to_dev
    d = c["d"]
    S, T = c["S"].clone(), c["T"].clone()
    o = torch.full((d.batch, k, d.num_v_heads, d.head_v_dim), float("nan"), device="cuda") if want_o else None
    st = torch.full((d.batch,), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(gdn.block_workspace_bytes(d, k), dtype=torch.uint8, device="cuda")
    gdn.block_commit(d, S, T, c["w"], c["x"], c["a"], c["b"], i32_to_dev(np.array(accepted, np.int32)), o, st, ws)
    torch.cuda.synchronize()
    return o, S, T, st.cpu().numpy()


def decode(c, steps):
    """Token-by-token decode of the whole batch over block positions 0..steps-1 (library
    calls); returns the outputs [steps][B][Hv][dv] and the states and tails after each step."""
    import gated_deltanet_decode_amd as gdn
    d = c["d"]
    S, T = c["S"].clone(), c["T"].clone()
    y = torch.empty(d.batch, d.C, device="cuda")
    outs, states, tails = [], [], []
    for t in range(steps):
        o = torch.empty(d.batch, d.num_v_heads, d.head_v_dim, device="cuda")
        gdn.conv_update(d, c["xs"][t], T, c["w"], y)
        gdn.decode_step(d, S, y, c["as_"][t], c["bs"][t], o)
        outs.append(o)
        states.append(S.clone())
        tails.append(T.clone())
    torch.cuda.synchronize()
    return outs, states, tails


@pytest.fixture(scope="module", params=[("27b", 3, 12), ("tiny", 5, 32)], ids=["27b_B3_k12", "tiny_B5_k32"])
def bcase(request):
    name, B, k = request.param
    shape = QWEN27B_LAYER if name == "27b" else TINY
    return gi.decode_inputs(120 + B, shape, B, k, state_sigma=0.1, tail_random=True)


def test_block_verify_equals_decode_bitwise(bcase):
    inp = bcase
    c = dev(inp)
    k = inp.steps
    S0, T0 = c["S"].clone(), c["T"].clone()
    o = verify(c, k)
    assert same_bits(c["S"], S0) and torch.equal(c["T"], T0), "verify wrote the checkpoint"
    outs, _, _ = decode(c, k)
    for t in range(k):
        assert same_bits(o[:, t], outs[t]), f"position {t}"


def test_block_verify_matches_oracle(bcase):
    inp = bcase
    c = dev(inp)
    k = inp.steps
    og = verify(c, k).cpu().numpy()
    for s in range(inp.batch):
        o_r, _, _ = oracle.run(inp.shape, inp.state[s], inp.tail[s], inp.w, inp.x[:, s], inp.a[:, s], inp.b[:, s])
        for t in range(k):
            assert normwise(og[s, t], o_r[t]) < TOL, f"sequence {s} position {t}"


def test_block_commit_equals_decode_bitwise(bcase):
    inp = bcase
    c = dev(inp)
    k, B = inp.steps, inp.batch
    accepted = [k, 0, 5] + [1, k - 1][:B - 3]
    o, S, T, st = commit(c, k, accepted)
    assert (st == 0).all()
    outs, states, tails = decode(c, k)
    for s, L in enumerate(accepted):
        if L == 0:
            assert same_bits(S[s], c["S"][s]) and torch.equal(T[s], c["T"][s])
            assert torch.isnan(o[s]).all()
            continue
        assert same_bits(S[s], states[L - 1][s]), f"sequence {s} state"
        assert torch.equal(T[s], tails[L - 1][s]), f"sequence {s} tail"
        for t in range(L):
            assert same_bits(o[s, t], outs[t][s])
        assert torch.isnan(o[s, L:]).all(), f"sequence {s}: written past its accepted count"


def test_block_commit_matches_oracle(bcase):
    from tests.gpu_util import act_to_host
    inp = bcase
    c = dev(inp)
    k, B = inp.steps, inp.batch
    accepted = [k, 0, 5] + [1, k - 1][:B - 3]
    _, S, T, st = commit(c, k, accepted, want_o=False)
    for s, L in enumerate(accepted):
        if L == 0:
            continue
        _, S_r, t_r = oracle.run(inp.shape, inp.state[s], inp.tail[s], inp.w, inp.x[:L, s], inp.a[:L, s],
                                 inp.b[:L, s])
        assert normwise(S[s].cpu().numpy(), S_r) < TOL
        assert np.array_equal(oracle.f64(act_to_host(T[s])), t_r)


def test_out_of_range_accepted_counts_are_refused_per_sequence():
    inp = gi.decode_inputs(130, QWEN27B_LAYER, 3, 6, state_sigma=0.1, tail_random=True)
    c = dev(inp)
    _, S, T, st = commit(c, 6, [-1, 3, 7], want_o=False)
    assert list(st) == [10, 0, 10]
    for s in (0, 2):
        assert same_bits(S[s], c["S"][s]) and torch.equal(T[s], c["T"][s])
    _, states, tails = decode(c, 3)
    assert same_bits(S[1], states[2][1]) and torch.equal(T[1], tails[2][1])


def test_single_token_block():
    inp = gi.decode_inputs(131, QWEN27B_LAYER, 2, 1, state_sigma=0.1, tail_random=True)
    c = dev(inp)
    o = verify(c, 1)
    outs, states, tails = decode(c, 1)
    assert same_bits(o[:, 0], outs[0])
    _, S, T, st = commit(c, 1, [1, 1], want_o=False)
    assert same_bits(S, states[0]) and torch.equal(T, tails[0])


def test_batch64_full_size_sampled():
    """The 27B-class layer at 64 sequences and 16-token blocks (the launches the block rows
    time): all outputs against decode, committed counts mixed."""
    B, k = 64, 16
    inp = gi.decode_inputs(132, QWEN27B_LAYER, B, k, state_sigma=0.1, tail_random=True)
    c = dev(inp)
    o = verify(c, k)
    outs, states, tails = decode(c, k)
    for t in range(k):
        assert same_bits(o[:, t], outs[t]), f"position {t}"
    accepted = [(7 * s) % (k + 1) for s in range(B)]
    _, S, T, st = commit(c, k, accepted, want_o=False)
    assert (st == 0).all()
    for s, L in enumerate(accepted):
        ref_S = c["S"][s] if L == 0 else states[L - 1][s]
        ref_T = c["T"][s] if L == 0 else tails[L - 1][s]
        assert same_bits(S[s], ref_S) and torch.equal(T[s], ref_T), f"sequence {s}"


def test_prep_in_groups_of_four_with_a_ragged_tail():
    """Sixteen 13-token blocks: the prep takes four positions per workgroup, the last group
    holding one; every position equals decode."""
    inp = gi.decode_inputs(133, QWEN27B_LAYER, 16, 13, state_sigma=0.1, tail_random=True)
    c = dev(inp)
    o = verify(c, 13)
    outs, _, _ = decode(c, 13)
    for t in range(13):
        assert same_bits(o[:, t], outs[t]), f"position {t}"


@pytest.mark.parametrize("shape,B,k,ut", [(QWEN27B_LAYER, 3, 12, False), (QWEN27B_LAYER, 16, 13, True),
                                          (QWEN27B_LAYER, 64, 16, True), (TINY, 5, 32, True)],
                         ids=["27b_B3_walk", "27b_B16_ut", "27b_B64_ut", "tiny_B5_ut"])
def test_prepared_block_commit_equals_block_commit_bitwise(shape, B, k, ut):
    """A block commit that reads the operands from the verify's workspace leaves the same
    state, tail, outputs and statuses, bit for bit, as the one that prepares them again
    (counts of 0, k and out of range included)."""
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import i32_to_dev
    inp = gi.decode_inputs(150 + B, shape, B, k, state_sigma=0.1, tail_random=True)
    c = dev(inp)
    d = c["d"]
    ws = torch.empty(gdn.block_workspace_bytes(d, k), dtype=torch.uint8, device="cuda")
    o = torch.empty(B, k, d.num_v_heads, d.head_v_dim, device="cuda")
    (gdn.block_verify_ut if ut else gdn.block_verify)(d, c["S"], c["T"], c["w"], c["x"], c["a"], c["b"], o, ws)
    accepted = [(5 * s + 2) % (k + 1) for s in range(B)]
    accepted[0], accepted[-1] = k, k + 3
    S1, T1 = c["S"].clone(), c["T"].clone()
    o1 = torch.full((B, k, d.num_v_heads, d.head_v_dim), float("nan"), device="cuda")
    st1 = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    gdn.block_commit_prepared(d, S1, T1, c["x"], i32_to_dev(np.array(accepted, np.int32)), ws, o1, st1)
    o2, S2, T2, st2 = commit(c, k, accepted)
    assert list(st1.cpu().numpy()) == list(st2)
    assert same_bits(S1, S2) and torch.equal(T1, T2)
    assert torch.equal(torch.isnan(o1), torch.isnan(o2))
    assert same_bits(torch.nan_to_num(o1), torch.nan_to_num(o2))
