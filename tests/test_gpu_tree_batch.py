"""GPU tree verify and path commit over a batch: one draft tree per sequence.

A batched call must give each sequence, bit for bit, what a call on that
sequence alone gives, and token-by-token decode of its paths; the batch-1
calls are held to the oracle in test_gpu_tree.py.  Here also: samples
against the oracle directly (1e-4 normwise), accepted paths of different
lengths in one call (the empty path included), a malformed tree or path in
one sequence leaving the others intact, and the full-size batch of 64.
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
    """[n][B][...] -> [B][n][...] (the calls' layout)."""
    return np.ascontiguousarray(np.swapaxes(arr, 0, 1))


def batch_case(inp, parent=None):
    from tests.gpu_util import act_to_dev, dims_of, f32_to_dev, i32_to_dev
    parent = inp.extra["parent"] if parent is None else parent
    return dict(d=dims_of(inp.shape, inp.batch), S=f32_to_dev(inp.state), tail=act_to_dev(inp.tail),
                w=act_to_dev(inp.w), parent=i32_to_dev(parent), x=act_to_dev(seq_major(inp.x)),
                a=f32_to_dev(seq_major(inp.a)), b=f32_to_dev(seq_major(inp.b)))


def one_case(inp, s, parent=None):
    """Sequence s alone, as a batch-1 call sees it."""
    from tests.gpu_util import act_to_dev, dims_of, f32_to_dev, i32_to_dev
    parent = inp.extra["parent"] if parent is None else parent
    return dict(d=dims_of(inp.shape, 1), S=f32_to_dev(inp.state[s]), tail=act_to_dev(inp.tail[s]),
                w=act_to_dev(inp.w), parent=i32_to_dev(parent[s]), x=act_to_dev(inp.x[:, s]),
                a=f32_to_dev(inp.a[:, s]), b=f32_to_dev(inp.b[:, s]))


def verify(c, B, n):
    import gated_deltanet_decode_amd as gdn
    d = c["d"]
    o = torch.full((B, n, d.num_v_heads, d.head_v_dim), float("nan"), device="cuda")
    st = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(gdn.tree_workspace_bytes(d, n), dtype=torch.uint8, device="cuda")
    gdn.tree_verify(d, c["S"], c["tail"], c["w"], c["parent"], c["x"], c["a"], c["b"], o, st, ws)
    torch.cuda.synchronize()
    return o, st.cpu().numpy()


def commit(c, B, path):
    """path [B][L] host array; returns (o, S, tail, status) on fresh copies of the checkpoints."""
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import i32_to_dev
    d = c["d"]
    S, tail = c["S"].clone(), c["tail"].clone()
    L = path.shape[1]
    o = torch.full((B, L, d.num_v_heads, d.head_v_dim), float("nan"), device="cuda")
    st = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    gdn.commit_path(d, S, tail, c["w"], c["parent"], c["x"], c["a"], c["b"], i32_to_dev(path), o, st)
    torch.cuda.synchronize()
    return o, S, tail, st.cpu().numpy()


def decode_path(c1, path):
    """Token-by-token batch-1 decode of `path` from copies of one sequence's checkpoint."""
    import gated_deltanet_decode_amd as gdn
    d = c1["d"]
    S, tail = c1["S"].clone(), c1["tail"].clone()
    y = torch.empty(1, d.C, device="cuda")
    outs = []
    for node in path:
        o = torch.empty(1, d.num_v_heads, d.head_v_dim, device="cuda")
        gdn.conv_update(d, c1["x"][node], tail, c1["w"], y)
        gdn.decode_step(d, S, y, c1["a"][node], c1["b"][node], o)
        outs.append(o)
    torch.cuda.synchronize()
    return (torch.cat(outs) if outs else None), S, tail


def same_bits(u, v):
    return torch.equal(u.contiguous().view(torch.int32), v.contiguous().view(torch.int32))


def row_len(row):
    ends = np.nonzero(row == -1)[0]
    return int(ends[0]) if len(ends) else len(row)


# Batches of 6 (27B-class) and 20 (tiny) take the prep launch with four nodes
# per workgroup; 3 and 5 the one-node form, as batch-1 calls do.
@pytest.fixture(scope="module", params=[("27b", 3), ("tiny", 5), ("27b", 6), ("tiny", 20)],
                ids=["27b_B3", "tiny_B5", "27b_B6", "tiny_B20"])
def bcase(request):
    name, B = request.param
    shape = QWEN27B_LAYER if name == "27b" else TINY
    return gi.tree_batch_inputs(70 + B, shape, B, n_nodes=32, max_depth=8)


def test_batched_verify_equals_single_calls_bitwise(bcase):
    inp = bcase
    B, n = inp.batch, inp.steps
    o, st = verify(batch_case(inp), B, n)
    assert (st == 0).all()
    for s in range(B):
        o1, st1 = verify(one_case(inp, s), 1, n)
        assert st1[0] == 0
        assert same_bits(o[s], o1[0]), f"sequence {s}"


def test_batched_verify_matches_oracle(bcase):
    inp = bcase
    B, n = inp.batch, inp.steps
    o, st = verify(batch_case(inp), B, n)
    assert (st == 0).all()
    og = o.cpu().numpy()
    for s in range(B):
        ref = oracle.tree_verify(inp.shape, inp.state[s], inp.tail[s], inp.w, inp.extra["parent"][s], inp.x[:, s],
                                 inp.a[:, s], inp.b[:, s])
        for node in range(n):
            err = normwise(og[s, node], ref[node])
            assert err < TOL, f"sequence {s} node {node}: error {err:.3e}"


def test_batched_verify_nodes_equal_decode_bitwise(bcase):
    """A sample of nodes per sequence against token-by-token decode of its path."""
    inp = bcase
    B, n = inp.batch, inp.steps
    o, _ = verify(batch_case(inp), B, n)
    rng = np.random.default_rng(5)
    for s in range(B):
        parent = inp.extra["parent"][s]
        c1 = one_case(inp, s)
        for node in rng.choice(n, 4, replace=False):
            o_dec, _, _ = decode_path(c1, gi.path_to(parent, int(node)))
            assert same_bits(o[s, node], o_dec[-1]), f"sequence {s} node {node}"


def test_batched_commit_equals_sequential_decode_bitwise(bcase):
    """Paths of different lengths in one call; entries past a row's end stay unwritten."""
    inp = bcase
    B = inp.batch
    path = inp.extra["path"]
    assert len({row_len(r) for r in path}) > 1, "the draw should mix path lengths"
    o, S, tail, st = commit(batch_case(inp), B, path)
    assert (st == 0).all()
    for s in range(B):
        L = row_len(path[s])
        o_d, S_d, t_d = decode_path(one_case(inp, s), path[s, :L])
        assert same_bits(S[s], S_d), f"sequence {s} state"
        assert torch.equal(tail[s], t_d), f"sequence {s} tail"
        assert same_bits(o[s, :L], o_d), f"sequence {s} outputs"
        assert torch.isnan(o[s, L:]).all(), f"sequence {s}: written past the path's end"


def test_batched_commit_matches_oracle(bcase):
    from tests.gpu_util import act_to_host
    inp = bcase
    B = inp.batch
    path = inp.extra["path"]
    o, S, tail, st = commit(batch_case(inp), B, path)
    assert (st == 0).all()
    for s in range(B):
        L = row_len(path[s])
        o_r, S_r, t_r = oracle.commit_path(inp.shape, inp.state[s], inp.tail[s], inp.w, inp.extra["parent"][s],
                                           inp.x[:, s], inp.a[:, s], inp.b[:, s], path[s, :L])
        assert normwise(S[s].cpu().numpy(), S_r) < TOL
        for j in range(L):
            assert normwise(o[s, j].cpu().numpy(), o_r[j]) < TOL
        assert np.array_equal(oracle.f64(act_to_host(tail[s])), t_r)


def test_empty_path_row_commits_nothing():
    inp = gi.tree_batch_inputs(81, TINY, 3, n_nodes=12, max_depth=8)
    path = inp.extra["path"].copy()
    path[1] = -1
    c = batch_case(inp)
    o, S, tail, st = commit(c, 3, path)
    assert (st == 0).all()
    assert same_bits(S[1], c["S"][1]) and torch.equal(tail[1], c["tail"][1])
    assert torch.isnan(o[1]).all()
    for s in (0, 2):
        L = row_len(path[s])
        _, S_d, t_d = decode_path(one_case(inp, s), path[s, :L])
        assert same_bits(S[s], S_d) and torch.equal(tail[s], t_d)


def test_malformed_tree_fails_only_its_sequence():
    inp = gi.tree_batch_inputs(82, QWEN27B_LAYER, 3, n_nodes=8, max_depth=8)
    parent = inp.extra["parent"].copy()
    parent[1] = [-1, 0, 1, 5, 0, 1, 2, 3]   # a parent after its child
    c = batch_case(inp, parent)
    o, st = verify(c, 3, 8)
    assert list(st) == [0, 5, 0]
    for s in (0, 2):
        o1, _ = verify(one_case(inp, s), 1, 8)
        assert same_bits(o[s], o1[0])
    # A commit over the same trees refuses sequence 1 only.
    path = inp.extra["path"]
    _, S, tail, st = commit(c, 3, path)
    assert list(st) == [0, 5, 0]
    assert same_bits(S[1], c["S"][1]) and torch.equal(tail[1], c["tail"][1])


@pytest.mark.parametrize("bad", [[0, -1, 3], [-1, 0], [0, 0], [1], [0, 40]],
                         ids=["gap", "starts_empty", "repeated", "not_from_root", "past_the_tree"])
def test_malformed_path_row_fails_only_its_sequence(bad):
    inp = gi.tree_batch_inputs(83, QWEN27B_LAYER, 3, n_nodes=32, max_depth=8)
    parent = inp.extra["parent"]
    path = inp.extra["path"].copy()
    row = np.full(path.shape[1], -1, np.int32)
    bad = list(bad)
    if bad == [0, -1, 3]:   # a valid second step after the padding
        bad[2] = int(next(i for i in range(1, 32) if parent[2][i] == 0))
    row[:len(bad)] = bad
    path[2] = row
    c = batch_case(inp)
    _, S, tail, st = commit(c, 3, path)
    assert list(st) == [0, 0, 5]
    assert same_bits(S[2], c["S"][2]) and torch.equal(tail[2], c["tail"][2])
    for s in (0, 1):
        L = row_len(path[s])
        _, S_d, t_d = decode_path(one_case(inp, s), path[s, :L])
        assert same_bits(S[s], S_d) and torch.equal(tail[s], t_d)


def test_batch64_full_size_sampled():
    """The 27B-class layer at 64 sequences, the launch the batched tree rows time: sampled
    sequences equal their own batch-1 calls bit for bit, and one sequence's sampled heads
    match the oracle."""
    inp = gi.tree_batch_inputs(84, QWEN27B_LAYER, 64, n_nodes=32, max_depth=8)
    B, n = 64, 32
    c = batch_case(inp)
    o, st = verify(c, B, n)
    assert (st == 0).all()
    path = inp.extra["path"]
    oc, S, tail, cst = commit(c, B, path)
    assert (cst == 0).all()
    for s in (0, 29, 63):
        o1, _ = verify(one_case(inp, s), 1, n)
        assert same_bits(o[s], o1[0]), f"verify sequence {s}"
        L = row_len(path[s])
        o_d, S_d, t_d = decode_path(one_case(inp, s), path[s, :L])
        assert same_bits(S[s], S_d) and torch.equal(tail[s], t_d), f"commit sequence {s}"
        assert same_bits(oc[s, :L], o_d)
    s, lo, hi = 41, 20, 23
    ref = oracle.tree_verify(inp.shape, inp.state[s], inp.tail[s], inp.w, inp.extra["parent"][s], inp.x[:, s],
                             inp.a[:, s], inp.b[:, s], h_range=(lo, hi))
    og = o[s].cpu().numpy()
    for node in range(n):
        assert normwise(og[node, lo:hi], ref[node, lo:hi]) < TOL, f"node {node}"


def test_siblings_at_the_deepest_level_batched():
    """The three-wave form (more than two workgroups per CU) on trees whose depth-7 nodes
    have several children, against batch-1 calls and token-by-token decode."""
    inp = gi.tree_batch_inputs(85, QWEN27B_LAYER, 3, n_nodes=15, max_depth=8)
    parent = inp.extra["parent"].copy()
    parent[0] = [-1, 0, 1, 2, 3, 4, 5, 6, 6, 6, 5, 10, 4, 1, 0]
    parent[2] = [-1, 0, 1, 2, 3, 4, 5, 6, 6, 0, 9, 10, 11, 12, 13]
    o, st = verify(batch_case(inp, parent), 3, 15)
    assert (st == 0).all()
    for s in range(3):
        c1 = one_case(inp, s, parent)
        o1, _ = verify(c1, 1, 15)
        assert same_bits(o[s], o1[0]), f"sequence {s}"
        for node in range(15):
            o_dec, _, _ = decode_path(c1, gi.path_to(parent[s], node))
            assert same_bits(o[s, node], o_dec[-1]), f"sequence {s} node {node}"


def test_narrow_heads_three_wave_form():
    """Heads of width 32 at 130 sequences (more than two workgroups per CU): sampled
    sequences against their batch-1 calls bit for bit, and one against the oracle."""
    B, n = 130, 32
    inp = gi.tree_batch_inputs(86, TINY, B, n_nodes=n, max_depth=8)
    o, st = verify(batch_case(inp), B, n)
    assert (st == 0).all()
    for s in (0, 77, 129):
        o1, _ = verify(one_case(inp, s), 1, n)
        assert same_bits(o[s], o1[0]), f"sequence {s}"
    s = 101
    ref = oracle.tree_verify(inp.shape, inp.state[s], inp.tail[s], inp.w, inp.extra["parent"][s], inp.x[:, s],
                             inp.a[:, s], inp.b[:, s])
    assert normwise(o[s].cpu().numpy(), ref) < TOL


def test_prep_in_groups_of_four_nodes_with_a_ragged_tail():
    """Eight 30-node trees: enough prep workgroups that each takes four nodes, the last
    group of each tree holding two; every sequence equals its own batch-1 call."""
    B, n = 8, 30
    inp = gi.tree_batch_inputs(87, QWEN27B_LAYER, B, n_nodes=n, max_depth=8)
    o, st = verify(batch_case(inp), B, n)
    assert (st == 0).all()
    for s in range(B):
        o1, _ = verify(one_case(inp, s), 1, n)
        assert same_bits(o[s], o1[0]), f"sequence {s}"


@pytest.mark.parametrize("shape,B,ut", [(QWEN27B_LAYER, 3, False), (QWEN27B_LAYER, 6, True), (TINY, 20, False),
                                        (TINY, 4, True)],
                         ids=["27b_B3_walk", "27b_B6_ut", "tiny_B20_walk", "tiny_B4_ut"])
def test_prepared_commit_equals_commit_bitwise(shape, B, ut):
    """A commit that reads the path's operands from the verify's workspace leaves the same
    state, tail and outputs, bit for bit, as the commit that convolves them again; an empty
    and a malformed path row behave the same way too."""
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import i32_to_dev
    n = 32
    inp = gi.tree_batch_inputs(240 + B, shape, B, n)
    c = batch_case(inp)
    d = c["d"]
    path = inp.extra["path"].copy()
    path[1] = -1                              # the empty commit
    if B > 2:
        path[2, 1] = 31 if inp.extra["parent"][2][31] != path[2, 0] else 30   # not a child of path[0]
    o = torch.empty(B, n, d.num_v_heads, d.head_v_dim, device="cuda")
    st = torch.zeros(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(gdn.tree_workspace_bytes(d, n), dtype=torch.uint8, device="cuda")
    (gdn.tree_verify_ut if ut else gdn.tree_verify)(d, c["S"], c["tail"], c["w"], c["parent"], c["x"], c["a"],
                                                    c["b"], o, st, ws)
    L = path.shape[1]
    S1, T1 = c["S"].clone(), c["tail"].clone()
    o1 = torch.full((B, L, d.num_v_heads, d.head_v_dim), float("nan"), device="cuda")
    st1 = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    gdn.commit_path_prepared(d, S1, T1, c["parent"], c["x"], i32_to_dev(path), ws, o1, st1)
    o2, S2, T2, st2 = commit(c, B, path)
    torch.cuda.synchronize()
    assert list(st1.cpu().numpy()) == list(st2)
    assert same_bits(S1, S2) and torch.equal(T1, T2)
    assert torch.equal(torch.isnan(o1), torch.isnan(o2))
    assert same_bits(torch.nan_to_num(o1), torch.nan_to_num(o2))
