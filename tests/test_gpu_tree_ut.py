"""GPU tree and block verify in the UT form (gdn_tree_verify_ut, gdn_block_verify_ut),
in both of its forms: one launch (no workspace) and two (prep into a workspace).

The UT form reorders the arithmetic, so it is held to the oracle's per-node
path replay within 1e-4 normwise (per node: over that node's heads and rows),
not to decode bit for bit; the exact walk (gdn_tree_verify) is the second check,
to the same bar.  Also: ragged node counts (1, 17), blocks of 1 and 32 (a
chain of depth 32, past the trees' depth limit), a malformed tree in one
sequence of a batch (status set, its outputs unwritten, the others verified),
the checkpoint left untouched, and the full-size batch of 64 sampled against
the oracle.  Batches of 6 (27B-class) and 70 (tiny) also run the prep
launch with four nodes per workgroup and two or more UT workgroups per CU.
At batch 1 and 2 the 27B-class verify splits each head over two workgroups;
a batch of 4 (whole heads) equals its sequences' batch-1 calls bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from gdn_inputs import F32, QWEN27B_LAYER, TINY, LayerShape
from tests.conftest import normwise
from tests.test_gpu_tree_batch import batch_case, seq_major

pytestmark = pytest.mark.gpu
TOL = 1e-4


FORMS = ["one_launch", "workspace"]


def verify(c, B, n, ut=True, form="one_launch"):
    """form: the UT form's one launch (no workspace) or its two (prep into a workspace)."""
    import gated_deltanet_decode_amd as gdn
    d = c["d"]
    o = torch.full((B, n, d.num_v_heads, d.head_v_dim), float("nan"), device="cuda")
    st = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(gdn.tree_workspace_bytes(d, n), dtype=torch.uint8, device="cuda")
    f = gdn.tree_verify_ut if ut else gdn.tree_verify
    f(d, c["S"], c["tail"], c["w"], c["parent"], c["x"], c["a"], c["b"], o, st,
      None if ut and form == "one_launch" else ws)
    torch.cuda.synchronize()
    return o, st.cpu().numpy()


def per_node(og, ref, what=""):
    """Normwise error of every node's output on its own; asserts each is within TOL."""
    for node in range(ref.shape[0]):
        err = normwise(og[node], ref[node])
        assert err < TOL, f"{what} node {node}: error {err:.3e}"


def oracle_tree(inp, s, parent=None):
    parent = inp.extra["parent"][s] if parent is None else parent
    return oracle.tree_verify(inp.shape, inp.state[s], inp.tail[s], inp.w, parent, inp.x[:, s], inp.a[:, s],
                              inp.b[:, s])


@pytest.mark.parametrize("shape,B,n,seed", [(QWEN27B_LAYER, 1, 32, 200), (QWEN27B_LAYER, 3, 32, 201),
                                            (TINY, 4, 32, 202), (TINY, 2, 17, 203), (QWEN27B_LAYER, 2, 1, 204),
                                            (TINY, 3, 9, 205), (QWEN27B_LAYER, 6, 32, 206), (TINY, 70, 23, 207)],
                         ids=["27b_B1", "27b_B3", "tiny_B4", "tiny_n17", "27b_n1", "tiny_n9", "27b_B6",
                              "tiny_B70"])
@pytest.mark.parametrize("form", FORMS)
def test_ut_verify_matches_oracle(shape, B, n, seed, form):
    inp = gi.tree_batch_inputs(seed, shape, B, n)
    c = batch_case(inp)
    S0, T0 = c["S"].clone(), c["tail"].clone()
    o, st = verify(c, B, n, form=form)
    assert (st == 0).all()
    assert torch.equal(c["S"], S0) and torch.equal(c["tail"], T0), "verify wrote the checkpoint"
    og = o.cpu().numpy()
    for s in range(B):
        per_node(og[s], oracle_tree(inp, s), f"sequence {s}")


@pytest.mark.parametrize("shape", [QWEN27B_LAYER, TINY], ids=["27b", "tiny"])
@pytest.mark.parametrize("form", FORMS)
def test_ut_verify_matches_the_exact_walk(shape, form):
    B, n = 4, 32
    inp = gi.tree_batch_inputs(210, shape, B, n)
    c = batch_case(inp)
    o_ut, _ = verify(c, B, n, form=form)
    o_w, _ = verify(c, B, n, ut=False)
    for s in range(B):
        per_node(o_ut[s].cpu().numpy(), o_w[s].cpu().numpy().astype(np.float64), f"sequence {s}")


@pytest.mark.parametrize("B", [3, 6], ids=["B3", "B6"])
@pytest.mark.parametrize("form", FORMS)
def test_malformed_tree_in_one_sequence(B, form):
    n = 32
    inp = gi.tree_batch_inputs(211, QWEN27B_LAYER, B, n)
    parent = inp.extra["parent"].copy()
    parent[1, 7] = 9                       # a parent after its child
    c = batch_case(inp, parent)
    o, st = verify(c, B, n, form=form)
    assert list(st) == [0, 5] + [0] * (B - 2)
    assert torch.isnan(o[1]).all(), "a malformed tree's outputs were written"
    og = o.cpu().numpy()
    for s in [0] + list(range(2, B)):
        per_node(og[s], oracle_tree(inp, s), f"sequence {s}")


@pytest.mark.parametrize("shape,B,k", [(QWEN27B_LAYER, 2, 32), (TINY, 3, 32), (QWEN27B_LAYER, 2, 1),
                                       (TINY, 2, 13), (QWEN27B_LAYER, 6, 32)],
                         ids=["27b_k32", "tiny_k32", "27b_k1", "tiny_k13", "27b_B6_k32"])
@pytest.mark.parametrize("form", FORMS)
def test_ut_block_verify_matches_oracle(shape, B, k, form):
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import act_to_dev, dims_of, f32_to_dev
    inp = gi.decode_inputs(220 + k, shape, B, k, state_sigma=0.1, tail_random=True)
    d = dims_of(shape, B)
    S, T = f32_to_dev(inp.state), act_to_dev(inp.tail)
    o = torch.full((B, k, shape.num_v_heads, shape.head_v_dim), float("nan"), device="cuda")
    ws = torch.empty(gdn.block_workspace_bytes(d, k), dtype=torch.uint8, device="cuda")
    gdn.block_verify_ut(d, S, T, act_to_dev(inp.w), act_to_dev(seq_major(inp.x)), f32_to_dev(seq_major(inp.a)),
                        f32_to_dev(seq_major(inp.b)), o, None if form == "one_launch" else ws)
    torch.cuda.synchronize()
    og = o.cpu().numpy()
    for s in range(B):
        o_r, _, _ = oracle.run(shape, inp.state[s], inp.tail[s], inp.w, inp.x[:, s], inp.a[:, s], inp.b[:, s])
        per_node(og[s], o_r, f"sequence {s}")


@pytest.mark.parametrize("form", FORMS)
def test_batch64_full_size_sampled(form):
    """The 27B-class layer, 64 trees of 32 nodes (the one-launch form is the launch the
    bench times): four sequences against the oracle; all 64 against the exact walk."""
    B, n = 64, 32
    inp = gi.tree_batch_inputs(230, QWEN27B_LAYER, B, n)
    c = batch_case(inp)
    o, st = verify(c, B, n, form=form)
    assert (st == 0).all()
    og = o.cpu().numpy()
    for s in (0, 21, 42, 63):
        per_node(og[s], oracle_tree(inp, s), f"sequence {s}")
    o_w, _ = verify(c, B, n, ut=False)
    ow = o_w.cpu().numpy().astype(np.float64)
    for s in range(B):
        per_node(og[s], ow[s], f"sequence {s}")


LAYER_F32 = LayerShape(16, 48, 128, 128, 4, F32)   # the 27B-class layer with fp32 activations


@pytest.mark.parametrize("shape", [QWEN27B_LAYER, LAYER_F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("form", FORMS)
def test_split_heads_equal_whole_heads_bitwise(form, shape):
    """At batch 1 and 2 each (sequence, value head) of the 27B-class layer is verified by
    two workgroups, one per half of the rows; from batch 4 on by one.  The arithmetic is
    the same either way, so every sequence of a batch of 4 equals its own batch-1 call, and
    the first two equal a batch-2 call, bit for bit."""
    from tests.test_gpu_tree_batch import one_case
    inp = gi.tree_batch_inputs(240, shape, 4, n_nodes=32, max_depth=8)
    n = inp.steps
    o4, st4 = verify(batch_case(inp), 4, n, form=form)
    assert (st4 == 0).all()
    for s in range(4):
        o1, st1 = verify(one_case(inp, s), 1, n, form=form)
        assert st1[0] == 0
        assert torch.equal(o4[s].view(torch.int32), o1[0].view(torch.int32)), f"{form}: sequence {s}"
    two = dataclasses.replace(inp, batch=2, x=inp.x[:, :2], a=inp.a[:, :2], b=inp.b[:, :2], state=inp.state[:2],
                              tail=inp.tail[:2],
                              extra={k: v[:2] if isinstance(v, np.ndarray) else v for k, v in inp.extra.items()})
    o2, st2 = verify(batch_case(two), 2, n, form=form)
    assert (st2 == 0).all()
    assert torch.equal(o2.view(torch.int32), o4[:2].view(torch.int32)), form


@pytest.mark.parametrize("form", FORMS)
def test_f32_activations_27b_layer_matches_oracle(form):
    """The 27B-class layer with fp32 activations at batch 1 (heads split over two workgroups
    in the one-launch form): every node within the bar of the oracle's path replay."""
    inp = gi.tree_batch_inputs(241, LAYER_F32, 1, n_nodes=32, max_depth=8)
    o, st = verify(batch_case(inp), 1, inp.steps, form=form)
    assert st[0] == 0
    per_node(o[0].cpu().numpy(), oracle_tree(inp, 0), f"{form}")
