"""GPU tree verify and path commit.

Against the CPU oracle: outputs within 1e-4 (normwise per node), tree tables
and conv tails exactly.  GPU against GPU, bit for bit: every node's output
equals token-by-token decode of its root-first path from the checkpoint, and
a commit equals token-by-token decode of the accepted path (state, tail and
per-token outputs).
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


def dev_case(inp):
    from tests.gpu_util import act_to_dev, dims_of, f32_to_dev, i32_to_dev
    return dict(d=dims_of(inp.shape, 1), S=f32_to_dev(inp.state[0]), tail=act_to_dev(inp.tail[0]),
                w=act_to_dev(inp.w), parent=i32_to_dev(inp.extra["parent"]), x=act_to_dev(inp.x[:, 0]),
                a=f32_to_dev(inp.a[:, 0]), b=f32_to_dev(inp.b[:, 0]))


def gpu_verify(c, n):
    import gated_deltanet_decode_amd as gdn
    d = c["d"]
    o = torch.full((n, d.num_v_heads, d.head_v_dim), float("nan"), device="cuda")
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(gdn.tree_workspace_bytes(d, n), dtype=torch.uint8, device="cuda")
    gdn.tree_verify(d, c["S"], c["tail"], c["w"], c["parent"], c["x"], c["a"], c["b"], o, st, ws)
    torch.cuda.synchronize()
    return o, int(st.item())


def gpu_decode_path(c, path):
    """Token-by-token library decode over `path` from copies of the checkpoint."""
    import gated_deltanet_decode_amd as gdn
    d = c["d"]
    S = c["S"].clone()
    tail = c["tail"].clone()
    y = torch.empty(1, d.C, device="cuda")
    os_ = []
    for node in path:
        o = torch.empty(1, d.num_v_heads, d.head_v_dim, device="cuda")
        gdn.conv_update(d, c["x"][node], tail, c["w"], y)
        gdn.decode_step(d, S, y, c["a"][node], c["b"][node], o)
        os_.append(o)
    torch.cuda.synchronize()
    return torch.cat(os_), S, tail


def gpu_commit(c, path, want_o=True):
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import i32_to_dev
    d = c["d"]
    S = c["S"].clone()
    tail = c["tail"].clone()
    o = torch.empty(len(path), d.num_v_heads, d.head_v_dim, device="cuda") if want_o else None
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    gdn.commit_path(d, S, tail, c["w"], c["parent"], c["x"], c["a"], c["b"], i32_to_dev(path), o, st)
    torch.cuda.synchronize()
    return o, S, tail, int(st.item())


@pytest.fixture(scope="module", params=["27b", "tiny"])
def case(request):
    if request.param == "27b":
        inp = gi.tree_inputs(3, QWEN27B_LAYER, n_nodes=32, max_depth=8)
    else:
        inp = gi.tree_inputs(30, TINY, n_nodes=32, max_depth=8)
    return inp


def test_tree_tables_exact():
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import i32_to_dev
    rng = np.random.default_rng(40)
    trees = [gi.random_tree(rng, n, 8) for n in (1, 2, 3, 7, 16, 31, 32) for _ in range(6)]
    trees += [np.arange(-1, 7, dtype=np.int32), np.array([-1] + [0] * 31, np.int32)]
    for parent in trees:
        n = len(parent)
        depth = torch.zeros(n, dtype=torch.int32, device="cuda")
        order = torch.zeros(n, dtype=torch.int32, device="cuda")
        st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        gdn.tree_tables(i32_to_dev(parent), depth, order, st)
        rc, d_ref, o_ref = oracle.tree_tables(parent, 8)
        assert rc == 0 and st.item() == 0
        assert np.array_equal(depth.cpu().numpy(), d_ref)
        assert np.array_equal(order.cpu().numpy(), o_ref)


@pytest.mark.parametrize("parent", [[0, 0], [-1, 1], [-1, 0, 3, 1], [-1, -1], list(range(-1, 8)), [-1, 0, 0, 2, 40]])
def test_tree_tables_reject(parent):
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import i32_to_dev
    n = len(parent)
    depth = torch.zeros(n, dtype=torch.int32, device="cuda")
    order = torch.zeros(n, dtype=torch.int32, device="cuda")
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    gdn.tree_tables(i32_to_dev(np.array(parent, np.int32)), depth, order, st)
    assert st.item() == 5
    assert oracle.tree_tables(np.array(parent, np.int32), 8)[0] == oracle.ERR_TREE


def test_verify_matches_oracle(case):
    inp = case
    c = dev_case(inp)
    n = len(inp.extra["parent"])
    o, st = gpu_verify(c, n)
    assert st == 0
    ref = oracle.tree_verify(inp.shape, inp.state[0], inp.tail[0], inp.w, inp.extra["parent"], inp.x[:, 0],
                             inp.a[:, 0], inp.b[:, 0])
    og = o.cpu().numpy()
    for node in range(n):
        err = normwise(og[node], ref[node])
        assert err < TOL, f"node {node}: error {err:.3e}"


def test_verify_rows_equal_decode_rows_bitwise(case):
    """Every node's output equals token-by-token decode of its path, bit for bit."""
    inp = case
    c = dev_case(inp)
    parent = inp.extra["parent"]
    o, st = gpu_verify(c, len(parent))
    for node in range(len(parent)):
        path = gi.path_to(parent, node)
        o_dec, _, _ = gpu_decode_path(c, path)
        assert torch.equal(o[node].view(torch.int32), o_dec[-1].view(torch.int32)), f"node {node} differs"


def test_verify_leaves_checkpoint_untouched(case):
    inp = case
    c = dev_case(inp)
    S0, t0 = c["S"].clone(), c["tail"].clone()
    gpu_verify(c, len(inp.extra["parent"]))
    assert torch.equal(c["S"].view(torch.int32), S0.view(torch.int32))
    assert torch.equal(c["tail"], t0)


def test_commit_equals_sequential_decode_bitwise(case):
    inp = case
    c = dev_case(inp)
    parent = inp.extra["parent"]
    rng = np.random.default_rng(41)
    paths = [inp.extra["path"]] + [gi.path_to(parent, int(m)) for m in rng.choice(len(parent), 6)]
    for path in paths:
        o_c, S_c, t_c, st = gpu_commit(c, path)
        assert st == 0
        o_d, S_d, t_d = gpu_decode_path(c, path)
        assert torch.equal(S_c.view(torch.int32), S_d.view(torch.int32))
        assert torch.equal(t_c, t_d)
        assert torch.equal(o_c.view(torch.int32), o_d.view(torch.int32))


def test_commit_matches_oracle(case):
    from tests.gpu_util import act_to_host
    inp = case
    c = dev_case(inp)
    path = inp.extra["path"]
    o_c, S_c, t_c, st = gpu_commit(c, path)
    o_r, S_r, t_r = oracle.commit_path(inp.shape, inp.state[0], inp.tail[0], inp.w, inp.extra["parent"],
                                       inp.x[:, 0], inp.a[:, 0], inp.b[:, 0], path)
    assert normwise(S_c.cpu().numpy(), S_r) < TOL
    for j in range(len(path)):
        assert normwise(o_c[j].cpu().numpy(), o_r[j]) < TOL
    assert np.array_equal(oracle.f64(act_to_host(t_c)), t_r)


def test_commit_without_outputs(case):
    inp = case
    c = dev_case(inp)
    path = inp.extra["path"]
    _, S1, t1, _ = gpu_commit(c, path, want_o=True)
    _, S2, t2, _ = gpu_commit(c, path, want_o=False)
    assert torch.equal(S1.view(torch.int32), S2.view(torch.int32)) and torch.equal(t1, t2)


@pytest.mark.parametrize("kind", ["not_from_root", "repeated_node", "skips_a_level", "past_the_tree"])
def test_commit_rejects_bad_path_and_leaves_state(kind):
    inp = gi.tree_inputs(3, QWEN27B_LAYER, n_nodes=32, max_depth=8)
    c = dev_case(inp)
    parent = inp.extra["parent"]
    n = len(parent)
    bad = {"not_from_root": [1], "repeated_node": [0, 0],
           "skips_a_level": [0, next(i for i in range(1, n) if parent[i] != 0)],
           "past_the_tree": [0, n]}[kind]
    bad = np.array(bad, np.int32)
    _, S, t, st = gpu_commit(c, bad, want_o=False)
    assert st == 5
    assert torch.equal(S.view(torch.int32), c["S"].view(torch.int32))
    assert torch.equal(t, c["tail"])


def test_verify_rejects_bad_tree():
    inp = gi.tree_inputs(3, QWEN27B_LAYER, n_nodes=8, max_depth=8)
    c = dev_case(inp)
    from tests.gpu_util import i32_to_dev
    c["parent"] = i32_to_dev(np.array([-1, 0, 1, 5, 0, 1, 2, 3], np.int32))
    _, st = gpu_verify(c, 8)
    assert st == 5


@pytest.mark.parametrize("shape", [LayerShape(2, 6, 128, 128, 4, "bf16"), LayerShape(4, 4, 32, 32, 4, "f32")])
@pytest.mark.parametrize("n", [1, 2, 9])
def test_small_trees(shape, n):
    inp = gi.tree_inputs(50 + n, shape, n_nodes=n, max_depth=8)
    c = dev_case(inp)
    o, st = gpu_verify(c, n)
    assert st == 0
    ref = oracle.tree_verify(shape, inp.state[0], inp.tail[0], inp.w, inp.extra["parent"], inp.x[:, 0],
                             inp.a[:, 0], inp.b[:, 0])
    assert normwise(o.cpu().numpy(), ref) < TOL


def test_deep_chain_and_wide_star():
    shape = QWEN27B_LAYER
    for parent in (np.arange(-1, 7, dtype=np.int32), np.array([-1] + [0] * 31, np.int32)):
        inp = gi.tree_inputs(60, shape, n_nodes=len(parent), max_depth=8)
        inp.extra["parent"] = parent
        c = dev_case(inp)
        o, st = gpu_verify(c, len(parent))
        assert st == 0
        for node in range(len(parent)):
            o_dec, _, _ = gpu_decode_path(c, gi.path_to(parent, node))
            assert torch.equal(o[node].view(torch.int32), o_dec[-1].view(torch.int32))


def test_siblings_at_the_deepest_level():
    """A depth-7 node with three children at depth 8, and siblings at every level above:
    the later children restart from the deepest saved row."""
    parent = np.array([-1, 0, 1, 2, 3, 4, 5, 6, 6, 6, 5, 10, 4, 1, 0], np.int32)
    assert gi.tree_depths(parent).max() == 8
    inp = gi.tree_inputs(61, QWEN27B_LAYER, n_nodes=len(parent), max_depth=8)
    inp.extra["parent"] = parent
    c = dev_case(inp)
    o, st = gpu_verify(c, len(parent))
    assert st == 0
    for node in range(len(parent)):
        o_dec, _, _ = gpu_decode_path(c, gi.path_to(parent, node))
        assert torch.equal(o[node].view(torch.int32), o_dec[-1].view(torch.int32)), f"node {node}"
