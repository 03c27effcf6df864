"""gdn_tree_verify_ut_noalloc through the C ABI: the tree verify that takes no
workspace (its operands go to the library's per-GPU scratch array) gives, bit
for bit, what gdn_tree_verify_ut gives with a caller workspace, on two calls in
a row, the second smaller than the first; a call whose operands would not fit
the array is refused before anything is written; no device memory is
allocated by the call."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from gdn_inputs import QWEN27B_LAYER, TINY
from tests.conftest import normwise

pytestmark = pytest.mark.gpu


def _case(inp):
    from tests.gpu_util import act_to_dev, dims_of, f32_to_dev, i32_to_dev
    sm = lambda arr: np.ascontiguousarray(np.swapaxes(arr, 0, 1))
    return dict(d=dims_of(inp.shape, inp.batch), S=f32_to_dev(inp.state), tail=act_to_dev(inp.tail),
                w=act_to_dev(inp.w), parent=i32_to_dev(inp.extra["parent"]), x=act_to_dev(sm(inp.x)),
                a=f32_to_dev(sm(inp.a)), b=f32_to_dev(sm(inp.b)))


def _both(inp):
    import gated_deltanet_decode_amd as gdn
    c = _case(inp)
    d, B, n = c["d"], inp.batch, inp.steps
    shape = (B, n, d.num_v_heads, d.head_v_dim)
    o_ref = torch.full(shape, float("nan"), device="cuda")
    st_ref = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(gdn.tree_workspace_bytes(d, n), dtype=torch.uint8, device="cuda")
    gdn.tree_verify_ut(d, c["S"], c["tail"], c["w"], c["parent"], c["x"], c["a"], c["b"], o_ref, st_ref, ws)
    torch.cuda.synchronize()
    del ws
    o = torch.full(shape, float("nan"), device="cuda")
    st = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    gdn.tree_verify_ut_noalloc(d, c["S"], c["tail"], c["w"], c["parent"], c["x"], c["a"], c["b"], o, st)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return o, st, o_ref, st_ref


@pytest.mark.parametrize("big_batch,small_shape,small_batch", [(8, QWEN27B_LAYER, 3), (1, TINY, 3)],
                         ids=["27b_eight_trees_then_three", "27b_one_tree_then_three_tiny"])
def test_two_calls_in_a_row_second_smaller(big_batch, small_shape, small_batch):
    big = gi.tree_batch_inputs(400, QWEN27B_LAYER, big_batch, 32)
    small = gi.tree_batch_inputs(401, small_shape, small_batch, 17)   # the second call, smaller
    for inp in (big, small):
        o, st, o_ref, st_ref = _both(inp)
        assert (st.cpu().numpy() == 0).all() and (st_ref.cpu().numpy() == 0).all()
        assert torch.equal(o.view(torch.int32), o_ref.view(torch.int32)), f"batch {inp.batch}"
        ref = oracle.tree_verify(inp.shape, inp.state[0], inp.tail[0], inp.w, inp.extra["parent"][0], inp.x[:, 0],
                                 inp.a[:, 0], inp.b[:, 0])
        og = o[0].cpu().numpy()
        for node in range(inp.steps):
            assert normwise(og[node], ref[node]) < 1e-4


def test_tiny_layer_and_a_malformed_tree():
    inp = gi.tree_batch_inputs(402, TINY, 20, 32)
    inp.extra["parent"][4, 9] = 12                                   # a parent after its child
    o, st, o_ref, st_ref = _both(inp)
    assert list(st.cpu().numpy()) == list(st_ref.cpu().numpy())
    assert st.cpu().numpy()[4] == 5
    assert torch.equal(torch.isnan(o), torch.isnan(o_ref))
    assert torch.equal(torch.nan_to_num(o).view(torch.int32), torch.nan_to_num(o_ref).view(torch.int32))


def test_too_large_for_the_scratch_is_refused():
    import gated_deltanet_decode_amd as gdn
    inp = gi.tree_batch_inputs(403, QWEN27B_LAYER, 13, 32)          # 17.4 MB > 16 MiB
    c = _case(inp)
    d = c["d"]
    assert gdn.tree_workspace_bytes(d, 32) > gdn.NOALLOC_SCRATCH_BYTES
    o = torch.full((13, 32, 48, 128), float("nan"), device="cuda")
    with pytest.raises(gdn.GdnError) as e:
        gdn.tree_verify_ut_noalloc(d, c["S"], c["tail"], c["w"], c["parent"], c["x"], c["a"], c["b"], o, None)
    assert e.value.status == 6
    torch.cuda.synchronize()
    assert torch.isnan(o).all()
