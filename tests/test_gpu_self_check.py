"""gdn_self_check on the GPU, through the C ABI: the load-time check that tree
verify and commit rows equal decode rows bit for bit passes on every supported
head width and activation type, fails when one replayed input bit is flipped
(its false branch), reports no tree or path error, and gives the same verdict
on a second call with another seed and on another stream."""
import numpy as np
import pytest
import torch

from gdn_inputs import QWEN27B_LAYER, TINY, LayerShape

pytestmark = pytest.mark.gpu

SHAPES = {"27b_bf16": QWEN27B_LAYER, "tiny_f32": TINY, "27b_f32": LayerShape(16, 48, 128, 128, 4, "f32"),
          "g8_bf16": LayerShape(2, 16, 128, 128, 4, "bf16"), "d32_g3_bf16": LayerShape(2, 6, 32, 32, 4, "bf16")}


def run(shape, seed, flags=0, stream=None):
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import dims_of
    d = dims_of(shape, 1)
    ws = torch.empty(gdn.self_check_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    res = torch.full((4,), -99, dtype=torch.int32, device="cuda")
    gdn.self_check(d, res, ws, seed=seed, flags=flags, stream=stream)
    torch.cuda.synchronize()
    return res.cpu().numpy()


@pytest.mark.parametrize("name", list(SHAPES))
def test_self_check_passes(name):
    r = run(SHAPES[name], 11)
    print(f"[self check] {name}: {list(r)}")
    assert list(r) == [0, 0, 0, 0]


@pytest.mark.parametrize("name", ["27b_bf16", "tiny_f32"])
def test_self_check_catches_a_flipped_input(name):
    import gated_deltanet_decode_amd as gdn
    r = run(SHAPES[name], 12, flags=gdn.SELF_CHECK_PERTURB)
    print(f"[self check] {name} perturbed: {list(r)}")
    assert r[0] == 11                  # GDN_ERR_SELF_CHECK
    assert r[1] > 0 and r[2] == 0      # outputs of one node differ; the committed path is untouched
    assert r[3] == 0


def test_self_check_other_seed_and_stream():
    s = torch.cuda.Stream()
    r1 = run(QWEN27B_LAYER, 0xC0FFEE, stream=s)
    r2 = run(QWEN27B_LAYER, 1)
    assert list(r1) == [0, 0, 0, 0] and list(r2) == [0, 0, 0, 0]
