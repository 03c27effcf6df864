"""GPU: the library's calls captured in one HIP graph and replayed.

The header promises that every call can be captured: nothing allocates,
synchronises or clears memory with a memset inside a call.  One speculative
round of the 27B-class layer at batch 2 (a fused decode token, the exact and
both UT-form tree verifies, the prepared path commit), a per-channel-decay
token, a one-launch block verify, a snapshot / restore pair and the self-check
are captured once; the graph is replayed three times, the inputs reset by eager
copies and the device synchronised between replays, and every replay must
equal, bit for bit, the same calls run eagerly.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gdn_inputs import QWEN27B_LAYER

pytestmark = pytest.mark.gpu


def test_a_round_of_calls_replays_bit_for_bit():
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import act_to_dev, dims_of, f32_to_dev, i32_to_dev
    shape, B, n = QWEN27B_LAYER, 2, 32
    Hv, D = shape.num_v_heads, shape.head_v_dim
    d = dims_of(shape, B)
    tin = gi.tree_batch_inputs(500, shape, B, n)
    kin = gi.kda_inputs(501, shape, B, 1)
    sm = lambda arr: np.ascontiguousarray(np.swapaxes(arr, 0, 1))
    # inputs (never written by the round)
    S0, T0, w = f32_to_dev(tin.state), act_to_dev(tin.tail), act_to_dev(tin.w)
    parent, path = i32_to_dev(tin.extra["parent"]), i32_to_dev(tin.extra["path"])
    x, a, b = act_to_dev(sm(tin.x)), f32_to_dev(sm(tin.a)), f32_to_dev(sm(tin.b))
    xk, ak, bk = act_to_dev(kin.x[0]), f32_to_dev(kin.a[0]), f32_to_dev(kin.b[0])
    x0, a0, b0 = act_to_dev(tin.x[0]), f32_to_dev(tin.a[0]), f32_to_dev(tin.b[0])
    seqs = torch.arange(B, dtype=torch.int32, device="cuda")
    # buffers the round writes
    bufs = dict(
        S_dec=torch.empty_like(S0), T_out=torch.empty_like(T0), o_dec=torch.empty(B, Hv, D, device="cuda"),
        S_kda=torch.empty_like(S0), Tk_out=torch.empty_like(T0), o_kda=torch.empty(B, Hv, D, device="cuda"),
        o_walk=torch.empty(B, n, Hv, D, device="cuda"), o_ut1=torch.empty(B, n, Hv, D, device="cuda"),
        o_ut2=torch.empty(B, n, Hv, D, device="cuda"), st=torch.empty(B, dtype=torch.int32, device="cuda"),
        S_com=torch.empty_like(S0), T_com=torch.empty_like(T0), o_com=torch.empty(B, path.shape[1], Hv, D,
                                                                                   device="cuda"),
        cst=torch.empty(B, dtype=torch.int32, device="cuda"),
        o_blk=torch.empty(B, 8, Hv, D, device="cuda"),
        S_snap=torch.empty_like(S0), T_snap=torch.empty_like(T0), sst=torch.empty(1, dtype=torch.int32, device="cuda"),
        chk=torch.empty(4, dtype=torch.int32, device="cuda"),
    )
    ws = torch.empty(gdn.tree_workspace_bytes(d, n), dtype=torch.uint8, device="cuda")
    blob = torch.empty(gdn.snapshot_bytes(d, B), dtype=torch.uint8, device="cuda")
    d1 = dims_of(shape, 1)
    cws = torch.empty(gdn.self_check_workspace_bytes(d1), dtype=torch.uint8, device="cuda")

    def reset():
        for k in ("S_dec", "S_kda", "S_com", "S_snap"):
            bufs[k].copy_(S0)
        for k in ("T_com", "T_snap"):
            bufs[k].copy_(T0)
        for k, v in bufs.items():
            if k.startswith("o_"):
                v.fill_(float("nan"))
        bufs["st"].fill_(-7)
        bufs["cst"].fill_(-7)
        bufs["sst"].fill_(-7)
        bufs["chk"].fill_(-7)

    def round_of_calls():
        gdn.decode_token(d, bufs["S_dec"], T0, bufs["T_out"], w, x0, a0, b0, bufs["o_dec"])
        gdn.kda_decode_token(d, bufs["S_kda"], T0, bufs["Tk_out"], w, xk, ak, bk, bufs["o_kda"])
        gdn.tree_verify(d, S0, T0, w, parent, x, a, b, bufs["o_walk"], bufs["st"], ws)
        gdn.tree_verify_ut(d, S0, T0, w, parent, x, a, b, bufs["o_ut2"], bufs["st"], ws)
        gdn.commit_path_prepared(d, bufs["S_com"], bufs["T_com"], parent, x, path, ws, bufs["o_com"], bufs["cst"])
        gdn.tree_verify_ut(d, S0, T0, w, parent, x, a, b, bufs["o_ut1"], bufs["st"])
        gdn.block_verify_ut(d, S0, T0, w, xb, ab, bb, bufs["o_blk"])
        gdn.snapshot(d, bufs["S_snap"], bufs["T_snap"], seqs, blob, bufs["sst"])
        bufs["S_snap"].mul_(0.5)                      # an eager-style change the restore undoes
        gdn.restore(d, bufs["S_snap"], bufs["T_snap"], seqs, blob, bufs["sst"])
        gdn.self_check(d1, bufs["chk"], cws, seed=7)

    xb = x.view(B, n, -1)[:, :8].contiguous()
    ab = a.view(B, n, Hv)[:, :8].contiguous()
    bb = b.view(B, n, Hv)[:, :8].contiguous()

    reset()
    torch.cuda.synchronize()
    round_of_calls()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in bufs.items()}
    assert (ref["st"].cpu().numpy() == 0).all() and (ref["cst"].cpu().numpy() == 0).all()
    assert ref["sst"].item() == 0 and (ref["chk"].cpu().numpy() == 0).all()
    assert torch.equal(ref["S_snap"], S0)

    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        round_of_calls()
    for replay in range(3):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in bufs.items():
            r = ref[k]
            same = torch.equal(v.view(torch.int32), r.view(torch.int32)) if v.dtype == torch.float32 else \
                torch.equal(v, r)
            assert same, f"replay {replay}: {k} differs from the eager calls"
