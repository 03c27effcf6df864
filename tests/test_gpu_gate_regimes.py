"""GPU parity at the ends of the gates' ranges, every call against the oracle.

The pages' workloads draw both gate inputs from N(0,1): the median decay is
then 1/2 per token, the state forgets within a few tokens, and rounding
differences between the chunked, tree and token-by-token forms die out
before they can grow.  The CPU page ("Serving a research architecture on
CPU", exactness section) warns that the chunked and sequential forms round
differently; these tests look where that matters most:
  long_memory    alpha -> 1: the state carries every token's rounding on
  strong_decay   alpha -> 0: gate products underflow inside a chunk or path
  beta_one       beta -> 1: a key's old value is replaced outright
  beta_zero      beta -> 0: writes almost vanish, the state only decays
  long_beta_one  both of the first and third
Tolerances are the same as everywhere (normwise per tensor: each step's o,
each node's o, the state; 1e-4 for decode, verify and commit, 2e-3 for the
chunked prefill), and integer/bitwise requirements are unchanged.  Each
case prints its measured error.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import oracle
from gdn_inputs import QWEN27B_LAYER, LayerShape
from tests.conftest import normwise

pytestmark = pytest.mark.gpu

TOL = 1e-4
TOL_PREFILL = 2e-3
REGIMES = ["long_memory", "strong_decay", "beta_one", "beta_zero", "long_beta_one"]
SMALL = LayerShape(2, 6, 128, 128, 4, "bf16")
ORACLE_THREADS = 16


def _seq_major(arr):
    return np.ascontiguousarray(np.swapaxes(arr, 0, 1))


def _same_bits(u, v):
    return torch.equal(u.contiguous().view(torch.int32), v.contiguous().view(torch.int32))


@pytest.mark.parametrize("gates", REGIMES)
def test_decode_chained_steps(gates):
    """512 chained decode steps of the 27B-class layer (all heads, two sequences),
    through the fused token call, each step's o and the final state against the oracle."""
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import act_to_dev, act_to_host, dims_of, f32_to_dev
    steps, B = 512, 2
    inp = gi.decode_inputs(300 + REGIMES.index(gates), QWEN27B_LAYER, B, steps, gates=gates)
    d = dims_of(QWEN27B_LAYER, B)
    S = f32_to_dev(inp.state)
    tails = [act_to_dev(inp.tail), act_to_dev(inp.tail)]
    w, x, a, b = act_to_dev(inp.w), act_to_dev(inp.x), f32_to_dev(inp.a), f32_to_dev(inp.b)
    o = torch.empty(steps, B, 48, 128, device="cuda")
    for t in range(steps):
        gdn.decode_token(d, S, tails[t % 2], tails[1 - t % 2], w, x[t], a[t], b[t], o[t])
    torch.cuda.synchronize()
    og, Sg, tg = o.cpu().numpy(), S.cpu().numpy(), act_to_host(tails[steps % 2])
    worst = 0.0
    for s in range(B):
        o_r, S_r, t_r = oracle.run_parallel(QWEN27B_LAYER, inp.state[s], inp.tail[s], inp.w, inp.x[:, s],
                                            inp.a[:, s], inp.b[:, s], threads=ORACLE_THREADS)
        errs = [normwise(og[t, s], o_r[t]) for t in range(steps)]
        err_s = normwise(Sg[s], S_r)
        worst = max(worst, max(errs), err_s)
        assert max(errs) < TOL, f"seq {s}: step {int(np.argmax(errs))} o error {max(errs):.3e}"
        assert err_s < TOL, f"seq {s}: state error {err_s:.3e}"
        assert np.array_equal(oracle.f64(tg[s]), t_r)
        assert np.all(np.isfinite(og[:, s]))
    print(f"[gate regimes] decode {gates}: worst normwise error {worst:.3e}")


@pytest.mark.parametrize("gates", REGIMES)
@pytest.mark.parametrize("ut", [False, True, "one_launch"], ids=["walk", "ut", "ut_one_launch"])
def test_tree_verify_and_commit(gates, ut):
    """Three 32-node trees of the 27B-class layer: every node's o (per node, normwise)
    against the oracle's path replay, in the exact-walk and the UT form (with a
    workspace, and in one launch without); the commit of each accepted path against
    the oracle and, bit for bit, against the walk's path rows and a token-by-token
    replay (after the one-launch form, which prepares nothing, gdn_commit_path)."""
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import act_to_host, i32_to_dev
    from tests.test_gpu_tree_batch import batch_case, decode_path, one_case, row_len
    B, n = 3, 32
    inp = gi.tree_batch_inputs(320 + REGIMES.index(gates), QWEN27B_LAYER, B, n, gates=gates)
    c = batch_case(inp)
    d = c["d"]
    o = torch.full((B, n, 48, 128), float("nan"), device="cuda")
    st = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(gdn.tree_workspace_bytes(d, n), dtype=torch.uint8, device="cuda")
    one = ut == "one_launch"
    (gdn.tree_verify_ut if ut else gdn.tree_verify)(d, c["S"], c["tail"], c["w"], c["parent"], c["x"], c["a"],
                                                    c["b"], o, st, None if one else ws)
    path = inp.extra["path"]
    S, tail = c["S"].clone(), c["tail"].clone()
    L = path.shape[1]
    oc = torch.full((B, L, 48, 128), float("nan"), device="cuda")
    cst = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    if one:
        gdn.commit_path(d, S, tail, c["w"], c["parent"], c["x"], c["a"], c["b"], i32_to_dev(path), oc, cst)
    else:
        gdn.commit_path_prepared(d, S, tail, c["parent"], c["x"], i32_to_dev(path), ws, oc, cst)
    torch.cuda.synchronize()
    assert (st.cpu().numpy() == 0).all() and (cst.cpu().numpy() == 0).all()
    og = o.cpu().numpy()
    worst = 0.0
    for s in range(B):
        ref = oracle.tree_verify(inp.shape, inp.state[s], inp.tail[s], inp.w, inp.extra["parent"][s], inp.x[:, s],
                                 inp.a[:, s], inp.b[:, s])
        for node in range(n):
            err = normwise(og[s, node], ref[node])
            worst = max(worst, err)
            assert err < TOL, f"sequence {s} node {node}: error {err:.3e}"
        Ls = row_len(path[s])
        o_r, S_r, t_r = oracle.commit_path(inp.shape, inp.state[s], inp.tail[s], inp.w, inp.extra["parent"][s],
                                           inp.x[:, s], inp.a[:, s], inp.b[:, s], path[s, :Ls])
        err_s = normwise(S[s].cpu().numpy(), S_r)
        worst = max(worst, err_s)
        assert err_s < TOL, f"sequence {s}: committed state error {err_s:.3e}"
        assert np.array_equal(oracle.f64(act_to_host(tail[s])), t_r)
        o_d, S_d, t_d = decode_path(one_case(inp, s), path[s, :Ls])
        assert _same_bits(S[s], S_d) and torch.equal(tail[s], t_d), f"sequence {s}: commit != decode"
        assert _same_bits(oc[s, :Ls], o_d)
        if not ut:
            assert _same_bits(o[s, path[s, Ls - 1]], o_d[-1]), f"sequence {s}: walk row != decode row"
    print(f"[gate regimes] tree {'ut one launch' if one else 'ut' if ut else 'walk'} {gates}: "
          f"worst normwise error {worst:.3e}")


@pytest.mark.parametrize("gates", REGIMES)
def test_block_verify_and_commit(gates):
    """32-token blocks at batch 2: the walk and the UT form (with a workspace, and in
    one launch without) against the oracle's chained decode (per position, normwise),
    the walk bit for bit against decode, and a commit of 21 tokens bit for bit against
    decode."""
    import gated_deltanet_decode_amd as gdn
    from tests.test_gpu_block import commit, decode, dev, verify
    B, k = 2, 32
    inp = gi.decode_inputs(340 + REGIMES.index(gates), QWEN27B_LAYER, B, k, gates=gates)
    c = dev(inp)
    d = c["d"]
    o_walk = verify(c, k)
    o_ut = torch.full_like(o_walk, float("nan"))
    ws = torch.empty(gdn.block_workspace_bytes(d, k), dtype=torch.uint8, device="cuda")
    gdn.block_verify_ut(d, c["S"], c["T"], c["w"], c["x"], c["a"], c["b"], o_ut, ws)
    o_one = torch.full_like(o_walk, float("nan"))
    gdn.block_verify_ut(d, c["S"], c["T"], c["w"], c["x"], c["a"], c["b"], o_one)
    torch.cuda.synchronize()
    outs, states, tails = decode(c, k)
    worst = 0.0
    for s in range(B):
        o_r, _, _ = oracle.run(inp.shape, inp.state[s], inp.tail[s], inp.w, inp.x[:, s], inp.a[:, s], inp.b[:, s])
        for t in range(k):
            for og in (o_walk, o_ut, o_one):
                err = normwise(og[s, t].cpu().numpy(), o_r[t])
                worst = max(worst, err)
                assert err < TOL, f"sequence {s} position {t}: error {err:.3e}"
            assert _same_bits(o_walk[s, t], outs[t][s])
    _, S, T, st = commit(c, k, [21, 21])
    assert (st == 0).all()
    assert _same_bits(S, states[20]) and torch.equal(T, tails[20])
    print(f"[gate regimes] block {gates}: worst normwise error {worst:.3e}")


def _prefill(inp, T):
    import gated_deltanet_decode_amd as gdn
    from tests.gpu_util import act_to_dev, dims_of, f32_to_dev
    shape = inp.shape
    d = dims_of(shape, 1)
    S, tail = f32_to_dev(inp.state), act_to_dev(inp.tail)
    x = act_to_dev(_seq_major(inp.x[:T]))
    a, b = f32_to_dev(_seq_major(inp.a[:T])), f32_to_dev(_seq_major(inp.b[:T]))
    o = torch.full((1, T, shape.num_v_heads, shape.head_v_dim), float("nan"), device="cuda")
    ws = torch.empty(gdn.prefill_workspace_bytes(d, T), dtype=torch.uint8, device="cuda")
    gdn.prefill_chunked(d, S, tail, act_to_dev(inp.w), x, a, b, o, ws)
    torch.cuda.synchronize()
    return o, S, tail


@pytest.mark.parametrize("gates", REGIMES)
@pytest.mark.parametrize("shape,T,state_sigma", [(SMALL, 4100, 0.1), (QWEN27B_LAYER, 4096, 0.0)],
                         ids=["small_4100_from_random_state", "27b_4096_fresh"])
def test_prefill(gates, shape, T, state_sigma):
    """Prompts of 4,096+ tokens (64+ chunks, so rounding can build up from chunk to
    chunk), all heads: every output and the final state against the oracle."""
    from tests.gpu_util import act_to_host
    inp = gi.prefill_inputs(360 + REGIMES.index(gates), shape, T, state_sigma=state_sigma,
                            tail_random=state_sigma > 0, gates=gates)
    o, S, tail = _prefill(inp, T)
    o_r, S_r, t_r = oracle.run_parallel(shape, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0], inp.a[:, 0],
                                        inp.b[:, 0], threads=ORACLE_THREADS)
    og = o[0].cpu().numpy()
    err_o = normwise(og, o_r)
    err_s = normwise(S[0].cpu().numpy(), S_r)
    print(f"[gate regimes] prefill {gates} T={T}: o error {err_o:.3e}, state error {err_s:.3e}")
    assert np.all(np.isfinite(og))
    assert err_o < TOL_PREFILL, f"o error {err_o:.3e}"
    assert err_s < TOL_PREFILL, f"state error {err_s:.3e}"
    assert np.array_equal(oracle.f64(act_to_host(tail)[0]), t_r)


@pytest.mark.parametrize("gates", ["long_memory", "long_beta_one"])
def test_prefill_32768_long_memory(gates):
    """The long-prompt shape (27B-class layer, T = 32,768 from a fresh state) where the
    state remembers: o on the first 2,048 tokens and the whole final state (all 48
    heads) against the oracle over all 32,768 tokens."""
    from tests.gpu_util import act_to_host
    T = 32768
    inp = gi.prefill_inputs(380 + REGIMES.index(gates), QWEN27B_LAYER, T, gates=gates)
    o, S, tail = _prefill(inp, T)
    og = o[0, :2048].cpu().numpy()
    assert torch.isfinite(o).all()
    del o
    o_r, _, _ = oracle.run_parallel(QWEN27B_LAYER, inp.state[0], inp.tail[0], inp.w, inp.x[:2048, 0],
                                    inp.a[:2048, 0], inp.b[:2048, 0], threads=ORACLE_THREADS)
    _, S_r, t_r = oracle.run_parallel(QWEN27B_LAYER, inp.state[0], inp.tail[0], inp.w, inp.x[:, 0], inp.a[:, 0],
                                      inp.b[:, 0], want_o=False, threads=ORACLE_THREADS)
    err_o = normwise(og, o_r)
    err_s = normwise(S[0].cpu().numpy(), S_r)
    print(f"[gate regimes] prefill {gates} T=32768: o[0:2048] error {err_o:.3e}, final state error {err_s:.3e}")
    assert err_o < TOL_PREFILL
    assert err_s < TOL_PREFILL
    assert np.array_equal(oracle.f64(act_to_host(tail)[0]), t_r)
