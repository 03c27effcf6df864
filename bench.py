#!/usr/bin/env python3
"""Throughput of the Gated DeltaNet mixer library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rows ...]

The headline line is one decode step of one 27B-class recurrent layer at
batch 1 (16 q/k heads and 48 value heads of 128, fp32 state of 3.15 MB, bf16
activations and conv tail), repeated for K chained steps: a step is one
gdn_decode_token call (conv update, q/k norm, gates and state step in one
launch; bit-identical to gdn_conv_update + gdn_decode_step).  Each step
advances the next of R independent states (R * 3.15 MB > the 256 MB Infinity
Cache), so every step reads its state from HBM, as it would in a model with
48 such layers and weights streaming in between.  The value is algorithmic
GB/s: bytes the step must move (state read + write, x, conv tail in and out,
weights, gates, o) over the time.

Extra rows, each with its own roofline fraction: the same step under a hip
graph and as two calls, the state step alone, batch-64 decode (ping-pong
over two batches), 32-node tree verify and path commit at batch 1 and over
64 sequences' trees, 16-token block verify and commit, snapshot and restore
of 64 sequences, chunked prefill
at T = 32,768; and the CPU oracle on a bounded sample as the host baseline.
Inputs are seeded synthetic tensors of the workload's shapes.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, published
MFMA_FP16_TFLOPS = 2500.0  # dense fp16/bf16 MFMA, published

SHAPE_DESC = {"num_k_heads": 16, "num_v_heads": 48, "head_k_dim": 128, "head_v_dim": 128, "conv_width": 4}


def step_bytes(B, shape):
    """Algorithmic bytes of one decode step (state step + conv update) for B sequences."""
    Hv, D, C = shape.num_v_heads, shape.head_k_dim, shape.conv_channels
    state = 2 * Hv * D * D * 4
    dec_vec = C * 4 + 2 * Hv * 4 + Hv * D * 4          # y, a, b in; o out
    conv = C * 2 + 2 * C * 4 * 2 + C * 4               # x in, tail in+out, y out (bf16 tail)
    conv_w = C * 4 * 2                                  # weights, read once per launch
    return B * (state + dec_vec), B * conv + conv_w


def token_bytes(B, shape):
    """Algorithmic bytes of one fused token (gdn_decode_token) for B sequences: state read +
    write, x, conv tail in + out (bf16), a, b, o; the conv weights once per launch."""
    Hv, D, C = shape.num_v_heads, shape.head_k_dim, shape.conv_channels
    per_seq = 2 * Hv * D * D * 4 + C * 2 + 2 * C * 4 * 2 + 2 * Hv * 4 + Hv * D * 4
    return B * per_seq + C * 4 * 2


def kda_token_bytes(B, shape):
    """gdn_kda_decode_token: token_bytes with the forget-gate input a widened from one value
    per value head to one per (value head, key channel)."""
    Hv, D = shape.num_v_heads, shape.head_k_dim
    return token_bytes(B, shape) + B * Hv * (D - 1) * 4


def tree_bytes(n, shape, B=1):
    """Algorithmic bytes of one tree verify over B sequences' trees of n nodes: per sequence the
    checkpoint read once, x, conv tail (bf16), gates, parent and o; the conv weights once."""
    Hv, D, C = shape.num_v_heads, shape.head_k_dim, shape.conv_channels
    per_seq = Hv * D * D * 4 + n * C * 2 + C * 4 * 2 + 2 * n * Hv * 4 + n * Hv * D * 4 + n * 4
    return B * per_seq + C * 4 * 2


def block_bytes(k, shape, B=1):
    """Algorithmic bytes of one block verify of k tokens over B sequences: per sequence the
    checkpoint read once, the tail, k rows of x, gates and o; the conv weights once."""
    Hv, D, C = shape.num_v_heads, shape.head_k_dim, shape.conv_channels
    per_seq = Hv * D * D * 4 + C * 4 * 2 + k * (C * 2 + 2 * Hv * 4 + Hv * D * 4)
    return B * per_seq + C * 4 * 2


def commit_bytes(lens, shape):
    """Algorithmic bytes of one commit without per-token outputs (o = NULL, the caller has them
    from verify): per sequence with L accepted tokens the state read and written, the conv
    tail read and written, L rows of x and gates; the conv weights once."""
    Hv, D, C = shape.num_v_heads, shape.head_k_dim, shape.conv_channels
    return sum(2 * Hv * D * D * 4 + 2 * C * 4 * 2 + L * (C * 2 + 2 * Hv * 4) for L in lens) + C * 4 * 2


COUNTERS = os.path.join(ROOT, "profiles", "token_kernel_b1_27b_layer_counters.md")
TOKEN_SOURCES = [os.path.join(ROOT, "gated_deltanet_decode_amd", "csrc", f) for f in ("gdn_token.hip", "gdn_core.hpp")]


def counter_traffic():
    """HBM bytes per launch of the batch-1 fused token kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary (copy-calibrated), or None when the kernel
    sources no longer hash to what was profiled."""
    import hashlib
    try:
        line = next(l for l in open(COUNTERS) if l.startswith("traffic-json:"))
        rec = json.loads(line.split(":", 1)[1])
        sha = hashlib.sha256(b"".join(open(f, "rb").read() for f in TOKEN_SOURCES)).hexdigest()
    except (OSError, StopIteration, ValueError):
        return None
    return rec["bytes_per_launch"] if rec.get("sources_sha256") == sha else None


class Timer:
    """HIP events on the stream the work is launched on.  With lead_in (a function that
    queues a long device operation, such as the cache eviction), the start event is queued
    behind it without a host synchronisation in between: while the GPU runs the lead-in,
    the host queues the start event and the timed launches, so the events time the device
    work of the timed steps, not the host's submission of them.  The region is still
    bracketed by synchronisations."""

    def __init__(self, torch, lead_in=None):
        self.torch = torch
        self.lead_in = lead_in
        self.s = torch.cuda.Event(enable_timing=True)
        self.e = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.torch.cuda.synchronize()
        if self.lead_in is not None:
            self.lead_in()
        self.s.record(self.torch.cuda.current_stream())
        return self

    def __exit__(self, *a):
        self.e.record(self.torch.cuda.current_stream())
        self.torch.cuda.synchronize()
        self.ms = self.s.elapsed_time(self.e)


def graph_time_us(torch, fn, n, reps=4):
    """Capture fn(0..n-1) into one hip graph, replay it `reps` times; microseconds per call.
    Replays skip the host-side cost of each call, so this is the device-side rate."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(3):
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    g.replay()
    with Timer(torch) as tm:
        for _ in range(reps):
            g.replay()
    del g
    return tm.ms * 1e3 / (reps * n)


def cold_graph_ms(torch, fn, n, evict):
    """Capture fn(0..n-1) into one hip graph, replay it twice untimed, then time one replay
    on the current stream right behind a cache eviction (evict() queues it); milliseconds."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    g.replay()
    g.replay()
    with Timer(torch, lead_in=evict) as tm:
        g.replay()
    del g
    return tm.ms


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4096)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--buffers", type=int, default=160, help="independent states rotated through (cold runs)")
    ap.add_argument("--rows", default="all", help="comma list of extra rows: graph,kernel,b64,kda,tree,commit,tree64,block,snapshot,prefill,hot,cpu or all/none")
    ap.add_argument("--copy-calibration", action="store_true", help="also run a plain 512 MiB device copy (for byte counters)")
    ap.add_argument("--details", default=None, help="write the full results JSON here")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (the mixer shards by q/k head "
              "groups with no exchange; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_deltanet_decode_amd as gdn
    import gdn_inputs as gi

    rows = set(["graph", "kernel", "b64", "kda", "tree", "commit", "tree64", "block", "snapshot", "prefill", "hot", "cpu"]) \
        if args.rows == "all" else \
        set() if args.rows == "none" else set(args.rows.split(","))
    dev = "cuda"
    torch.cuda.set_device(0)
    shape = gi.QWEN27B_LAYER
    K, W, R = args.steps, args.warmup, args.buffers
    C, Hv, D = shape.conv_channels, shape.num_v_heads, shape.head_k_dim

    def act(arr):
        arr = np.ascontiguousarray(arr)
        return torch.from_numpy(arr.view(np.int16)).to(dev).view(torch.bfloat16)

    def f32(arr):
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(dev)

    # ---------------------------------------------------------------- inputs
    t0 = time.time()

    def note(what):
        """Progress on stderr, so a long run shows it is alive (the JSON line is stdout's only line)."""
        print(f"[bench] {what} at {time.time() - t0:.0f} s", file=sys.stderr, flush=True)
    steps_total = K + W
    inp = gi.decode_inputs(1, shape, 1, steps_total, state_sigma=0.1, tail_random=True)
    pool = gi.decode_inputs(101, shape, R, 1, state_sigma=0.1, tail_random=True)  # R independent states
    x = act(inp.x[:, 0])
    a = f32(inp.a[:, 0])
    b = f32(inp.b[:, 0])
    w = act(inp.w)
    S_pool = f32(pool.state)
    tail_pool = act(pool.tail)
    tail_pool2 = torch.empty_like(tail_pool)
    tails = (tail_pool, tail_pool2)
    cnt = [0] * R   # steps applied to each state: its current tail is tails[cnt % 2]
    del pool
    d1 = gdn.dims(1, 16, 48, 128, 128, 4, "bf16")
    y = torch.empty(1, C, device=dev)
    o = torch.empty(1, Hv, D, device=dev)
    gen_s = time.time() - t0

    def step(t, r):
        """One token on state r: the fused call, the tail going from one buffer to the other."""
        i = cnt[r] % 2
        gdn.decode_token(d1, S_pool[r], tails[i][r], tails[1 - i][r], w, x[t], a[t], b[t], o)
        cnt[r] += 1

    def step_two_calls(t, r):
        """The same token through gdn_conv_update + gdn_decode_step (tail in place)."""
        tail = tails[cnt[r] % 2][r]
        gdn.conv_update(d1, x[t], tail, w, y)
        gdn.decode_step(d1, S_pool[r], y, a[t], b[t], o)

    res = {}
    per_step = token_bytes(1, shape)
    dec_b, conv_b = step_bytes(1, shape)

    # ---------------------------------------------------------------- headline: cold, eager launches
    evict_src = torch.empty(1 << 28, dtype=torch.float32, device=dev)    # 1 GiB
    evict_dst = torch.empty_like(evict_src)

    def evict():
        """Push every earlier state out of the 256 MB Infinity Cache (outside any timed region)."""
        evict_dst.copy_(evict_src)

    for t in range(W):
        step(t, t % R)
    with Timer(torch, lead_in=evict) as tm:
        for t in range(W, W + K):
            step(t, t % R)
    cold_ms = tm.ms
    res["decode_b1_cold_eager"] = {"ms_per_step": cold_ms / K, "GBps": per_step * K / cold_ms / 1e6,
                                   "tokens_per_s": K / cold_ms * 1e3}

    # ---------------------------------------------------------------- same steps under a hip graph
    # One graph of exactly the K timed steps, step t on state t % R.  It is
    # replayed twice untimed (an even number, so every state's tail is back in
    # the buffer the captured steps read first), then the 256 MB Infinity Cache
    # is evicted by a 1 GiB device copy, and one replay is timed: every state
    # the timed steps touch is read from HBM.
    graph_ms = None
    note("graph")
    if "graph" in rows:
        ms = cold_graph_ms(torch, lambda t: step(W + t, t % R), K, evict)
        graph_ms = ms
        res["decode_b1_cold_graph"] = {"ms_per_step": ms / K, "GBps": per_step * K / ms / 1e6,
                                       "tokens_per_s": K / ms * 1e3, "graph_steps": K,
                                       "distinct_states": min(K, R)}
        # The same steps rotated over all R states twice (2R steps), whatever K is.
        ms2 = cold_graph_ms(torch, lambda t: step(W + t % K, t % R), 2 * R, evict)
        res["decode_b1_cold_graph_all_states"] = {"ms_per_step": ms2 / (2 * R), "GBps": per_step * 2 * R / ms2 / 1e6,
                                                  "tokens_per_s": 2 * R / ms2 * 1e3, "graph_steps": 2 * R,
                                                  "distinct_states": R,
                                                  "states_bytes": R * Hv * D * D * 4}
        us2 = graph_time_us(torch, lambda t: step_two_calls(W + t % K, t % R), 2 * R, reps=2)
        res["decode_b1_two_calls_graph"] = {"ms_per_step": us2 / 1e3, "GBps": (dec_b + conv_b) / us2 / 1e3,
                                            "tokens_per_s": 1e6 / us2, "calls": "gdn_conv_update + gdn_decode_step",
                                            "graph_steps": 2 * R}

    # ---------------------------------------------------------------- the state-step kernel alone
    note("kernel")
    if "kernel" in rows:
        yk = torch.empty(R, 1, C, device=dev)
        for r in range(R):
            gdn.conv_update(d1, x[r % steps_total], tails[cnt[r] % 2][r], w, yk[r])
        us = graph_time_us(torch, lambda t: gdn.decode_step(d1, S_pool[t % R], yk[t % R], a[t % steps_total],
                                                             b[t % steps_total], o), 512, reps=max(1, K // 512))
        res["decode_b1_state_step_kernel"] = {"kernel": "decode_kernel<128,1>", "bytes_per_launch": dec_b,
                                              "us_per_launch_graph": us, "GBps": dec_b / us / 1e3,
                                              "frac_hbm": dec_b / us / 1e3 / HBM_PEAK_GBS}
        del yk

    # ---------------------------------------------------------------- hot: one state buffer
    note("hot")
    if "hot" in rows:
        S1 = S_pool[0].clone()
        th = (tails[cnt[0] % 2][0].clone(), tails[cnt[0] % 2][0].clone())
        for t in range(W):
            gdn.decode_token(d1, S1, th[t % 2], th[1 - t % 2], w, x[t], a[t], b[t], o)
        with Timer(torch) as tm:
            for t in range(W, W + K):
                gdn.decode_token(d1, S1, th[t % 2], th[1 - t % 2], w, x[t], a[t], b[t], o)
        res["decode_b1_hot_eager"] = {"ms_per_step": tm.ms / K, "GBps": per_step * K / tm.ms / 1e6,
                                      "note": "one 3.15 MB state: served from cache, not HBM"}

    # ---------------------------------------------------------------- per-channel decay at batch 1
    # The same cold graph as decode_b1_cold_graph_all_states (2R steps over the R
    # states, Infinity Cache evicted before the timed replay), through
    # gdn_kda_decode_token with one gate input per (value head, key channel).
    note("kda")
    if "kda" in rows:
        ak = f32(gi.channel_gates(5, shape, 1, 2 * R)[:, 0])
        kb = kda_token_bytes(1, shape)

        def kda_step(t, r):
            i = cnt[r] % 2
            gdn.kda_decode_token(d1, S_pool[r], tails[i][r], tails[1 - i][r], w, x[W + t % K], ak[t],
                                 b[W + t % K], o)
            cnt[r] += 1

        ms = cold_graph_ms(torch, lambda t: kda_step(t, t % R), 2 * R, evict)
        res["kda_decode_b1_cold_graph"] = {"ms_per_step": ms / (2 * R), "GBps": kb * 2 * R / ms / 1e6,
                                           "tokens_per_s": 2 * R / ms * 1e3, "graph_steps": 2 * R,
                                           "distinct_states": R, "bytes_per_token": kb,
                                           "call": "gdn_kda_decode_token"}
        del ak

    # ---------------------------------------------------------------- batch 64, ping-pong over two batches
    note("b64")
    if "b64" in rows:
        B = 64
        steps64 = 256
        del S_pool  # make room; tree/commit use their own pool below
        S_pool = None
        inp64 = gi.decode_inputs(2, shape, 2 * B, 1, state_sigma=0.1, tail_random=True)
        S64 = f32(inp64.state).view(2, B, Hv, D, D)
        T64 = act(inp64.tail).view(2, B, C, 4)
        w64 = act(inp64.w)
        del inp64
        xs = gi.decode_inputs(3, shape, B, steps64 + 16, state_sigma=0.0, tail_random=False)
        x64, a64, b64 = act(xs.x), f32(xs.a), f32(xs.b)
        del xs
        d64 = gdn.dims(B, 16, 48, 128, 128, 4, "bf16")
        y64 = torch.empty(B, C, device=dev)
        o64 = torch.empty(B, Hv, D, device=dev)

        tails64 = (T64, torch.empty_like(T64))
        cnt64 = [0, 0]

        def step64(t):
            p = t % 2
            i = cnt64[p] % 2
            gdn.decode_token(d64, S64[p], tails64[i][p], tails64[1 - i][p], w64, x64[t], a64[t], b64[t], o64)
            cnt64[p] += 1

        db, cb = step_bytes(B, shape)
        tb = token_bytes(B, shape)
        us = graph_time_us(torch, lambda t: step64(16 + t), steps64, reps=2)
        res["decode_b64"] = {"ms_per_step": us / 1e3, "GBps": tb / us / 1e3,
                             "tokens_per_s": B / us * 1e6, "frac_hbm": tb / us / 1e3 / HBM_PEAK_GBS,
                             "launch": "hipGraph", "call": "gdn_decode_token",
                             "state_buffers": "2 batches of 64 (ping-pong, 403 MB)"}
        us = graph_time_us(torch, lambda t: gdn.decode_step(d64, S64[t % 2], y64, a64[t], b64[t], o64), steps64,
                           reps=2)
        res["decode_b64"]["kernel_us"] = us
        res["decode_b64"]["kernel_GBps"] = db / us / 1e3
        res["decode_b64"]["kernel_frac_hbm"] = db / us / 1e3 / HBM_PEAK_GBS
        # the same steps in place on one batch of 64 states (201 MB, which fits the 256 MB Infinity Cache)
        cnt_ip = [0]

        def step64_in_place(t):
            i = cnt_ip[0] % 2
            gdn.decode_token(d64, S64[0], tails64[i][0], tails64[1 - i][0], w64, x64[t], a64[t], b64[t], o64)
            cnt_ip[0] += 1

        us = graph_time_us(torch, lambda t: step64_in_place(16 + t), steps64, reps=2)
        res["decode_b64_in_place"] = {"ms_per_step": us / 1e3, "GBps": tb / us / 1e3,
                                      "tokens_per_s": B / us * 1e6, "frac_hbm": tb / us / 1e3 / HBM_PEAK_GBS,
                                      "launch": "hipGraph", "call": "gdn_decode_token",
                                      "state_buffers": "1 batch of 64 in place (201 MB: may be served from the "
                                                       "Infinity Cache rather than HBM)"}
        if "kda" in rows:
            ak64 = f32(gi.channel_gates(6, shape, B, steps64 + 16))

            def kda64(t):
                p = t % 2
                i = cnt64[p] % 2
                gdn.kda_decode_token(d64, S64[p], tails64[i][p], tails64[1 - i][p], w64, x64[t], ak64[t], b64[t],
                                     o64)
                cnt64[p] += 1

            kb = kda_token_bytes(B, shape)
            us = graph_time_us(torch, lambda t: kda64(16 + t), steps64, reps=2)
            res["kda_decode_b64"] = {"ms_per_step": us / 1e3, "GBps": kb / us / 1e3,
                                     "tokens_per_s": B / us * 1e6, "frac_hbm": kb / us / 1e3 / HBM_PEAK_GBS,
                                     "launch": "hipGraph", "call": "gdn_kda_decode_token",
                                     "state_buffers": "2 batches of 64 (ping-pong, 403 MB)"}
            del ak64
        del S64, T64, tails64, x64, a64, b64, y64, o64

    # ---------------------------------------------------------------- tree verify + commit
    note("tree")
    if "tree" in rows or "commit" in rows:
        tin = gi.tree_inputs(3, shape, n_nodes=32, max_depth=8)
        pool = gi.decode_inputs(103, shape, R, 1, state_sigma=0.1, tail_random=True)
        Sp = f32(pool.state)
        Tp = act(pool.tail)
        del pool
        parent = torch.from_numpy(tin.extra["parent"]).to(dev)
        path = torch.from_numpy(tin.extra["path"]).to(dev)
        L = int(path.numel())
        xt, at, bt, wt = act(tin.x[:, 0]), f32(tin.a[:, 0]), f32(tin.b[:, 0]), act(tin.w)
        ot = torch.empty(32, Hv, D, device=dev)
        st = torch.zeros(1, dtype=torch.int32, device=dev)
        tws = torch.empty(gdn.tree_workspace_bytes(d1, 32), dtype=torch.uint8, device=dev)
        nrep = 512
        if "tree" in rows:
            us = graph_time_us(torch, lambda r: gdn.tree_verify(d1, Sp[r % R], Tp[r % R], wt, parent, xt, at, bt,
                                                                 ot, st, tws), nrep)
            tb = tree_bytes(32, shape)
            res["tree_verify_n32"] = {"us": us, "GBps": tb / us / 1e3, "frac_hbm": tb / us / 1e3 / HBM_PEAK_GBS,
                                      "nodes_per_s": 32 / us * 1e6, "bytes": tb, "launch": "hipGraph"}
            # The UT form in one launch (no workspace) and in two (prep into a workspace).
            for key, wsx in (("tree_verify_ut_n32", None), ("tree_verify_ut_ws_n32", tws)):
                us = graph_time_us(torch, lambda r: gdn.tree_verify_ut(d1, Sp[r % R], Tp[r % R], wt, parent, xt, at,
                                                                        bt, ot, st, wsx), nrep)
                res[key] = {"us": us, "GBps": tb / us / 1e3, "frac_hbm": tb / us / 1e3 / HBM_PEAK_GBS,
                            "nodes_per_s": 32 / us * 1e6, "bytes": tb, "launch": "hipGraph",
                            "call": "gdn_tree_verify_ut", "workspace": wsx is not None}
        if "commit" in rows:
            us = graph_time_us(torch, lambda r: gdn.commit_path(d1, Sp[r % R], Tp[r % R], wt, parent, xt, at, bt,
                                                                 path, None, st), nrep)
            cbt = commit_bytes([L], shape)
            res["commit_path"] = {"us": us, "path_len": L, "GBps": cbt / us / 1e3,
                                  "frac_hbm": cbt / us / 1e3 / HBM_PEAK_GBS, "bytes": cbt, "launch": "hipGraph"}
            if "tree_verify_n32" in res:
                res["commit_path"]["committed_tokens_per_s"] = L / (us + res["tree_verify_n32"]["us"]) * 1e6
            # the same commit reading the path's operands from the verify's workspace (the
            # workspace holds the last verify's; the work per call is the same)
            us = graph_time_us(torch, lambda r: gdn.commit_path_prepared(d1, Sp[r % R], Tp[r % R], parent, xt, path,
                                                                          tws, None, st), nrep)
            res["commit_path_prepared"] = {"us": us, "path_len": L, "GBps": cbt / us / 1e3,
                                           "frac_hbm": cbt / us / 1e3 / HBM_PEAK_GBS, "bytes": cbt,
                                           "launch": "hipGraph", "call": "gdn_commit_path_prepared"}
        assert st.item() == 0
        del Sp, Tp

    # ---------------------------------------------------------------- batched tree verify + commit
    # 64 sequences, one 32-node tree each, accepted paths of mixed lengths;
    # two batches of checkpoints (403 MB) alternate so states come from HBM.
    note("tree64")
    if "tree64" in rows:
        B = 64
        tbi = gi.tree_batch_inputs(5, shape, B, n_nodes=32, max_depth=8)
        pool = gi.decode_inputs(105, shape, 2 * B, 1, state_sigma=0.1, tail_random=True)
        S2 = f32(pool.state).view(2, B, Hv, D, D)
        T2 = act(pool.tail).view(2, B, C, 4)
        del pool
        dB = gdn.dims(B, 16, 48, 128, 128, 4, "bf16")
        seq = lambda arr: np.ascontiguousarray(np.swapaxes(arr, 0, 1))   # [n][B][...] -> [B][n][...]
        xB, aB, bB, wB = act(seq(tbi.x)), f32(seq(tbi.a)), f32(seq(tbi.b)), act(tbi.w)
        parentB = torch.from_numpy(tbi.extra["parent"]).to(dev)
        pathB = torch.from_numpy(tbi.extra["path"]).to(dev)
        lens = [int(np.argmax(r == -1)) if (r == -1).any() else len(r) for r in tbi.extra["path"]]
        oB = torch.empty(B, 32, Hv, D, device=dev)
        stB = torch.zeros(B, dtype=torch.int32, device=dev)
        wsB = torch.empty(gdn.tree_workspace_bytes(dB, 32), dtype=torch.uint8, device=dev)
        us = graph_time_us(torch, lambda r: gdn.tree_verify(dB, S2[r % 2], T2[r % 2], wB, parentB, xB, aB, bB, oB,
                                                             stB, wsB), 32, reps=2)
        tb = tree_bytes(32, shape, B)
        res["tree_verify_b64_n32"] = {"us": us, "GBps": tb / us / 1e3, "frac_hbm": tb / us / 1e3 / HBM_PEAK_GBS,
                                      "nodes_per_s": B * 32 / us * 1e6, "bytes": tb, "launch": "hipGraph",
                                      "state_buffers": "2 batches of 64 (ping-pong, 403 MB)"}
        for key, wsx in (("tree_verify_ut_b64_n32", None), ("tree_verify_ut_ws_b64_n32", wsB)):
            us = graph_time_us(torch, lambda r: gdn.tree_verify_ut(dB, S2[r % 2], T2[r % 2], wB, parentB, xB, aB, bB,
                                                                    oB, stB, wsx), 32, reps=2)
            res[key] = {"us": us, "GBps": tb / us / 1e3, "frac_hbm": tb / us / 1e3 / HBM_PEAK_GBS,
                        "nodes_per_s": B * 32 / us * 1e6, "bytes": tb, "launch": "hipGraph",
                        "call": "gdn_tree_verify_ut", "workspace": wsx is not None,
                        "state_buffers": "2 batches of 64 (ping-pong, 403 MB)"}
        us = graph_time_us(torch, lambda r: gdn.commit_path(dB, S2[r % 2], T2[r % 2], wB, parentB, xB, aB, bB, pathB,
                                                             None, stB), 32, reps=2)
        cbt = commit_bytes(lens, shape)
        res["commit_path_b64"] = {"us": us, "accepted_tokens": sum(lens), "GBps": cbt / us / 1e3,
                                  "frac_hbm": cbt / us / 1e3 / HBM_PEAK_GBS, "bytes": cbt, "launch": "hipGraph",
                                  "committed_tokens_per_s": sum(lens) / (us + res["tree_verify_b64_n32"]["us"]) * 1e6}
        us = graph_time_us(torch, lambda r: gdn.commit_path_prepared(dB, S2[r % 2], T2[r % 2], parentB, xB, pathB, wsB,
                                                                      None, stB), 32, reps=2)
        res["commit_path_prepared_b64"] = {"us": us, "accepted_tokens": sum(lens), "GBps": cbt / us / 1e3,
                                           "frac_hbm": cbt / us / 1e3 / HBM_PEAK_GBS, "bytes": cbt,
                                           "launch": "hipGraph", "call": "gdn_commit_path_prepared"}
        assert int(stB.abs().sum().item()) == 0
        del S2, T2, xB, aB, bB, oB, wsB

    # ---------------------------------------------------------------- block verify + commit, 16 tokens
    # Batch 1 rotates over the R cold states; batch 64 alternates two batches.
    note("block")
    if "block" in rows:
        kb = 16
        for B, nbuf in ((1, R), (64, 2)):
            pool = gi.decode_inputs(107, shape, nbuf * B, 1, state_sigma=0.1, tail_random=True)
            Sb = f32(pool.state).view(nbuf, B, Hv, D, D)
            Tb = act(pool.tail).view(nbuf, B, C, 4)
            del pool
            bi = gi.decode_inputs(8, shape, B, kb, state_sigma=0.0, tail_random=False)
            seqm = lambda arr: np.ascontiguousarray(np.swapaxes(arr, 0, 1))
            xB, aB, bB, wB = act(seqm(bi.x)), f32(seqm(bi.a)), f32(seqm(bi.b)), act(bi.w)
            dB = gdn.dims(B, 16, 48, 128, 128, 4, "bf16")
            oB = torch.empty(B, kb, Hv, D, device=dev)
            wsB = torch.empty(gdn.block_workspace_bytes(dB, kb), dtype=torch.uint8, device=dev)
            n = 256 if B == 1 else 32
            us = graph_time_us(torch, lambda r: gdn.block_verify(dB, Sb[r % nbuf], Tb[r % nbuf], wB, xB, aB, bB, oB,
                                                                  wsB), n, reps=2)
            vb = block_bytes(kb, shape, B)
            res[f"block_verify_b{B}_k{kb}"] = {"us": us, "GBps": vb / us / 1e3, "frac_hbm": vb / us / 1e3 / HBM_PEAK_GBS,
                                               "tokens_per_s": B * kb / us * 1e6, "bytes": vb, "launch": "hipGraph"}
            for key, wsx in ((f"block_verify_ut_b{B}_k{kb}", None), (f"block_verify_ut_ws_b{B}_k{kb}", wsB)):
                us = graph_time_us(torch, lambda r: gdn.block_verify_ut(dB, Sb[r % nbuf], Tb[r % nbuf], wB, xB, aB,
                                                                         bB, oB, wsx), n, reps=2)
                res[key] = {"us": us, "GBps": vb / us / 1e3, "frac_hbm": vb / us / 1e3 / HBM_PEAK_GBS,
                            "tokens_per_s": B * kb / us * 1e6, "bytes": vb, "launch": "hipGraph",
                            "call": "gdn_block_verify_ut", "workspace": wsx is not None}
            if B == 64:
                acc_np = np.array([(7 * s) % (kb + 1) for s in range(B)], np.int32)
                acc = torch.from_numpy(acc_np).to(dev)
                stB = torch.zeros(B, dtype=torch.int32, device=dev)
                us = graph_time_us(torch, lambda r: gdn.block_commit(dB, Sb[r % nbuf], Tb[r % nbuf], wB, xB, aB, bB,
                                                                      acc, None, stB, wsB), n, reps=2)
                cb = commit_bytes([int(L) for L in acc_np if L > 0], shape)
                res[f"block_commit_b{B}_k{kb}"] = {"us": us, "accepted_tokens": int(acc_np.sum()), "GBps": cb / us / 1e3,
                                                   "frac_hbm": cb / us / 1e3 / HBM_PEAK_GBS, "bytes": cb,
                                                   "launch": "hipGraph"}
                us = graph_time_us(torch, lambda r: gdn.block_commit_prepared(dB, Sb[r % nbuf], Tb[r % nbuf], xB, acc, wsB,
                                                                               None, stB), n, reps=2)
                res[f"block_commit_prepared_b{B}_k{kb}"] = {"us": us, "accepted_tokens": int(acc_np.sum()),
                                                            "GBps": cb / us / 1e3,
                                                            "frac_hbm": cb / us / 1e3 / HBM_PEAK_GBS, "bytes": cb,
                                                            "launch": "hipGraph", "call": "gdn_block_commit_prepared"}
                assert int(stB.abs().sum().item()) == 0
            del Sb, Tb, xB, aB, bB, oB, wsB

    # ---------------------------------------------------------------- snapshot / restore, 64 sequences
    # Save all 64 sequences of one batch into a blob and restore them into the
    # other batch; the two batches and the blob (1.2 GB) exceed the cache.
    note("snapshot")
    if "snapshot" in rows:
        B = 64
        pool = gi.decode_inputs(106, shape, 2 * B, 1, state_sigma=0.1, tail_random=True)
        S2 = f32(pool.state).view(2, B, Hv, D, D)
        T2 = act(pool.tail).view(2, B, C, 4)
        del pool
        dB = gdn.dims(B, 16, 48, 128, 128, 4, "bf16")
        seqs = torch.arange(B, dtype=torch.int32, device=dev)
        blobs = [torch.empty(gdn.snapshot_bytes(dB, B), dtype=torch.uint8, device=dev) for _ in range(2)]
        stS = torch.zeros(1, dtype=torch.int32, device=dev)
        per_seq = Hv * D * D * 4 + C * 4 * 2
        moved = 2 * B * per_seq                           # each byte read once and written once
        us_s = graph_time_us(torch, lambda r: gdn.snapshot(dB, S2[r % 2], T2[r % 2], seqs, blobs[r % 2], stS), 16,
                             reps=2)
        us_r = graph_time_us(torch, lambda r: gdn.restore(dB, S2[1 - r % 2], T2[1 - r % 2], seqs, blobs[r % 2], stS),
                             16, reps=2)
        assert stS.item() == 0
        res["snapshot_b64"] = {"us": us_s, "GBps": moved / us_s / 1e3, "frac_hbm": moved / us_s / 1e3 / HBM_PEAK_GBS,
                               "bytes": moved, "launch": "hipGraph"}
        res["restore_b64"] = {"us": us_r, "GBps": moved / us_r / 1e3, "frac_hbm": moved / us_r / 1e3 / HBM_PEAK_GBS,
                              "bytes": moved, "launch": "hipGraph"}
        del S2, T2, blobs

    # ---------------------------------------------------------------- chunked prefill
    note("prefill")
    if "prefill" in rows:
        try:
            T = 32768
            pin = gi.prefill_inputs(4, shape, T)
            dP = gdn.dims(1, 16, 48, 128, 128, 4, "bf16")
            Sx = f32(pin.state)
            Tx = act(pin.tail)
            xP, aP, bP, wP = act(pin.x), f32(pin.a), f32(pin.b), act(pin.w)
            oP = torch.empty(1, T, Hv, D, device=dev)
            ws_n = gdn.prefill_workspace_bytes(dP, T)
            ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=dev)
            gdn.prefill_chunked(dP, Sx, Tx, wP, xP, aP, bP, oP, ws)
            reps = 5
            with Timer(torch) as tm:
                for _ in range(reps):
                    gdn.prefill_chunked(dP, Sx, Tx, wP, xP, aP, bP, oP, ws)
            us = tm.ms * 1e3 / reps
            flop = prefill_flops(T, shape)
            res["prefill_t32768"] = {"us": us, "tokens_per_s": T / us * 1e6, "TFLOPs": flop / us / 1e6,
                                     "frac_mfma_fp16": flop / us / 1e6 / MFMA_FP16_TFLOPS}
        except Exception as e:  # reported, not hidden
            res["prefill_t32768"] = {"error": str(e)}

    # ---------------------------------------------------------------- copy calibration for byte counters
    if args.copy_calibration:
        n = 512 * 1024 * 1024 // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = {"read": n * 4, "write": n * 4, "launches": 4}
        del src, dst

    # ---------------------------------------------------------------- CPU oracle on a bounded sample
    # The oracle (fp64 scalar C, unchanged) runs chained batch-1 decode steps of
    # the same layer, all 48 heads, cycling over the drawn tokens: first on one
    # host core (this thread pinned to one CPU), then on every core the process
    # may use, its heads split by q/k head group over threads (each head keeps
    # its own token order, so the results are the same numbers).
    cpu = None
    note("cpu")
    if "cpu" in rows:
        import oracle
        oracle.build(force=False)
        cpus = sorted(os.sched_getaffinity(0))
        host = {"nproc": len(cpus), "cpu_model": _cpu_model(), "oracle_cflags": " ".join(oracle.CFLAGS),
                "compiler": _gcc_version()}

        def leg(budget_s, threads):
            tok, S0, tail0 = 0, inp.state[0], inp.tail[0]
            chunk = 8 if threads == 1 else 64
            t0 = time.time()
            while time.time() - t0 < budget_s:
                j = tok % (steps_total - steps_total % chunk) if steps_total >= chunk else 0
                xs, as_, bs = inp.x[j:j + chunk, 0], inp.a[j:j + chunk, 0], inp.b[j:j + chunk, 0]
                if threads == 1:
                    _, S0, tail0 = oracle.run(shape, S0, tail0, inp.w, xs, as_, bs)
                else:
                    _, S0, tail0 = oracle.run_parallel(shape, S0, tail0, inp.w, xs, as_, bs, threads=threads)
                tok += xs.shape[0]
            return tok, time.time() - t0

        os.sched_setaffinity(0, {cpus[0]})
        try:
            tok1, el1 = leg(10.0, 1)
        finally:
            os.sched_setaffinity(0, set(cpus))
        nthr = min(len(cpus), shape.num_k_heads)
        tokn, eln = leg(10.0, nthr)
        one = {"value": round(per_step * tok1 / el1 / 1e9, 3), "unit": "GB/s", "cores": 1,
               "tokens_per_s": round(tok1 / el1, 1), "tokens": tok1, "seconds": round(el1, 1)}
        cpu = {"value": round(per_step * tokn / eln / 1e9, 3), "unit": "GB/s", "cores": nthr, "kind": "oracle",
               "tokens_per_s": round(tokn / eln, 1),
               "sample": f"{tokn} chained decode steps of the batch-1 27B-class layer (all 48 heads, fp64 scalar "
                         f"C, cycling over the {steps_total} drawn tokens) in {eln:.1f} s, the heads split by q/k "
                         f"head group over {nthr} host threads; the one-core leg ran {tok1} steps in {el1:.1f} s",
               "one_core": one, "host": host}

    # ---------------------------------------------------------------- the line
    best_ms = cold_ms if graph_ms is None else min(cold_ms, graph_ms)
    launch = "eager" if graph_ms is None or cold_ms <= graph_ms else "hipGraph"
    value = per_step * K / best_ms / 1e6
    # The headline step is one launch of the fused token kernel, so its per-step
    # time (HIP events over the timed region) is that kernel's launch time.
    us = best_ms * 1e3 / K
    ach = per_step / us / 1e3
    roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": counter_traffic(),
            "kernel": "token_kernel<128,1,bf16>", "bytes_per_launch": per_step, "us_per_launch": round(us, 3)}
    line = {
        "metric": "GDN state GB/s & tokens/s per layer (decode, 32-node tree, prefill); % roofline",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(best_ms / K, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "tokens_per_s_per_layer": round(K / best_ms * 1e3, 1),
        "config": {"workload": f"decode_b1_27b_layer_{K}_steps", "batch": 1, **SHAPE_DESC,
                   "state_bytes": 3_145_728, "act": "bf16", "state_buffers_rotated": min(K, R),
                   "states_touched_bytes": min(K, R) * 3_145_728,
                   "cache": "Infinity Cache evicted (1 GiB device copy) just before the timed steps",
                   "launch": launch,
                   "bytes_per_step": per_step},
        "roofline": roof, "cpu_baseline": cpu, "rows": {k: _round(v) for k, v in res.items()},
        "input_gen_s": round(gen_s, 1),
    }
    if args.details:
        with open(args.details, "w") as f:
            json.dump(line, f, indent=1)
    print(json.dumps(line))


def prefill_flops(T, shape):
    """Algorithmic flops of the chunked form at chunk 64 (per chunk: K.K^T and Q.K^T per
    q/k head; T.bV, T.bgK, P.W, Wk.S0^T, gQ.S0^T, W^T.K~ and the triangular solve per value head)."""
    Cc, D = 64, shape.head_k_dim
    nchunks = (T + Cc - 1) // Cc
    per_qk = 2 * (2 * Cc * Cc * D)
    per_v = 3 * (2 * Cc * Cc * D) + 3 * (2 * Cc * D * D) + Cc ** 3 // 3
    return nchunks * (shape.num_k_heads * per_qk + shape.num_v_heads * per_v)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _gcc_version():
    import subprocess
    try:
        return subprocess.run(["gcc", "--version"], capture_output=True, text=True).stdout.splitlines()[0]
    except (OSError, IndexError):
        return "unknown"


def _round(v):
    if isinstance(v, dict):
        return {k: _round(x) for k, x in v.items()}
    if isinstance(v, float):
        return round(v, 4)
    return v


if __name__ == "__main__":
    main()
