"""Streams and graph capture through the C ABI.

The library keeps no state, allocates nothing and never synchronises, so
calls on different streams may run at once and a sequence of calls may be
captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.  Each
replay is checked against the eager result on the same inputs, with eager
work and a synchronisation between replays.
"""
import math

import pytest
import torch

import tiled_scaled_dot_amd as tsd
from tiled_scaled_dot_amd.workloads import random_inputs, scaled_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def gpu(*ts):
    return [t.to(DEV) for t in ts]


def test_two_streams_at_once():
    """attn_fwd on one stream and split-KV on another, launched together,
    give the results of the same calls run one after the other."""
    qa, ka, va = gpu(*random_inputs((2, 8, 1024, 128), (2, 8, 1024, 128), (2, 8, 1024, 128),
                                    "bf16", seed=11))
    qb, kb, vb = gpu(*random_inputs((1, 8, 64, 128), (1, 8, 9000, 128), (1, 8, 9000, 128),
                                    "bf16", seed=12))
    oa_ref, la_ref = tsd.attn_fwd(qa, ka, va, causal=True)
    ob_ref, lb_ref = tsd.attn_fwd_splitkv(qb, kb, vb, causal=True, causal_offset=9000 - 64,
                                          n_splits=6)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    oa, la = torch.empty_like(oa_ref), torch.empty_like(la_ref)
    ob, lb = torch.empty_like(ob_ref), torch.empty_like(lb_ref)
    torch.cuda.current_stream().synchronize()
    for _ in range(3):
        with torch.cuda.stream(s1):
            tsd.attn_fwd(qa, ka, va, causal=True, out=oa, lse=la)
        with torch.cuda.stream(s2):
            tsd.attn_fwd_splitkv(qb, kb, vb, causal=True, causal_offset=9000 - 64, n_splits=6,
                                 out=ob, lse=lb)
        torch.cuda.synchronize()
        assert torch.equal(oa, oa_ref) and torch.equal(la, la_ref)
        assert torch.equal(ob, ob_ref) and torch.equal(lb, lb_ref)


def test_graph_replay_matches_eager():
    """attn_fwd, attn_fwd_ext (grouped heads, window), attn_fwd_splitkv and
    attn_fwd_scaled (fp8) captured into one graph; three replays with new
    inputs copied in between, each equal to the eager calls."""
    B, H, S, D = 1, 8, 700, 128
    q, k, v = gpu(*random_inputs((B, H, S, D), (B, H, S, D), (B, H, S, D), "bf16", seed=21))
    kg, vg = k[:, :2].contiguous(), v[:, :2].contiguous()
    qd, kd, vd = gpu(*random_inputs((1, 8, 16, 128), (1, 8, 6000, 128), (1, 8, 6000, 128),
                                    "bf16", seed=22))
    q8, k8, v8, qs, ks = gpu(*scaled_inputs(1, 4, 300, 500, 128, 128, 128, 64, "fp8_e4m3",
                                            "bf16", seed=23))
    _, _, ws = tsd.attn_splitkv_plan(1, 8, 16, 6000, 128, 128, True, "bf16",
                                     tsd.make_mask(6000, 6000 - 16), 5)
    work = torch.empty(ws, dtype=torch.uint8, device=DEV)
    outs = {
        "fwd": (torch.empty((B, H, S, D), dtype=torch.bfloat16, device=DEV),
                torch.empty((B, H, S), dtype=torch.float32, device=DEV)),
        "ext": (torch.empty((B, H, S, D), dtype=torch.bfloat16, device=DEV),
                torch.empty((B, H, S), dtype=torch.float32, device=DEV)),
        "skv": (torch.empty((1, 8, 16, 128), dtype=torch.bfloat16, device=DEV),
                torch.empty((1, 8, 16), dtype=torch.float32, device=DEV)),
        "fp8": (torch.empty((1, 4, 300, 128), dtype=torch.bfloat16, device=DEV),
                torch.empty((1, 4, 300), dtype=torch.float32, device=DEV)),
    }

    def calls():
        tsd.attn_fwd(q, k, v, causal=True, out=outs["fwd"][0], lse=outs["fwd"][1])
        tsd.attn_fwd_ext(q, kg, vg, causal=True, window=200, out=outs["ext"][0],
                         lse=outs["ext"][1])
        tsd.attn_fwd_splitkv(qd, kd, vd, causal=True, causal_offset=6000 - 16, n_splits=5,
                             workspace=work, out=outs["skv"][0], lse=outs["skv"][1])
        tsd.attn_fwd_scaled(q8, k8, v8, qs, ks, 128, 64, causal=True, out=outs["fp8"][0],
                            lse=outs["fp8"][1])

    # warm up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()

    g = torch.Generator(device="cpu").manual_seed(24)
    for replay in range(3):
        # new inputs, copied in eagerly
        q.copy_(torch.randn(q.shape, generator=g).to(q.dtype))
        vd.copy_(torch.randn(vd.shape, generator=g).to(vd.dtype))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {n: (o.clone(), l.clone()) for n, (o, l) in outs.items()}
        calls()   # eager, same inputs
        torch.cuda.synchronize()
        for n, (o, l) in outs.items():
            assert torch.equal(got[n][0], o), f"replay {replay}: {n} O differs from eager"
            assert torch.equal(got[n][1], l), f"replay {replay}: {n} LSE differs from eager"


def test_graph_replay_noalloc_splitkv():
    """attn_fwd_splitkv_noalloc, the entry point for callers that cannot
    allocate (graph capture among them), captured into a graph after one
    eager call (which looks up the device's scratch array) and replayed
    three times with new inputs; each replay equals the eager call and the
    workspace form of split-KV on the same inputs."""
    B, H, H_kv, S_q, S_k, D = 2, 16, 4, 4, 9000, 128
    q, k, v = gpu(*random_inputs((B, H, S_q, D), (B, H_kv, S_k, D), (B, H_kv, S_k, D),
                                 "bf16", seed=31))
    kw = dict(causal=True, causal_offset=S_k - S_q, n_splits=6)
    out = torch.empty((B, H, S_q, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H, S_q), dtype=torch.float32, device=DEV)

    def call():
        tsd.attn_fwd_splitkv_noalloc(q, k, v, out=out, lse=lse, **kw)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()

    g = torch.Generator(device="cpu").manual_seed(32)
    for replay in range(3):
        q.copy_(torch.randn(q.shape, generator=g).to(q.dtype))
        v.copy_(torch.randn(v.shape, generator=g).to(v.dtype))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        call()   # eager, same inputs
        torch.cuda.synchronize()
        assert torch.equal(got_o, out) and torch.equal(got_l, lse), f"replay {replay}"
        o_ws, l_ws = tsd.attn_fwd_splitkv(q, k, v, **kw)
        torch.cuda.synchronize()
        assert torch.equal(got_o, o_ws) and torch.equal(got_l, l_ws), f"replay {replay}"
