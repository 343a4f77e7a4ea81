"""Concurrent calls on different streams.

The library keeps no mutable state between calls, so calls enqueued on two
streams at once (default priority) with their own buffers must give exactly
what the same calls give one after another: forward, split-KV decode with a
workspace per stream, and backward with a workspace per stream.
"""

import math

import numpy as np
import pytest
import torch

import seeded_inputs as SI

pytestmark = pytest.mark.gpu


def fa():
    import exact_io_aware_online_amd as m
    m.lib()
    return m


def note(msg):
    print(msg, flush=True)


def _problem(m, seed, dev):
    B, Hq, Hkv, N, d = 2, 8, 2, 900, 128
    q, k, v = SI.prefill_inputs(B=B, Hq=Hq, Hkv=Hkv, Nq=N, Nk=N, d=d, seed=seed, device=dev)
    qd, kc, vc, lens = SI.decode_inputs(16, Hq, Hkv, 3000, d, seed=seed + 1, len_lo=1, device=dev)
    dout = torch.randn(q.shape, generator=torch.Generator(device=dev).manual_seed(seed + 2), device=dev).to(q.dtype)
    S = m.fa_kvcache_default_splits(16, Hkv, 3000, d)
    ws = torch.empty(m.fa_fwd_kvcache_workspace_size(16, Hq, d, S), dtype=torch.uint8, device=dev)
    bws = torch.empty(m.fa_bwd_workspace_size(B, Hq, N), dtype=torch.uint8, device=dev)
    return dict(q=q, k=k, v=v, qd=qd, kc=kc, vc=vc, lens=lens, dout=dout, S=S, ws=ws, bws=bws,
                sc=float(np.float32(1.0 / math.sqrt(d))))


def _run(m, P, stream):
    o, lse = m.fa_fwd(P["q"], P["k"], P["v"], causal=True, scale=P["sc"], stream=stream)
    od, lsed = m.fa_fwd_kvcache(P["qd"], P["kc"], P["vc"], P["lens"], num_splits=P["S"], scale=P["sc"],
                                workspace=P["ws"], stream=stream)
    dq, dk, dv = m.fa_bwd(P["q"], P["k"], P["v"], o, lse, P["dout"], causal=True, scale=P["sc"], workspace=P["bws"],
                          stream=stream)
    return [o, lse, od, lsed, dq, dk, dv]


def test_two_streams_equal_serial_calls():
    m = fa()
    dev = torch.device("cuda")
    note("two streams: forward, decode and backward concurrently vs serially")
    P = [_problem(m, 100, dev), _problem(m, 200, dev)]
    torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    serial = [_run(m, p, main) for p in P]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    for rep in range(3):
        for s in streams:
            s.wait_stream(main)
        outs = [None, None]
        # interleave the enqueues: each stream's calls run beside the other's
        for i in (0, 1):
            with torch.cuda.stream(streams[i]):
                outs[i] = _run(m, P[i], streams[i])
        for s in streams:
            main.wait_stream(s)
        torch.cuda.synchronize()
        for i in (0, 1):
            for j, (a, b) in enumerate(zip(outs[i], serial[i])):
                assert torch.equal(a.view(torch.int8), b.view(torch.int8)), (rep, i, j)
        note(f"  round {rep}: both streams equal to the serial calls")
