"""The hot path captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

fa_fwd, fa_fwd_kvcache with a caller workspace and fa_fwd_kvcache_noalloc
(the entry point for callers that cannot allocate, e.g. under capture), and
in a second graph fa_bwd with a caller workspace and the FP8 quantise +
forward pipeline, are recorded once and replayed several times; between
replays the inputs are
rewritten in place by ordinary eager work, and every replay must equal the
eager calls on the same inputs bit for bit. None of the calls records a
memset or allocates: the split partials go to the caller's workspace or to
the library's static scratch, and every partial is written before it is read.
"""

import math

import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import sdpa as O

pytestmark = pytest.mark.gpu


def fa():
    import exact_io_aware_online_amd as m
    m.lib()
    return m


def note(msg):
    print(msg, flush=True)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def test_graph_replays_equal_eager_calls():
    m = fa()
    dev = torch.device("cuda")
    note("graph capture: fa_fwd + fa_fwd_kvcache + fa_fwd_kvcache_noalloc")
    # prefill: causal GQA with ragged tiles; decode: GQA, lengths up to the capacity
    B, Hq, Hkv, N, d = 2, 8, 2, 700, 128
    q, k, v = SI.prefill_inputs(B=B, Hq=Hq, Hkv=Hkv, Nq=N, Nk=N, d=d, seed=81, device=dev)
    Bd, cap = 8, 2048
    qd, kc, vc, lens = SI.decode_inputs(Bd, Hq, Hkv, cap, d, seed=82, len_lo=1, device=dev)
    sc = float(np.float32(1.0 / math.sqrt(d)))
    S = m.fa_kvcache_default_splits(Bd, Hkv, cap, d)
    assert S >= 2  # the split path, with its partials
    ws = torch.empty(m.fa_fwd_kvcache_workspace_size(Bd, Hq, d, S), dtype=torch.uint8, device=dev)

    def outputs():
        return (torch.empty_like(q), torch.empty(B, Hq, N, dtype=torch.float32, device=dev),
                torch.empty_like(qd), torch.empty(Bd, Hq, dtype=torch.float32, device=dev),
                torch.empty_like(qd), torch.empty(Bd, Hq, dtype=torch.float32, device=dev))

    def run(o, lse, od, lsed, on, lsen):
        m.fa_fwd(q, k, v, o=o, lse=lse, causal=True, scale=sc)
        m.fa_fwd_kvcache(qd, kc, vc, lens, o=od, lse=lsed, num_splits=S, scale=sc, workspace=ws)
        m.fa_fwd_kvcache_noalloc(qd, kc, vc, lens, o=on, lse=lsen, num_splits=S, scale=sc)

    graph_out = outputs()
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(*graph_out)  # warm-up outside the capture (first-use lookups)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(*graph_out)
    torch.cuda.synchronize()

    gen = torch.Generator(device=dev)
    gen.manual_seed(83)
    names = ("O", "LSE", "decode O", "decode LSE", "no-alloc O", "no-alloc LSE")
    for rep in range(4):
        # new inputs in place, by eager kernels, between replays
        for t in (q, k, v, qd, kc, vc):
            t.copy_(torch.randn(t.shape, generator=gen, device=dev).to(t.dtype))
        lens.copy_(torch.randint(1, cap + 1, (Bd,), generator=gen, device=dev, dtype=torch.int32))
        if rep == 3:
            lens[0] = 0  # an empty sequence: O = 0, LSE = -inf
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in graph_out]
        eager = outputs()
        run(*eager)
        torch.cuda.synchronize()
        for name, a, b in zip(names, got, eager):
            assert torch.equal(a.view(torch.int8), b.view(torch.int8)), (rep, name)
        assert torch.equal(got[2].view(torch.int16), got[4].view(torch.int16)), (rep, "no-alloc vs workspace")
        # and the replay is the attention of its inputs: a few rows against the oracle
        o_ref, l_ref = O.attention_rows(f64(q[1:2, :, Hq - 1:Hq]), f64(k[1:2, :, Hkv - 1:Hkv]),
                                        f64(v[1:2, :, Hkv - 1:Hkv]), True, sc, 0, 0, rows=np.arange(N - 40, N))
        assert np.max(np.abs(f64(got[0][1, N - 40:, Hq - 1]) - o_ref)) <= 2e-2
        assert np.max(np.abs(f64(got[1][1, Hq - 1, N - 40:]) - l_ref)) <= 1e-3
        n = int(lens[Bd - 1])
        od_ref, ld_ref = O.decode(f64(qd[Bd - 1:]), f64(kc[Bd - 1:, :n]), f64(vc[Bd - 1:, :n]), [n], sc)
        assert np.max(np.abs(f64(got[2][Bd - 1, 0]) - od_ref[0])) <= 2e-2
        assert np.max(np.abs(f64(got[3][Bd - 1]) - ld_ref[0])) <= 1e-3
        note(f"  replay {rep}: equal to the eager calls; sampled rows within the oracle bars")
    del g
    torch.cuda.synchronize()


def test_graph_replays_of_backward_and_fp8_equal_eager_calls():
    m = fa()
    dev = torch.device("cuda")
    note("graph capture: fa_bwd (caller workspace), fa_quantize_fp8 x3 + fa_fwd_fp8")
    B, Hq, Hkv, N, d = 2, 4, 2, 300, 128
    q, k, v = SI.prefill_inputs(B=B, Hq=Hq, Hkv=Hkv, Nq=N, Nk=N, d=d, seed=91, device=dev)
    sc = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = m.fa_fwd(q, k, v, causal=True, scale=sc)
    dout = torch.randn(q.shape, generator=torch.Generator(device=dev).manual_seed(92), device=dev).to(q.dtype)
    bws = torch.empty(m.fa_bwd_workspace_size(B, Hq, N), dtype=torch.uint8, device=dev)
    signs = SI.random_signs(d, seed=93, device=dev)
    Np = m.fa_fp8_padded_rows(N)

    def outputs():
        codes = [torch.empty(B, Hq, Np, d, dtype=torch.uint8, device=dev),
                 torch.empty(B, Hkv, Np, d, dtype=torch.uint8, device=dev),
                 torch.empty(B, Hkv, d, Np, dtype=torch.uint8, device=dev)]
        scales = [torch.empty(B, h, Np // 64, dtype=torch.uint8, device=dev) for h in (Hq, Hkv, Hkv)]
        return ([torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)], codes, scales,
                [torch.empty_like(q), torch.empty(B, Hq, N, dtype=torch.float32, device=dev)])

    def run(grads, codes, scales, fo):
        m.fa_bwd(q, k, v, o, lse, dout, causal=True, scale=sc, dq=grads[0], dk=grads[1], dv=grads[2], workspace=bws)
        m.fa_quantize_fp8(q, signs, codes=codes[0], scales=scales[0])
        m.fa_quantize_fp8(k, signs, codes=codes[1], scales=scales[1])
        m.fa_quantize_fp8(v, transpose=True, codes=codes[2], scales=scales[2])
        m.fa_fwd_fp8(codes[0], scales[0], codes[1], scales[1], codes[2], scales[2], N, N, causal=True, scale=sc,
                     o=fo[0], lse=fo[1])

    graph_out = outputs()
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(*graph_out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(*graph_out)
    torch.cuda.synchronize()

    flat = lambda outs: [t for group in outs for t in group]
    gen = torch.Generator(device=dev)
    gen.manual_seed(94)
    for rep in range(3):
        for t in (q, k, v, dout):
            t.copy_(torch.randn(t.shape, generator=gen, device=dev).to(t.dtype))
        m.fa_fwd(q, k, v, o=o, lse=lse, causal=True, scale=sc)  # the forward the backward reads
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in flat(graph_out)]
        eager = outputs()
        run(*eager)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, flat(eager))):
            assert torch.equal(a.view(torch.int8), b.view(torch.int8)), (rep, i)
        note(f"  replay {rep}: dq, dk, dv, the FP8 codes and scales, O and LSE equal to the eager calls")
    del g
    torch.cuda.synchronize()


def test_graph_replays_of_balanced_append_equal_eager_calls():
    m = fa()
    dev = torch.device("cuda")
    note("graph capture: fa_fwd_kvcache_append, 2 new tokens, 64 (sequence, KV head) pairs (balanced schedule)")
    B, Nq, Hq, Hkv, cap, d = 32, 2, 8, 2, 1024, 128
    sc = float(np.float32(1.0 / math.sqrt(d)))
    gen = torch.Generator(device=dev)
    gen.manual_seed(95)
    rnd = lambda *s: torch.randn(s, generator=gen, device=dev).to(torch.bfloat16)
    q, kn, vn = rnd(B, Nq, Hq, d), rnd(B, Nq, Hkv, d), rnd(B, Nq, Hkv, d)
    kc, vc = rnd(B, cap, Hkv, d), rnd(B, cap, Hkv, d)
    lens = torch.randint(0, cap - Nq + 1, (B,), generator=gen, device=dev, dtype=torch.int32)
    S = m.fa_kvcache_append_default_splits(B, Nq, Hkv, Hq, cap, d)
    assert S >= 2
    ws = torch.empty(m.fa_fwd_kvcache_workspace_size(B * Nq, Hq, d, S), dtype=torch.uint8, device=dev)

    def outputs():
        return torch.empty_like(q), torch.empty(B, Hq, Nq, dtype=torch.float32, device=dev)

    def run(o, lse):
        m.fa_fwd_kvcache_append(q, kc, vc, lens, kn, vn, causal=True, o=o, lse=lse, num_splits=S, scale=sc,
                                workspace=ws)

    graph_out = outputs()
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(*graph_out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(*graph_out)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (q, kn, vn, kc, vc):
            t.copy_(torch.randn(t.shape, generator=gen, device=dev).to(t.dtype))
        lens.copy_(torch.randint(0, cap - Nq + 1, (B,), generator=gen, device=dev, dtype=torch.int32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in graph_out]
        cache_after = (kc.clone(), vc.clone())
        eager = outputs()
        run(*eager)
        torch.cuda.synchronize()
        for name, a, b in zip(("O", "LSE"), got, eager):
            assert torch.equal(a.view(torch.int8), b.view(torch.int8)), (rep, name)
        # the appended rows are in the cache, and the result is the attention of the grown cache
        b0 = int(lens[0])
        assert torch.equal(cache_after[0][0, b0:b0 + Nq], kn[0]) and torch.equal(cache_after[1][0, b0:b0 + Nq], vn[0])
        k2, v2, o_ref, l_ref = O.decode_append(f64(q[:1]), f64(kc[:1]), f64(vc[:1]), [b0], f64(kn[:1]), f64(vn[:1]),
                                               True, sc)
        assert np.max(np.abs(f64(got[0][:1]) - o_ref)) <= 2e-2
        assert np.max(np.abs(f64(got[1][:1]) - l_ref)) <= 1e-3
        note(f"  replay {rep}: equal to the eager call; sequence 0 within the oracle bars")
    del g
    torch.cuda.synchronize()
