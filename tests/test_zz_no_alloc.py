"""The allocation-free decode entry point (fa_fwd_kvcache_noalloc) against
fa_fwd_kvcache, called through the C ABI: two calls in a row, the second
with a smaller input, each compared with the entry point that takes a
caller workspace (same kernels, so the results must agree bit for bit, and
both lie within the decode bars of the float64 oracle)."""

import ctypes
import math

import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import sdpa as O

pytestmark = pytest.mark.gpu


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def note(msg):
    print(msg, flush=True)


def _call_noalloc(L, q, kc, vc, lens, o, lse, S, scale):
    B, _, Hq, d = q.shape
    _, cap, Hkv, _ = kc.shape
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    return L.fa_fwd_kvcache_noalloc(p(q), p(kc), p(vc), p(lens), p(o), p(lse), S, B, Hq, Hkv, cap, d,
                                    ctypes.c_float(scale), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _call_ws(L, q, kc, vc, lens, o, lse, S, scale, ws):
    B, _, Hq, d = q.shape
    _, cap, Hkv, _ = kc.shape
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    return L.fa_fwd_kvcache(p(q), p(kc), p(vc), p(lens), p(o), p(lse), S, B, Hq, Hkv, cap, d, ctypes.c_float(scale),
                            p(ws), ws.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.timeout(300)
def test_noalloc_decode_matches_workspace_decode_twice():
    import exact_io_aware_online_amd as fa
    L = fa.lib()
    dev = torch.device("cuda")
    # the decode workload, then a smaller batch with fewer heads and splits
    w = SI.DECODE_WORKLOADS["gqa_bf16_decode_b64_h32kv8_cap8192_d128"]
    small = dict(B=5, Hq=8, Hkv=2, capacity=700, d=128, len_lo=1, len_hi=700, seed=41)
    for n, (cfg, S) in enumerate(((w, fa.fa_kvcache_default_splits(w["B"], w["Hkv"], w["capacity"], w["d"])),
                                  (small, 3))):
        note(f"call {n}: B={cfg['B']} Hq={cfg['Hq']} Hkv={cfg['Hkv']} cap={cfg['capacity']} S={S}")
        q, kc, vc, lens = SI.decode_inputs(device=dev, **cfg)
        scale = float(np.float32(1.0 / math.sqrt(cfg["d"])))
        o1, o2 = torch.full_like(q, float("nan")), torch.full_like(q, float("nan"))
        l1 = torch.full((cfg["B"], cfg["Hq"]), float("nan"), device=dev)
        l2 = torch.full_like(l1, float("nan"))
        assert _call_noalloc(L, q, kc, vc, lens, o1, l1, S, scale) == fa.FA_OK
        ws = torch.empty(max(fa.fa_fwd_kvcache_workspace_size(cfg["B"], cfg["Hq"], cfg["d"], S), 1),
                         dtype=torch.uint8, device=dev)
        assert _call_ws(L, q, kc, vc, lens, o2, l2, S, scale, ws) == fa.FA_OK
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        # and both within the bars of the oracle, on every sequence
        lh = lens.cpu().numpy()
        seqs = range(cfg["B"]) if cfg["B"] <= 8 else sorted({0, cfg["B"] - 1, 7, 31})
        for b in seqs:
            nb = int(lh[b])
            o_ref, l_ref = O.decode(f64(q[b:b + 1]), f64(kc[b:b + 1, :nb]), f64(vc[b:b + 1, :nb]), [nb], scale)
            assert np.max(np.abs(f64(o1[b, 0]) - o_ref[0])) <= 2e-2
            assert np.max(np.abs(f64(l1[b]) - l_ref[0])) <= 1e-3


def test_noalloc_rejects_sizes_beyond_its_scratch():
    import exact_io_aware_online_amd as fa
    L = fa.lib()
    # B=4096, Hq=32, d=128, 8 splits: 4096*32*8*129*4 bytes > 16 MiB, rejected on the host
    null = None
    assert L.fa_fwd_kvcache_noalloc(null, null, null, null, null, null, 8, 4096, 32, 8, 8192, 128,
                                    ctypes.c_float(0.1), null) == fa.FA_ERR_WORKSPACE
