"""GPU parity of the decode step with in-place cache append
(fa_fwd_kvcache_append, fa_fwd_kvcache_paged_append) against the float64
oracle (oracle.sdpa.decode_append).

The cache after the call must equal the oracle's cache bit for bit (the
append is a copy); O and LSE are compared within the decode tolerances.
Rows the call must neither read nor write are poisoned (K large, V NaN).
"""

import math

import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import sdpa as O

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 2e-2, 1e-3


def fa():
    import exact_io_aware_online_amd as m
    m.lib()
    return m


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def note(msg):
    print(msg, flush=True)


def make(B, Nq, Hq, Hkv, d, cap, lens, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Nq, Hq, d, generator=g).to(torch.bfloat16)
    kc = torch.randn(B, cap, Hkv, d, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, cap, Hkv, d, generator=g).to(torch.bfloat16)
    kn = torch.randn(B, Nq, Hkv, d, generator=g).to(torch.bfloat16)
    vn = torch.randn(B, Nq, Hkv, d, generator=g).to(torch.bfloat16)
    for b, n in enumerate(lens):  # rows past the held ones and the new ones are never read
        kc[b, min(max(n, 0) + Nq, cap):] = 1e4
        vc[b, min(max(n, 0) + Nq, cap):] = float("nan")
    return q, kc, vc, kn, vn


def compare(o, lse, o_ref, l_ref):
    eo = float(np.max(np.abs(f64(o) - o_ref)))
    L = f64(lse)
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(L), fin), "queries without keys must have LSE = -inf"
    el = float(np.max(np.abs(L[fin] - l_ref[fin]), initial=0.0))
    note(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O and el <= TOL_LSE


# (B, Nq, Hq, Hkv, d, capacity, lens, splits)
CASES = [
    (3, 1, 8, 2, 128, 512, [300, 0, 511], [1, 3]),       # one query; last sequence fills the cache
    (2, 4, 8, 2, 128, 640, [257, 64], [1, 4]),           # 16 (query, head) pairs: one column group
    (2, 5, 8, 2, 128, 640, [100, 500], [1, 2, 5]),       # 20 pairs: two column groups
    (2, 3, 32, 8, 128, 1024, [1022, 1], [1, 8]),         # capacity overflow on sequence 0
    (1, 7, 16, 1, 64, 384, [129], [1, 3]),               # 112 pairs: seven groups, d = 64
    (2, 2, 4, 4, 256, 320, [64, 190], [1, 2]),           # d = 256
    (2, 16, 2, 2, 128, 256, [0, 17], [1, 2]),            # more queries than held rows
]


@pytest.mark.parametrize("append", [True, False])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}q{}H{}kv{}d{}cap{}".format(*c[:6]))
def test_append_matches_oracle(case, causal, append):
    B, Nq, Hq, Hkv, d, cap, lens, splits = case
    dev = torch.device("cuda")
    q, kc, vc, kn, vn = make(B, Nq, Hq, Hkv, d, cap, lens, seed=101)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    k2, v2, o_ref, l_ref = O.decode_append(f64(q), f64(kc), f64(vc), lens, f64(kn) if append else None,
                                           f64(vn) if append else None, causal, scale)
    lt = torch.tensor(lens, dtype=torch.int32, device=dev)
    m = fa()
    for S in splits:
        note(f"append B={B} Nq={Nq} Hq={Hq} Hkv={Hkv} d={d} cap={cap} lens={lens} S={S} causal={causal} "
             f"append={append}")
        kd, vd = kc.to(dev), vc.to(dev)
        o, lse = m.fa_fwd_kvcache_append(q.to(dev), kd, vd, lt, kn.to(dev) if append else None,
                                         vn.to(dev) if append else None, causal=causal, num_splits=S, scale=scale)
        torch.cuda.synchronize()
        compare(o, lse, o_ref, l_ref)
        # the cache is the oracle's, bit for bit (NaN poison where it stays)
        assert np.array_equal(f64(kd), k2, equal_nan=True) and np.array_equal(f64(vd), v2, equal_nan=True)


def test_append_one_query_without_rows_is_fa_fwd_kvcache_bitwise():
    dev = torch.device("cuda")
    q, kc, vc, _, _ = make(3, 1, 8, 2, 128, 1024, [700, 64, 1], seed=102)
    lt = torch.tensor([700, 64, 1], dtype=torch.int32, device=dev)
    m = fa()
    for S in (1, 4):
        o1, l1 = m.fa_fwd_kvcache(q.to(dev), kc.to(dev), vc.to(dev), lt, num_splits=S)
        o2, l2 = m.fa_fwd_kvcache_append(q.to(dev), kc.to(dev), vc.to(dev), lt, causal=True, num_splits=S)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2[:, :, 0])


def test_fused_append_equals_copy_then_attend_bitwise():
    # writing the rows first (torch copy) and attending to the grown cache
    # reads the same tiles in the same order
    dev = torch.device("cuda")
    B, Nq, Hq, Hkv, d, cap = 2, 3, 8, 2, 128, 512
    lens = [200, 61]
    q, kc, vc, kn, vn = (t.to(dev) for t in make(B, Nq, Hq, Hkv, d, cap, lens, seed=103))
    kc2, vc2 = kc.clone(), vc.clone()
    for b, n in enumerate(lens):
        kc2[b, n:n + Nq] = kn[b]
        vc2[b, n:n + Nq] = vn[b]
    m = fa()
    for S in (1, 3):
        ka, va = kc.clone(), vc.clone()
        o1, l1 = m.fa_fwd_kvcache_append(q, ka, va, torch.tensor(lens, dtype=torch.int32, device=dev), kn, vn,
                                         causal=True, num_splits=S)
        o2, l2 = m.fa_fwd_kvcache_append(q, kc2, vc2, torch.tensor([n + Nq for n in lens], dtype=torch.int32,
                                                                   device=dev), causal=True, num_splits=S)
        torch.cuda.synchronize()
        bits = lambda t: t.view(torch.int16)  # the poison is NaN: compare bit patterns
        assert torch.equal(bits(ka), bits(kc2)) and torch.equal(bits(va), bits(vc2))
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_generation_loop():
    # a prefix, then six steps of one new token each, the lengths advanced
    # by the caller between steps; every step checked against the oracle
    dev = torch.device("cuda")
    B, Hq, Hkv, d, cap = 2, 8, 2, 128, 320
    lens = [250, 3]
    g = torch.Generator().manual_seed(104)
    kc = torch.randn(B, cap, Hkv, d, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, cap, Hkv, d, generator=g).to(torch.bfloat16)
    kd, vd = kc.to(dev), vc.to(dev)
    kr, vr = f64(kc), f64(vc)
    m = fa()
    scale = float(np.float32(1.0 / math.sqrt(d)))
    for step in range(6):
        q = torch.randn(B, 1, Hq, d, generator=g).to(torch.bfloat16)
        kn = torch.randn(B, 1, Hkv, d, generator=g).to(torch.bfloat16)
        vn = torch.randn(B, 1, Hkv, d, generator=g).to(torch.bfloat16)
        note(f"generation step {step} lens={lens}")
        o, lse = m.fa_fwd_kvcache_append(q.to(dev), kd, vd, torch.tensor(lens, dtype=torch.int32, device=dev),
                                         kn.to(dev), vn.to(dev), causal=True, num_splits=2, scale=scale)
        torch.cuda.synchronize()
        kr, vr, o_ref, l_ref = O.decode_append(f64(q), kr, vr, lens, f64(kn), f64(vn), True, scale)
        compare(o, lse, o_ref, l_ref)
        lens = [n + 1 for n in lens]
    assert np.array_equal(f64(kd), kr) and np.array_equal(f64(vd), vr)


PAGED = [
    # (B, Nq, Hq, Hkv, d, page_size, pages_per_seq, lens, splits)
    (3, 1, 8, 2, 128, 64, 8, [500, 63, 0], [1, 3]),
    (2, 4, 8, 2, 128, 128, 4, [126, 300], [1, 2]),      # new rows straddle a page boundary
    (2, 6, 16, 2, 64, 64, 3, [190, 40], [1, 3]),         # overflow on sequence 0; three column groups
]


@pytest.mark.parametrize("case", PAGED, ids=lambda c: "B{}q{}H{}kv{}d{}P{}".format(*c[:6]))
def test_paged_append_matches_oracle(case):
    B, Nq, Hq, Hkv, d, P, pps, lens, splits = case
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(105)
    num_pages = B * pps + 2
    q = torch.randn(B, Nq, Hq, d, generator=g).to(torch.bfloat16)
    kp = torch.randn(num_pages, P, Hkv, d, generator=g).to(torch.bfloat16)
    vp = torch.randn(num_pages, P, Hkv, d, generator=g).to(torch.bfloat16)
    kn = torch.randn(B, Nq, Hkv, d, generator=g).to(torch.bfloat16)
    vn = torch.randn(B, Nq, Hkv, d, generator=g).to(torch.bfloat16)
    bt = torch.randperm(num_pages, generator=g)[: B * pps].reshape(B, pps).to(torch.int32)
    cap = P * pps
    # the oracle sees the contiguous cache the pages describe
    kc = kp[bt.long()].reshape(B, cap, Hkv, d)
    vc = vp[bt.long()].reshape(B, cap, Hkv, d)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    k2, v2, o_ref, l_ref = O.decode_append(f64(q), f64(kc), f64(vc), lens, f64(kn), f64(vn), True, scale)
    m = fa()
    for S in splits:
        note(f"paged append B={B} Nq={Nq} Hq={Hq} Hkv={Hkv} d={d} page={P} lens={lens} S={S}")
        kd, vd = kp.to(dev), vp.to(dev)
        o, lse = m.fa_fwd_kvcache_paged_append(q.to(dev), kd, vd, bt.to(dev),
                                               torch.tensor(lens, dtype=torch.int32, device=dev), kn.to(dev),
                                               vn.to(dev), causal=True, num_splits=S, scale=scale)
        torch.cuda.synchronize()
        compare(o, lse, o_ref, l_ref)
        got_k = f64(kd.cpu()[bt.long()].reshape(B, cap, Hkv, d))
        got_v = f64(vd.cpu()[bt.long()].reshape(B, cap, Hkv, d))
        assert np.array_equal(got_k, k2) and np.array_equal(got_v, v2)
        # pages no sequence owns are untouched
        spare = sorted(set(range(num_pages)) - set(bt.flatten().tolist()))
        assert torch.equal(kd.cpu()[spare], kp[spare]) and torch.equal(vd.cpu()[spare], vp[spare])


def test_full_size_one_token_append_sampled():
    # the decode workload (64 sequences, 32 query / 8 key-value heads, cache
    # 8192, head_dim 128) with one appended token per sequence, default splits
    w = dict(SI.DECODE_WORKLOADS["gqa_bf16_decode_b64_h32kv8_cap8192_d128"])
    dev = torch.device("cuda")
    q, kc, vc, lens = SI.decode_inputs(device=dev, **w)
    B, Hq, Hkv, d = w["B"], w["Hq"], w["Hkv"], w["d"]
    lens = torch.clamp(lens, max=w["capacity"] - 1)
    g = torch.Generator(device=dev).manual_seed(106)
    kn = torch.randn(B, 1, Hkv, d, generator=g, device=dev).to(torch.bfloat16)
    vn = torch.randn(B, 1, Hkv, d, generator=g, device=dev).to(torch.bfloat16)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = fa().fa_fwd_kvcache_append(q, kc, vc, lens, kn, vn, causal=True, scale=scale)
    torch.cuda.synchronize()
    L = lens.cpu().numpy()
    rng = np.random.default_rng(107)
    for b in {0, B - 1, int(rng.integers(B)), int(rng.integers(B))}:
        n = int(L[b])
        assert torch.equal(kc[b, n], kn[b, 0]) and torch.equal(vc[b, n], vn[b, 0])
        heads = sorted({0, Hq - 1, int(rng.integers(Hq))})
        o_ref, l_ref = O.decode(f64(q[b:b + 1]), f64(kc[b:b + 1, :n + 1]), f64(vc[b:b + 1, :n + 1]), [n + 1], scale,
                                heads=heads)
        for h in heads:
            eo = np.max(np.abs(f64(o[b, 0, h]) - o_ref[0, h]))
            el = abs(float(lse[b, h, 0]) - l_ref[0, h])
            note(f"  b={b} h={h} len={n + 1} max|dO|={eo:.3e} |dLSE|={el:.3e}")
            assert eo <= TOL_O and el <= TOL_LSE
