"""GPU parity of the decode with appended rows on a seeded sweep of random shapes.

Random batch, new tokens per sequence (1 to 8, each also a query), group
size, head dimension, capacity, held lengths (empty caches and ones the new
rows overflow included), mask and split count; each case runs the
contiguous append and the paged append (random page size, scattered pages)
and is compared with the float64 oracle: the cache afterwards bit for bit
(rows past the held and new ones are poisoned and must stay as they were),
O within 2e-2 and LSE within 1e-3 (queries that see no key: LSE = -inf), and
the paged result equal to the contiguous one bit for bit. A second set has
64 or more (sequence, key/value head) pairs with at most 16 (query, query
head) columns each, the calls that take the balanced schedule, with and
without appended rows.
"""

import math

import numpy as np
import pytest
import torch

from oracle import sdpa as O

pytestmark = pytest.mark.gpu


def fa():
    import exact_io_aware_online_amd as m
    m.lib()
    return m


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _cases(n=16, seed=2030):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128, 256]))
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 4, 8]))
        B = int(rng.integers(1, 6))
        Nq = int(rng.integers(1, 9))
        page = int(rng.choice([64, 128]))
        pps = int(rng.integers(1, 9))
        cap = page * pps  # the contiguous case uses the paged capacity, so both describe one cache
        lens = [int(x) for x in rng.integers(0, cap + 1, B)]
        if B > 1:
            lens[1] = max(cap - Nq + 1, 0)  # the new rows overflow the capacity
        S = int(rng.choice([1, 2, 3, 8]))
        out.append((B, Nq, hkv * g, hkv, d, page, pps, tuple(lens), S, bool(rng.random() < 0.7), 1300 + i))
    return out


def _balanced_cases(n=15, seed=2034):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = (64, 128, 256)[i % 3]
        hkv = int(rng.choice([4, 8]))
        g = int(rng.choice([1, 2, 4, 8]))
        Nq = int(rng.integers(1, 16 // g + 1))
        B = int(rng.integers(64 // hkv, 64 // hkv + 18))
        page = int(rng.choice([64, 128]))
        pps = int(rng.integers(1, 7))
        pps = max(1, min(pps, 8_000_000 // (B * hkv * d * page)))  # keeps the float64 oracle's copies small
        cap = page * pps
        lens = [int(x) for x in rng.integers(0, cap + 1, B)]
        lens[1] = max(cap - Nq + 1, 0)  # the new rows overflow the capacity
        lens[2] = 0
        S = int(rng.choice([0, 2, 3, 5]))  # 0: the library's default
        append = bool(rng.random() < 0.75)
        out.append((B, Nq, hkv * g, hkv, d, page, pps, tuple(lens), S, bool(rng.random() < 0.7), 1400 + i, append))
    return out


CASES = _cases()
BALANCED = _balanced_cases()


@pytest.mark.parametrize("case", CASES, ids=["B{}q{}H{}kv{}d{}p{}x{}".format(*c[:7]) + f"s{c[-1]}" for c in CASES])
def test_append_sweep(case):
    _run(*case)


@pytest.mark.parametrize("case", BALANCED,
                         ids=["B{}q{}H{}kv{}d{}p{}x{}".format(*c[:7]) + f"s{c[-2]}a{int(c[-1])}" for c in BALANCED])
def test_balanced_multi_query_sweep(case):
    B, Nq, Hq, Hkv = case[:4]
    assert B * Hkv >= 64 and Nq * (Hq // Hkv) <= 16
    _run(*case)


def _run(B, Nq, Hq, Hkv, d, page, pps, lens, S, causal, seed, append=True):
    m = fa()
    if S == 0:
        S = m.fa_kvcache_append_default_splits(B, Nq, Hkv, Hq, page * pps, d)
    print(f"append sweep B={B} Nq={Nq} Hq={Hq} Hkv={Hkv} d={d} page={page}x{pps} lens={lens} S={S} "
          f"causal={causal} seed={seed} append={append}", flush=True)
    dev = torch.device("cuda")
    cap = page * pps
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Nq, Hq, d, generator=g).to(torch.bfloat16)
    kc = torch.randn(B, cap, Hkv, d, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, cap, Hkv, d, generator=g).to(torch.bfloat16)
    kn = torch.randn(B, Nq, Hkv, d, generator=g).to(torch.bfloat16)
    vn = torch.randn(B, Nq, Hkv, d, generator=g).to(torch.bfloat16)
    for b, n in enumerate(lens):  # rows past the held and the new ones are never read
        kc[b, min(n + Nq, cap):] = 1e4
        vc[b, min(n + Nq, cap):] = float("nan")
    scale = float(np.float32(1.0 / math.sqrt(d)))
    if not append:
        kn = vn = None
    k2, v2, o_ref, l_ref = O.decode_append(f64(q), f64(kc), f64(vc), list(lens), None if kn is None else f64(kn),
                                           None if vn is None else f64(vn), causal, scale)
    lt = torch.tensor(lens, dtype=torch.int32, device=dev)
    knd = None if kn is None else kn.to(dev)
    vnd = None if vn is None else vn.to(dev)

    kd, vd = kc.to(dev), vc.to(dev)
    o, lse = m.fa_fwd_kvcache_append(q.to(dev), kd, vd, lt, knd, vnd, causal=causal, num_splits=S, scale=scale)
    # the same cache as scattered pages, spare pages between
    num_pages = B * pps + 3
    bt = torch.randperm(num_pages, generator=g)[:B * pps].reshape(B, pps).to(torch.int32)
    kp = torch.zeros(num_pages, page, Hkv, d, dtype=torch.bfloat16)
    vp = torch.zeros_like(kp)
    kp[bt.long()] = kc.reshape(B, pps, page, Hkv, d)
    vp[bt.long()] = vc.reshape(B, pps, page, Hkv, d)
    kpd, vpd = kp.to(dev), vp.to(dev)
    op, lp = m.fa_fwd_kvcache_paged_append(q.to(dev), kpd, vpd, bt.to(dev), lt, knd, vnd, causal=causal,
                                           num_splits=S, scale=scale)
    torch.cuda.synchronize()

    assert np.array_equal(f64(kd), k2, equal_nan=True) and np.array_equal(f64(vd), v2, equal_nan=True)
    got_k = f64(kpd.cpu()[bt.long()].reshape(B, cap, Hkv, d))
    got_v = f64(vpd.cpu()[bt.long()].reshape(B, cap, Hkv, d))
    assert np.array_equal(got_k, k2, equal_nan=True) and np.array_equal(got_v, v2, equal_nan=True)
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(f64(lse)), fin)
    assert np.max(np.abs(f64(o) - o_ref), initial=0.0) <= 2e-2
    assert np.max(np.abs(f64(lse)[fin] - l_ref[fin]), initial=0.0) <= 1e-3
    assert torch.equal(op.view(torch.int16), o.view(torch.int16))
    assert torch.equal(lp.view(torch.int32), lse.view(torch.int32))
