"""GPU parity of the paged-cache decode (fa_fwd_kvcache_paged).

Against the float64 oracle (oracle.sdpa.decode_paged: the pages of
block_table[b] laid end to end), and bitwise against the contiguous decode
on the gathered cache (same tiles, same split boundaries). Pages no
sequence uses, and the rows past each sequence's length, are poisoned (K
large, V NaN) so any stray read shows.
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


def make(B, Hq, Hkv, d, page_size, pps, lens, seed):
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(seed)
    num_pages = B * pps + 3
    q = torch.randn(B, 1, Hq, d, generator=g).to(torch.bfloat16)
    kp = torch.randn(num_pages, page_size, Hkv, d, generator=g).to(torch.bfloat16)
    vp = torch.randn(num_pages, page_size, Hkv, d, generator=g).to(torch.bfloat16)
    perm = torch.randperm(num_pages, generator=g)
    bt = perm[: B * pps].reshape(B, pps).to(torch.int32)
    # poison every row no sequence reads
    used = torch.zeros(num_pages, page_size, dtype=torch.bool)
    for b, n in enumerate(lens):
        for i in range(n):
            used[bt[b, i // page_size], i % page_size] = True
    kp[~used] = 1e4
    vp[~used] = float("nan")
    lt = torch.tensor(lens, dtype=torch.int32)
    return [t.to(dev) for t in (q, kp, vp, bt, lt)]


CASES = [
    # (B, Hq, Hkv, d, page_size, pages_per_seq, lens, splits)
    (3, 8, 2, 128, 64, 8, [512, 100, 1], [1, 3]),
    (3, 8, 2, 128, 256, 2, [512, 257, 64], [1, 2, 5]),
    (2, 4, 4, 64, 128, 3, [384, 129], [1, 2]),
    (2, 8, 2, 256, 64, 4, [256, 63], [1, 3]),
    (2, 16, 1, 128, 192, 2, [384, 200], [1, 4]),   # 16 query heads per KV head
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}kv{c[2]}d{c[3]}P{c[4]}")
def test_paged_decode(case):
    B, Hq, Hkv, d, P, pps, lens, splits = case
    q, kp, vp, bt, lt = make(B, Hq, Hkv, d, P, pps, lens, seed=81)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o_ref, l_ref = O.decode_paged(f64(q), f64(kp), f64(vp), bt.cpu().numpy(), lens, scale)
    # the contiguous cache the pages describe
    kc = kp[bt.long()].reshape(B, pps * P, Hkv, d).contiguous()
    vc = vp[bt.long()].reshape(B, pps * P, Hkv, d).contiguous()
    m = fa()
    for S in splits:
        print(f"paged decode B={B} Hq={Hq} Hkv={Hkv} d={d} page={P} S={S}", flush=True)
        o, lse = m.fa_fwd_kvcache_paged(q, kp, vp, bt, lt, num_splits=S, scale=scale)
        oc, lc = m.fa_fwd_kvcache(q, kc, vc, lt, num_splits=S, scale=scale)
        torch.cuda.synchronize()
        eo = np.max(np.abs(f64(o)[:, 0] - o_ref))
        el = np.max(np.abs(f64(lse) - l_ref))
        print(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
        assert eo <= 2e-2 and el <= 1e-3
        assert torch.equal(o, oc) and torch.equal(lse, lc), "paged != contiguous on the same keys"


def test_paged_decode_out_of_range_entries_are_clamped():
    # invalid page indices read a valid page (never out of bounds); the
    # entries that are valid still give the right answer for their sequence
    B, Hq, Hkv, d, P, pps = 2, 4, 2, 128, 64, 2
    q, kp, vp, bt, lt = make(B, Hq, Hkv, d, P, pps, [128, 64], seed=82)
    kp = torch.nan_to_num(kp, nan=0.0)
    vp = torch.nan_to_num(vp, nan=0.0)
    bt2 = bt.clone()
    bt2[1, 1] = 10 ** 6   # past the pool; sequence 1 only reads page slot 0
    o1, l1 = fa().fa_fwd_kvcache_paged(q, kp, vp, bt, lt, num_splits=1)
    o2, l2 = fa().fa_fwd_kvcache_paged(q, kp, vp, bt2, lt, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(o1[1], o2[1]) and torch.equal(l1[1], l2[1])
