"""GPU parity of the decode on a seeded sweep of random shapes.

The hand-picked decode cases fix particular splits and tails; this sweep
draws batch size, key/value heads, group size (1 to 16 query heads per key/
value head), head dimension, cache capacity (not always a multiple of the
64-key tile), lengths (0 and the full capacity included) and the split
count (1, small, large, more runs than tiles, the default) from a fixed
numpy generator, plus cases with 256 or more (sequence, key/value head)
pairs, which take the 32-key-tile shape of the balanced decode at d = 64 and
128. Each case runs the contiguous decode and the same keys as a
paged cache (random page size, pages scattered over a pool with spare pages)
and compares O and LSE with the float64 oracle (O 2e-2, LSE 1e-3), and the
paged result with the contiguous one bit for bit.
"""

import math

import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import sdpa as O

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=2027):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128, 256]))
        g = int(rng.choice([1, 2, 4, 8, 16]))
        hkv = int(rng.choice([1, 2, 4, 8]))
        B = int(rng.integers(1, 41))
        cap = int(rng.choice([64, 100, 513, 1024, 2000, 4096]))
        S = int(rng.choice([0, 1, 2, 3, 5, 16, 64]))  # 0: the library's default
        page = int(rng.choice([64, 128, 256]))
        B = min(B, max(2, 40_000_000 // (cap * hkv * d)))  # keeps the float64 oracle's copies small
        out.append((B, hkv * g, hkv, cap, d, S, page, 700 + i))
    return out


def _many_pair_cases(n=10, seed=2032, d=128):
    # at least 256 (sequence, key/value head) pairs: the 32-key-tile shape of the balanced decode at d = 64 and 128
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hkv = int(rng.choice([4, 8]))
        g = int(rng.choice([1, 2, 4, 8]))
        B = int(rng.integers(256 // hkv, 256 // hkv + 40))
        cap = int(rng.choice([64, 100, 513, 1024, 2000]))
        S = int(rng.choice([0, 2, 3, 5]))
        page = int(rng.choice([64, 128, 256]))
        out.append((B, hkv * g, hkv, cap, d, S, page, (800 if d == 128 else 850) + i))
    return out


CASES = _cases() + _many_pair_cases() + _many_pair_cases(n=8, seed=2033, d=64)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


@pytest.mark.parametrize("case", CASES, ids=["B{}H{}kv{}cap{}d{}S{}p{}s{}".format(*c) for c in CASES])
def test_decode_sweep(case):
    import exact_io_aware_online_amd as fa
    B, Hq, Hkv, cap, d, S, page, seed = case
    print(f"decode sweep B={B} Hq={Hq} Hkv={Hkv} cap={cap} d={d} S={S} page={page} seed={seed}", flush=True)
    dev = torch.device("cuda")
    q, kc, vc, lens = SI.decode_inputs(B, Hq, Hkv, cap, d, seed=seed, len_lo=0, device=dev)
    lens[0] = cap  # one full cache, and one empty when there is a second sequence
    if B > 1:
        lens[B - 1] = 0
    S = S or fa.fa_kvcache_default_splits(B, Hkv, cap, d)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = fa.fa_fwd_kvcache(q, kc, vc, lens, num_splits=S, scale=scale)

    # the same keys in a paged pool: pages of each sequence scattered, spare pages between
    pps = (cap + page - 1) // page
    pool = B * pps + 7
    gen = torch.Generator().manual_seed(seed)
    bt = torch.randperm(pool, generator=gen)[:B * pps].to(torch.int32).view(B, pps)
    kp = torch.zeros(pool, page, Hkv, d, dtype=torch.bfloat16, device=dev)
    vp = torch.zeros_like(kp)
    for b in range(B):
        for j in range(pps):
            r0, r1 = j * page, min((j + 1) * page, cap)
            kp[int(bt[b, j]), :r1 - r0] = kc[b, r0:r1]
            vp[int(bt[b, j]), :r1 - r0] = vc[b, r0:r1]
    op, lp = fa.fa_fwd_kvcache_paged(q, kp, vp, bt.to(dev), lens, num_splits=S, scale=scale)
    torch.cuda.synchronize()

    lh = lens.cpu().numpy()
    qh, kh, vh = f64(q), f64(kc), f64(vc)
    o_ref, l_ref = O.decode(qh, kh, vh, [int(x) for x in lh], scale)
    assert np.max(np.abs(f64(o)[:, 0] - o_ref)) <= 2e-2
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(f64(lse)), fin)
    if fin.any():
        assert np.max(np.abs(f64(lse)[fin] - l_ref[fin])) <= 1e-3
    assert not f64(o)[:, 0][~fin].any()  # rows without keys: O = 0
    assert torch.equal(op.view(torch.int16), o.view(torch.int16))
    assert torch.equal(lp.view(torch.int32), lse.view(torch.int32))
