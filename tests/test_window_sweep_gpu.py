"""GPU parity of windows and packed batches on a seeded sweep of random shapes.

Dense batches with random Nq != Nk, GQA groups, head dimensions and window
bounds (unlimited, zero, or random on either side; bottom-right aligned) go
through fa_fwd_window and, at d = 64 / 128, fa_bwd_window; packed batches with
random sequence lengths (empty sequences included) through fa_fwd_varlen and
fa_bwd_varlen. Each is compared with the float64 oracle: O and LSE at the
bars of the other parity tests (rows that see no key: O = 0, LSE = -inf), the
gradients within 2e-2 x max(1, max|reference|).
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


def _window(rng):
    r = rng.random()
    if r < 0.25:
        return -1
    if r < 0.4:
        return 0
    return int(rng.integers(1, 300))


def _dense_cases(n=16, seed=2028):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128, 256]))
        hkv = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 2, 4]))
        out.append((int(rng.choice([1, 2])), hkv * g, hkv, int(rng.integers(1, 400)), int(rng.integers(1, 400)), d,
                    _window(rng), _window(rng), 1100 + i))
    return out


def _packed_cases(n=10, seed=2029):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128, 256]))
        hkv = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 2, 4]))
        B = int(rng.integers(1, 6))
        lq = [int(x) for x in rng.integers(0, 300, B)]
        lk = [int(x) for x in rng.integers(0, 300, B)]
        lq[0] = max(lq[0], 1)
        out.append((tuple(lq), tuple(lk), hkv * g, hkv, d, _window(rng), _window(rng), 1200 + i))
    return out


def _check_fwd(o, lse, o_ref, l_ref):
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(f64(lse)), fin)
    assert np.max(np.abs(f64(o) - o_ref), initial=0.0) <= 2e-2
    assert np.max(np.abs(f64(lse)[fin] - l_ref[fin]), initial=0.0) <= 1e-3


def _check_grad(got, ref):
    err = np.max(np.abs(f64(got) - ref), initial=0.0)
    assert err <= 2e-2 * max(1.0, float(np.max(np.abs(ref), initial=0.0))), err


DENSE = _dense_cases()


@pytest.mark.parametrize("case", DENSE, ids=["B{}H{}kv{}q{}k{}d{}w{}_{}s{}".format(*c) for c in DENSE])
def test_window_sweep(case):
    B, Hq, Hkv, Nq, Nk, d, wl, wr, seed = case
    print(f"window sweep B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} wl={wl} wr={wr} seed={seed}", flush=True)
    m = fa()
    dev = torch.device("cuda")
    g = torch.Generator(device=dev).manual_seed(seed)
    q = torch.randn(B, Nq, Hq, d, generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn(B, Nk, Hkv, d, generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn(B, Nk, Hkv, d, generator=g, device=dev).to(torch.bfloat16)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = m.fa_fwd_window(q, k, v, wl, wr, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = O.attention_window(f64(q), f64(k), f64(v), wl, wr, scale)
    _check_fwd(o, lse, o_ref, l_ref)
    if d in (64, 128):
        do = torch.randn(q.shape, generator=g, device=dev).to(torch.bfloat16)
        dq, dk, dv = m.fa_bwd_window(q, k, v, o, lse, do, wl, wr, scale=scale)
        torch.cuda.synchronize()
        rq, rk, rv = O.attention_backward_window(f64(q), f64(k), f64(v), f64(do), wl, wr, scale)
        for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
            _check_grad(got, ref)


PACKED = _packed_cases()


@pytest.mark.parametrize("case", PACKED, ids=["n{}H{}kv{}d{}w{}_{}s{}".format(len(c[0]), *c[2:]) for c in PACKED])
def test_varlen_sweep(case):
    lq, lk, Hq, Hkv, d, wl, wr, seed = case
    print(f"varlen sweep lq={lq} lk={lk} Hq={Hq} Hkv={Hkv} d={d} wl={wl} wr={wr} seed={seed}", flush=True)
    m = fa()
    dev = torch.device("cuda")
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    g = torch.Generator(device=dev).manual_seed(seed)
    q = torch.randn(int(cu_q[-1]), Hq, d, generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn(max(int(cu_k[-1]), 1), Hkv, d, generator=g, device=dev).to(torch.bfloat16)[:int(cu_k[-1])]
    v = torch.randn(max(int(cu_k[-1]), 1), Hkv, d, generator=g, device=dev).to(torch.bfloat16)[:int(cu_k[-1])]
    scale = float(np.float32(1.0 / math.sqrt(d)))
    cq, ck = torch.tensor(cu_q, device=dev), torch.tensor(cu_k, device=dev)
    o, lse = m.fa_fwd_varlen(q, k, v, cq, ck, max(lq), wl, wr, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = O.attention_varlen(f64(q), f64(k), f64(v), cu_q, cu_k, wl, wr, scale)
    _check_fwd(o, lse, o_ref, l_ref)
    if d in (64, 128):
        do = torch.randn(q.shape, generator=g, device=dev).to(torch.bfloat16)
        dq, dk, dv = m.fa_bwd_varlen(q, k, v, o, lse, do, cq, ck, max(lq), max(lk), wl, wr, scale=scale)
        torch.cuda.synchronize()
        rq, rk, rv = O.attention_backward_varlen(f64(q), f64(k), f64(v), f64(do), cu_q, cu_k, wl, wr, scale)
        for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
            _check_grad(got, ref)
