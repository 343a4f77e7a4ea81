"""GPU parity of the backward under bottom-right windows (fa_bwd_window) and
over packed variable-length batches (fa_bwd_varlen) against the float64
oracle (oracle.sdpa.attention_backward_window / _varlen), plus bitwise
agreement with fa_bwd where the two describe the same attention.

The GPU backward gets the GPU forward's O and LSE, as a training step
would. Bound: element-wise max-abs error <= 2e-2 * max(1, max |reference|)
per gradient (bf16 inputs and outputs, bf16 P and dS in the products).
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


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def note(msg):
    print(msg, flush=True)


def tol(ref):
    return 2e-2 * max(1.0, float(np.max(np.abs(ref))) if ref.size else 1.0)


def check(name, got, ref):
    err = float(np.max(np.abs(f64(got) - ref))) if ref.size else 0.0
    note(f"  {name}: max|err|={err:.3e} (bound {tol(ref):.3e})")
    assert np.isfinite(f64(got)).all()
    assert err <= tol(ref), (name, err)


# (B, Hq, Hkv, Nq, Nk, d, window_left, window_right)
WINDOW_CASES = [
    (1, 4, 2, 200, 500, 128, -1, 0),     # bottom-right causal, more keys than queries
    (1, 4, 2, 500, 200, 128, -1, 0),     # more queries: the first 300 rows see no key
    (2, 2, 2, 400, 400, 128, 100, 0),    # causal sliding window of 101 keys
    (1, 4, 4, 333, 333, 128, 50, 70),    # two-sided window
    (1, 2, 1, 257, 400, 128, 130, -1),   # left bound only
    (1, 2, 2, 300, 300, 64, 64, 0),      # d = 64
    (1, 2, 2, 128, 128, 128, 0, 0),      # each query sees exactly one key
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: "q{}k{}d{}w{}_{}".format(*c[3:]))
def test_backward_window(case):
    B, Hq, Hkv, Nq, Nk, d, wl, wr = case
    note(f"backward window B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} wl={wl} wr={wr}")
    dev = torch.device("cuda")
    q, k, v = SI.prefill_inputs(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, seed=111, device=dev)
    do = torch.randn(q.shape, generator=torch.Generator(device=dev).manual_seed(112), device=dev).to(torch.bfloat16)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    m = fa()
    o, lse = m.fa_fwd_window(q, k, v, wl, wr, scale=scale)
    dq, dk, dv = m.fa_bwd_window(q, k, v, o, lse, do, wl, wr, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv = O.attention_backward_window(f64(q), f64(k), f64(v), f64(do), wl, wr, scale)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        check(name, got, ref)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_window_matches_fa_bwd_bitwise(causal):
    dev = torch.device("cuda")
    q, k, v = SI.prefill_inputs(B=2, Hq=4, Hkv=2, Nq=300, Nk=300, d=128, seed=113, device=dev)
    do = torch.randn(q.shape, generator=torch.Generator(device=dev).manual_seed(114), device=dev).to(torch.bfloat16)
    m = fa()
    o, lse = m.fa_fwd(q, k, v, causal=causal)
    a = m.fa_bwd(q, k, v, o, lse, do, causal=causal)
    b = m.fa_bwd_window(q, k, v, o, lse, do, -1, 0 if causal else -1)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


VARLEN_CASES = [
    # (query lengths, key lengths, Hq, Hkv, d, window_left, window_right)
    ([300, 1, 0, 129, 64], [300, 50, 7, 129, 200], 4, 2, 128, -1, -1),
    ([300, 1, 0, 129, 64], [300, 50, 7, 129, 200], 4, 2, 128, -1, 0),
    ([257, 511, 33], [257, 511, 100], 2, 2, 128, 64, 0),
    ([200, 130], [260, 130], 4, 1, 64, -1, 0),
    ([90, 40], [0, 120], 2, 2, 128, -1, -1),           # a sequence without keys
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: f"n{len(c[0])}d{c[4]}w{c[5]}_{c[6]}")
def test_backward_varlen(case):
    lq, lk, Hq, Hkv, d, wl, wr = case
    note(f"backward varlen lq={lq} lk={lk} Hq={Hq} Hkv={Hkv} d={d} wl={wl} wr={wr}")
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(115)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q = torch.randn(int(cu_q[-1]), Hq, d, generator=g).to(torch.bfloat16).to(dev)
    k = torch.randn(int(cu_k[-1]), Hkv, d, generator=g).to(torch.bfloat16).to(dev)
    v = torch.randn(int(cu_k[-1]), Hkv, d, generator=g).to(torch.bfloat16).to(dev)
    do = torch.randn(int(cu_q[-1]), Hq, d, generator=g).to(torch.bfloat16).to(dev)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    cq, ck = torch.tensor(cu_q, device=dev), torch.tensor(cu_k, device=dev)
    m = fa()
    o, lse = m.fa_fwd_varlen(q, k, v, cq, ck, max(lq), wl, wr, scale=scale)
    dq, dk, dv = m.fa_bwd_varlen(q, k, v, o, lse, do, cq, ck, max(lq), max(lk), wl, wr, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv = O.attention_backward_varlen(f64(q), f64(k), f64(v), f64(do), cu_q, cu_k, wl, wr, scale)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        check(name, got, ref)


def test_backward_varlen_equals_dense_bitwise():
    # a packed batch of equal-length sequences is the dense batch
    dev = torch.device("cuda")
    q, k, v = SI.prefill_inputs(B=3, Hq=4, Hkv=2, Nq=200, Nk=200, d=128, seed=116, device=dev)
    do = torch.randn(q.shape, generator=torch.Generator(device=dev).manual_seed(117), device=dev).to(torch.bfloat16)
    m = fa()
    o, lse = m.fa_fwd_window(q, k, v, -1, 0)
    a = m.fa_bwd_window(q, k, v, o, lse, do, -1, 0)
    cu = torch.arange(0, 601, 200, dtype=torch.int32, device=dev)
    pk = lambda t: t.reshape(600, t.shape[2], t.shape[3])
    ov, lv = m.fa_fwd_varlen(pk(q), pk(k), pk(v), cu, cu, 200, -1, 0)
    b = m.fa_bwd_varlen(pk(q), pk(k), pk(v), ov, lv, pk(do), cu, cu, 200, 200, -1, 0)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(pk(x), y)


@pytest.mark.parametrize("which", ["q", "k"])
def test_backward_varlen_sequence_longer_than_max_seqlen_is_nan(which):
    # a sequence longer than max_seqlen_q (or _k) gets NaN in every dq, dk
    # and dv row (rows past the grid included); the others are unaffected
    lq, lk = [150, 200, 70], [150, 260, 90]
    Hq, Hkv, d = 4, 2, 128
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(118)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q = torch.randn(int(cu_q[-1]), Hq, d, generator=g).to(torch.bfloat16).to(dev)
    k = torch.randn(int(cu_k[-1]), Hkv, d, generator=g).to(torch.bfloat16).to(dev)
    v = torch.randn(int(cu_k[-1]), Hkv, d, generator=g).to(torch.bfloat16).to(dev)
    do = torch.randn(int(cu_q[-1]), Hq, d, generator=g).to(torch.bfloat16).to(dev)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    cq, ck = torch.tensor(cu_q, device=dev), torch.tensor(cu_k, device=dev)
    m = fa()
    o, lse = m.fa_fwd_varlen(q, k, v, cq, ck, max(lq), -1, 0, scale=scale)
    mq, mk = (150, max(lk)) if which == "q" else (max(lq), 200)
    dq, dk, dv = (torch.zeros_like(t) for t in (q, k, v))
    m.fa_bwd_varlen(q, k, v, o, lse, do, cq, ck, mq, mk, -1, 0, scale=scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    bq, bk = slice(int(cu_q[1]), int(cu_q[2])), slice(int(cu_k[1]), int(cu_k[2]))
    assert torch.isnan(dq[bq].float()).all()
    assert torch.isnan(dk[bk].float()).all() and torch.isnan(dv[bk].float()).all()
    rq, rk, rv = O.attention_backward_varlen(f64(q), f64(k), f64(v), f64(do), cu_q, cu_k, -1, 0, scale)
    for sq_, sk_ in ((slice(0, int(cu_q[1])), slice(0, int(cu_k[1]))),
                     (slice(int(cu_q[2]), int(cu_q[3])), slice(int(cu_k[2]), int(cu_k[3])))):
        check("dq", dq[sq_], rq[sq_])
        check("dk", dk[sk_], rk[sk_])
        check("dv", dv[sk_], rv[sk_])


def test_backward_split_pass_variant_takes_windows_and_packed_batches(monkeypatch):
    # FA_BWD_VARIANT=1 computes dK and dV in two passes; it must honour the
    # window rule and the packed layout like the default kernel
    monkeypatch.setenv("FA_BWD_VARIANT", "1")
    test_backward_window(WINDOW_CASES[2])
    test_backward_window(WINDOW_CASES[3])
    test_backward_varlen(VARLEN_CASES[1])
