"""GPU parity of local windows (fa_fwd_window) and packed variable-length
batches (fa_fwd_varlen) against the float64 oracle (oracle.sdpa
.attention_window / .attention_varlen), plus bitwise agreement with fa_fwd
where the two describe the same attention.
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


def compare(o, lse, o_ref, l_ref):
    eo = float(np.max(np.abs(f64(o) - o_ref))) if o_ref.size else 0.0
    L = f64(lse)
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(L), fin), "rows without keys must have LSE = -inf"
    el = float(np.max(np.abs(L[fin] - l_ref[fin]), initial=0.0))
    note(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O and el <= TOL_LSE


# (B, Hq, Hkv, Nq, Nk, d, window_left, window_right)
WINDOW_CASES = [
    (1, 4, 2, 300, 300, 128, -1, 0),     # bottom-right causal, square (= top-left)
    (1, 4, 2, 200, 500, 128, -1, 0),     # bottom-right causal, more keys than queries
    (1, 4, 2, 500, 200, 128, -1, 0),     # more queries: the first 300 rows see no key
    (2, 2, 2, 400, 400, 128, 100, 0),    # causal sliding window of 101 keys
    (1, 4, 4, 333, 333, 128, 50, 70),    # two-sided window
    (1, 2, 1, 257, 400, 128, 130, -1),   # left bound only
    (1, 2, 2, 300, 300, 64, 64, 0),      # d = 64
    (1, 2, 2, 200, 260, 256, 31, 1),     # d = 256
    (1, 2, 2, 128, 128, 128, 0, 0),      # each query sees exactly one key
    (1, 2, 2, 100, 100, 128, -1, -1),    # no mask
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: "q{}k{}d{}w{}_{}".format(*c[3:]))
def test_window(case):
    B, Hq, Hkv, Nq, Nk, d, wl, wr = case
    note(f"window B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} wl={wl} wr={wr}")
    q, k, v = SI.prefill_inputs(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, seed=91, device=torch.device("cuda"))
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = fa().fa_fwd_window(q, k, v, wl, wr, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = O.attention_window(f64(q), f64(k), f64(v), wl, wr, scale)
    compare(o, lse, o_ref, l_ref)


@pytest.mark.parametrize("causal", [False, True])
def test_window_matches_fa_fwd_bitwise(causal):
    q, k, v = SI.prefill_inputs(B=2, Hq=4, Hkv=2, Nq=300, Nk=300, d=128, seed=92, device=torch.device("cuda"))
    m = fa()
    o1, l1 = m.fa_fwd(q, k, v, causal=causal)
    o2, l2 = m.fa_fwd_window(q, k, v, -1, 0 if causal else -1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


VARLEN_CASES = [
    # (query lengths, key lengths, Hq, Hkv, d, window_left, window_right)
    ([300, 1, 0, 129, 64], [300, 50, 7, 129, 200], 4, 2, 128, -1, -1),
    ([300, 1, 0, 129, 64], [300, 50, 7, 129, 200], 4, 2, 128, -1, 0),
    ([257, 511, 33], [257, 511, 100], 2, 2, 128, 64, 0),
    ([200, 130], [260, 130], 4, 1, 64, -1, 0),
    ([100, 90], [100, 300], 2, 2, 256, 20, 20),
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: f"n{len(c[0])}d{c[4]}w{c[5]}_{c[6]}")
def test_varlen(case):
    lq, lk, Hq, Hkv, d, wl, wr = case
    note(f"varlen lq={lq} lk={lk} Hq={Hq} Hkv={Hkv} d={d} wl={wl} wr={wr}")
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(93)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q = torch.randn(int(cu_q[-1]), Hq, d, generator=g).to(torch.bfloat16)
    k = torch.randn(int(cu_k[-1]), Hkv, d, generator=g).to(torch.bfloat16)
    v = torch.randn(int(cu_k[-1]), Hkv, d, generator=g).to(torch.bfloat16)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = fa().fa_fwd_varlen(q.to(dev), k.to(dev), v.to(dev), torch.tensor(cu_q, device=dev),
                                torch.tensor(cu_k, device=dev), max(lq), wl, wr, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = O.attention_varlen(f64(q), f64(k), f64(v), cu_q, cu_k, wl, wr, scale)
    compare(o, lse, o_ref, l_ref)


def test_varlen_equals_dense_per_sequence_bitwise():
    # a packed batch of equal-length sequences is the dense batch
    dev = torch.device("cuda")
    q, k, v = SI.prefill_inputs(B=3, Hq=4, Hkv=2, Nq=200, Nk=200, d=128, seed=94, device=dev)
    m = fa()
    od, ld = m.fa_fwd_window(q, k, v, -1, 0)
    cu = torch.arange(0, 601, 200, dtype=torch.int32, device=dev)
    ov, lv = m.fa_fwd_varlen(q.reshape(600, 4, 128), k.reshape(600, 2, 128), v.reshape(600, 2, 128), cu, cu, 200,
                             -1, 0)
    torch.cuda.synchronize()
    assert torch.equal(od.reshape(600, 4, 128), ov)
    assert torch.equal(ld.permute(1, 0, 2).reshape(4, 600), lv)


def test_varlen_sequence_longer_than_max_seqlen_is_nan():
    # max_seqlen_q sizes the launch; a sequence longer than it gets NaN in
    # every O and LSE row (the rows past the grid included), and the other
    # sequences are unaffected
    lq, lk = [150, 300, 70], [150, 320, 90]
    Hq, Hkv, d = 4, 2, 128
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(95)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q = torch.randn(int(cu_q[-1]), Hq, d, generator=g).to(torch.bfloat16)
    k = torch.randn(int(cu_k[-1]), Hkv, d, generator=g).to(torch.bfloat16)
    v = torch.randn(int(cu_k[-1]), Hkv, d, generator=g).to(torch.bfloat16)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o = torch.zeros(int(cu_q[-1]), Hq, d, dtype=torch.bfloat16, device=dev)
    lse = torch.zeros(Hq, int(cu_q[-1]), dtype=torch.float32, device=dev)
    fa().fa_fwd_varlen(q.to(dev), k.to(dev), v.to(dev), torch.tensor(cu_q, device=dev), torch.tensor(cu_k, device=dev),
                       200, -1, 0, o=o, lse=lse, scale=scale)
    torch.cuda.synchronize()
    bad = slice(int(cu_q[1]), int(cu_q[2]))
    assert torch.isnan(o[bad].float()).all() and torch.isnan(lse[:, bad]).all()
    o_ref, l_ref = O.attention_varlen(f64(q), f64(k), f64(v), cu_q, cu_k, -1, 0, scale)
    for s in (slice(0, int(cu_q[1])), slice(int(cu_q[2]), int(cu_q[3]))):
        assert np.max(np.abs(f64(o[s]) - o_ref[s])) <= 2e-2
        assert np.max(np.abs(f64(lse[:, s]) - l_ref[:, s])) <= 1e-3
