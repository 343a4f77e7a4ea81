"""GPU parity of the hand-scheduled 64-row prefill shape (head dim 128,
selected with FA_FWD_VARIANT=5): every case against the float64 oracle with
the bars of the other parity tests (O 2e-2, LSE 1e-3 absolute), over ragged
query and key counts around the 64-row wavefront, the 128-row workgroup and
the 64-key tile, causal and not, GQA, Nq != Nk, sliding windows (masked
tiles at both ends), packed batches, rows that see no key, and a workload
long enough for many unmasked tiles in a row, where the shape also has to
agree with the default one within the same bars."""

import math

import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import sdpa as O

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 2e-2, 1e-3


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def fa():
    import exact_io_aware_online_amd as m
    m.lib()
    return m


def check(o, lse, o_ref, l_ref):
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(f64(lse)), fin)
    eo = float(np.max(np.abs(f64(o) - o_ref))) if o_ref.size else 0.0
    el = float(np.max(np.abs(f64(lse)[fin] - l_ref[fin]), initial=0.0))
    print(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O and el <= TOL_LSE


CASES = [(1, 2, 2, 1, 1, True), (1, 2, 2, 63, 63, True), (1, 2, 1, 64, 64, True), (2, 4, 2, 65, 65, True),
         (1, 2, 2, 127, 127, False), (1, 4, 4, 128, 128, True), (2, 2, 1, 129, 129, True), (1, 2, 2, 300, 300, True),
         (1, 2, 2, 300, 300, False), (2, 4, 1, 257, 520, False), (1, 2, 2, 520, 257, True), (1, 2, 2, 333, 129, False),
         (2, 2, 2, 1, 77, False), (1, 8, 2, 1000, 1000, True)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}kv{}q{}k{}{}".format(*c))
def test_asm_shape_dense(case, monkeypatch):
    B, Hq, Hkv, Nq, Nk, causal = case
    print(f"asm shape dense B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} causal={causal}", flush=True)
    monkeypatch.setenv("FA_FWD_VARIANT", "5")
    dev = torch.device("cuda")
    q, k, v = SI.prefill_inputs(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=128, seed=1500 + Nq + Nk, device=dev)
    scale = float(np.float32(1.0 / math.sqrt(128)))
    o, lse = fa().fa_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    check(o, lse, *O.attention(f64(q), f64(k), f64(v), causal, scale))


@pytest.mark.parametrize("case", [(300, 300, 40, 0), (400, 400, 100, 0), (333, 333, 50, 70), (257, 400, 130, -1),
                                  (200, 500, -1, 0), (500, 200, -1, 0), (128, 128, 0, 0)],
                         ids=lambda c: "q{}k{}w{}_{}".format(*c))
def test_asm_shape_window(case, monkeypatch):
    Nq, Nk, wl, wr = case
    print(f"asm shape window Nq={Nq} Nk={Nk} window=({wl}, {wr})", flush=True)
    monkeypatch.setenv("FA_FWD_VARIANT", "5")
    dev = torch.device("cuda")
    q, k, v = SI.prefill_inputs(B=1, Hq=4, Hkv=2, Nq=Nq, Nk=Nk, d=128, seed=1600 + Nq, device=dev)
    scale = float(np.float32(1.0 / math.sqrt(128)))
    o, lse = fa().fa_fwd_window(q, k, v, wl, wr, scale=scale)
    torch.cuda.synchronize()
    check(o, lse, *O.attention_window(f64(q), f64(k), f64(v), wl, wr, scale))


def test_asm_shape_varlen(monkeypatch):
    print("asm shape varlen", flush=True)
    monkeypatch.setenv("FA_FWD_VARIANT", "5")
    dev = torch.device("cuda")
    lq, lk = [130, 0, 64, 257, 1], [200, 5, 64, 257, 0]
    Hq, Hkv, d = 4, 2, 128
    g = torch.Generator(device=dev).manual_seed(1700)
    q = torch.randn(sum(lq), Hq, d, generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn(sum(lk), Hkv, d, generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn(sum(lk), Hkv, d, generator=g, device=dev).to(torch.bfloat16)
    cq = torch.tensor(np.concatenate([[0], np.cumsum(lq)]), dtype=torch.int32, device=dev)
    ck = torch.tensor(np.concatenate([[0], np.cumsum(lk)]), dtype=torch.int32, device=dev)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = fa().fa_fwd_varlen(q, k, v, cq, ck, max(lq), -1, 0, scale=scale)
    torch.cuda.synchronize()
    check(o, lse, *O.attention_varlen(f64(q), f64(k), f64(v), cq.cpu().numpy(), ck.cpu().numpy(), -1, 0, scale))


def test_asm_shape_long_causal_matches_default(monkeypatch):
    # many unmasked tiles per wavefront, the two-chunk work order
    print("asm shape long causal B=2 Hq=8 Hkv=2 N=2048", flush=True)
    dev = torch.device("cuda")
    q, k, v = SI.prefill_inputs(B=2, Hq=8, Hkv=2, Nq=2048, Nk=2048, d=128, seed=1800, device=dev)
    scale = float(np.float32(1.0 / math.sqrt(128)))
    monkeypatch.setenv("FA_FWD_VARIANT", "5")
    o, lse = fa().fa_fwd(q, k, v, causal=True, scale=scale)
    monkeypatch.setenv("FA_FWD_VARIANT", "0")
    o0, l0 = fa().fa_fwd(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    assert float((o.float() - o0.float()).abs().max()) <= TOL_O
    assert float((lse - l0).abs().max()) <= TOL_LSE
    # the oracle on two heads' rows
    for b, h in ((0, 3), (1, 6)):
        kv = h // 4
        o_ref, l_ref = O.attention(f64(q[b:b + 1, :, h:h + 1]), f64(k[b:b + 1, :, kv:kv + 1]),
                                   f64(v[b:b + 1, :, kv:kv + 1]), True, scale)
        check(o[b:b + 1, :, h:h + 1], lse[b:b + 1, h:h + 1], o_ref, l_ref)
