"""GPU parity of the FP8 forward: fa_quantize_fp8 against the oracle's block
quantisation (oracle.fp8.quantize_bhnd), fa_fwd_fp8 against the oracle's
attention on quantised operands (oracle.fp8.attention_fp8), and the whole
FP8 path against exact attention on the bf16 inputs (error statistics,
including the incoherent rotation's effect on outlier features).
"""

import math

import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import fp8 as F8
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


QUANT_CASES = [
    # (B, N, H, d)
    (2, 100, 3, 128),
    (1, 64, 2, 128),
    (1, 200, 2, 64),
    (2, 130, 1, 256),
    (1, 1, 1, 128),
]


@pytest.mark.parametrize("transpose", [False, True])
@pytest.mark.parametrize("case", QUANT_CASES, ids=lambda c: "B{}N{}H{}d{}".format(*c))
def test_quantize_bit_exact(case, transpose):
    B, N, H, d = case
    note(f"quantize B={B} N={N} H={H} d={d} transpose={transpose}")
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(300 + N)
    x = (torch.randn(B, N, H, d, generator=g) * 2.0 ** torch.randint(-6, 7, (B, N, H, 1), generator=g)).to(
        torch.bfloat16)
    codes, scales = fa().fa_quantize_fp8(x.to(dev), transpose=transpose)
    torch.cuda.synchronize()
    rc, re = F8.quantize_bhnd(f64(x))
    got_c = codes.cpu().numpy()
    if transpose:
        got_c = np.swapaxes(got_c, 2, 3)
    assert np.array_equal(scales.cpu().numpy().astype(np.int64) - 127, re)
    assert np.array_equal(got_c, rc)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_quantize_rotated(d):
    # The transform runs in float32 on the GPU and in float64 in the oracle:
    # a code may differ only where the oracle's unrounded value sits within
    # float32 rounding of the midpoint between two e4m3 neighbours.
    B, N, H = 2, 150, 2
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(310 + d)
    x = torch.randn(B, N, H, d, generator=g).to(torch.bfloat16)
    signs = SI.random_signs(d, seed=311)
    codes, scales = fa().fa_quantize_fp8(x.to(dev), signs=signs.to(dev))
    torch.cuda.synchronize()
    rc, re = F8.quantize_bhnd(f64(x), signs=signs.numpy().astype(np.float64))
    ge = scales.cpu().numpy().astype(np.int64) - 127
    assert np.array_equal(ge, re), "block exponents"
    gc = codes.cpu().numpy()
    bad = np.argwhere(gc != rc)
    note(f"  d={d}: {len(bad)} of {gc.size} codes differ")
    for bb, h, n, j in bad:
        assert n < N, ("padding row written", n)
        row = F8.rotate(f64(x)[bb, n, h], signs.numpy()) * 2.0 ** (-re[bb, h, n // 64])
        y = row[j]
        a, c = F8.e4m3_decode(rc[bb, h, n, j]), F8.e4m3_decode(gc[bb, h, n, j])
        assert abs(a - c) <= 2.0 ** -3 * max(abs(a), abs(c), 2.0 ** -6), ("codes are not neighbours", a, c)
        assert abs(y - (a + c) / 2) <= 1e-5 * np.max(np.abs(row)), ("code differs away from a midpoint", y, a, c)
    assert len(bad) <= max(2, gc.size // 10000)


# (B, Hq, Hkv, Nq, Nk, causal, d)
FWD_CASES = [
    (1, 2, 2, 128, 128, False, 128),
    (1, 2, 2, 128, 128, True, 128),
    (2, 4, 2, 300, 300, True, 128),     # ragged tiles, GQA
    (1, 4, 1, 200, 333, False, 128),    # Nq < Nk, MQA
    (1, 2, 2, 333, 100, True, 128),     # Nq > Nk: rows past the keys see all of them
    (1, 2, 2, 1, 70, False, 128),       # one query
    (1, 2, 1, 65, 1, False, 128),       # one key
    (2, 2, 2, 1000, 1000, True, 128),
    (2, 4, 2, 300, 300, True, 64),
    (1, 2, 1, 200, 333, False, 64),
    (2, 2, 2, 300, 300, True, 256),
    (1, 2, 1, 130, 257, False, 256),
]


@pytest.mark.parametrize("case", FWD_CASES,
                         ids=lambda c: "B{}H{}kv{}q{}k{}{}d{}".format(*c[:5], "c" if c[5] else "", c[6]))
def test_fwd_fp8_matches_oracle(case):
    B, Hq, Hkv, Nq, Nk, causal, d = case
    note(f"fp8 fwd B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} causal={causal}")
    dev = torch.device("cuda")
    ins = SI.fp8_inputs(B, Hq, Hkv, Nq, Nk, d, seed=320 + Nq)
    q8, qs, k8, ks, vt8, vs = ins
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = fa().fa_fwd_fp8(*(t.to(dev) for t in ins), Nq, Nk, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = F8.attention_fp8(q8.numpy(), qs.numpy().astype(np.int64) - 127, k8.numpy(),
                                    ks.numpy().astype(np.int64) - 127, np.swapaxes(vt8.numpy(), 2, 3),
                                    vs.numpy().astype(np.int64) - 127, Nq, Nk, causal, scale)
    eo = float(np.max(np.abs(f64(o) - o_ref)))
    L = f64(lse)
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(L), fin)
    el = float(np.max(np.abs(L[fin] - l_ref[fin]), initial=0.0))
    # The bf16 bar scaled by the output's size (as the backward tests do): a
    # probability within float32 rounding of an e4m3 midpoint may take the
    # other code (kernel scores are float32, the oracle's float64), moving a
    # row that averages few values by a few percent of one value.
    tol = TOL_O * max(1.0, float(np.max(np.abs(o_ref))))
    note(f"  max|dO|={eo:.3e} (max|O|={np.max(np.abs(o_ref)):.2f}, bound {tol:.3e}) max|dLSE|={el:.3e}")
    assert eo <= tol and el <= TOL_LSE


def test_fwd_fp8_no_keys():
    dev = torch.device("cuda")
    ins = SI.fp8_inputs(1, 2, 2, 70, 0, 128, seed=330)
    o, lse = fa().fa_fwd_fp8(*(t.to(dev) for t in ins), 70, 0, causal=False)
    torch.cuda.synchronize()
    assert not o.float().abs().max().item() and bool(torch.all(lse == -float("inf")))


def _pipeline(q, k, v, causal, signs):
    m = fa()
    q8, qs = m.fa_quantize_fp8(q, signs=signs)
    k8, ks = m.fa_quantize_fp8(k, signs=signs)
    vt8, vs = m.fa_quantize_fp8(v, transpose=True)
    return m.fa_fwd_fp8(q8, qs, k8, ks, vt8, vs, q.shape[1], k.shape[1], causal=causal,
                        scale=float(np.float32(1.0 / math.sqrt(q.shape[3]))))


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fp8_pipeline_error_against_exact_attention(d):
    # bf16 inputs -> FP8 quantisation -> FP8 attention, against exact fp64
    # attention on the bf16 inputs: the relative RMS error stays at the
    # level e4m3 rounding of Q, K and V allows (about 5% here: early causal
    # rows average few values, each off by up to 2^-4 relative), with and
    # without rotation
    dev = torch.device("cuda")
    q, k, v = SI.prefill_inputs(B=1, Hq=4, Hkv=2, Nq=512, Nk=512, d=d, seed=340, device=dev)
    ref, _ = O.attention(f64(q), f64(k), f64(v), True, float(np.float32(1.0 / math.sqrt(d))))
    for rot in (False, True):
        signs = SI.random_signs(d, seed=341).to(dev) if rot else None
        o, _ = _pipeline(q, k, v, True, signs)
        torch.cuda.synchronize()
        rel = float(np.sqrt(np.mean((f64(o) - ref) ** 2) / np.mean(ref ** 2)))
        note(f"  d={d} rotation={rot}: relative RMS error {rel:.4f}")
        assert rel < 0.08


def test_rotation_reduces_error_with_outlier_features():
    # a few head dimensions 8x larger than the rest (outlier features): one
    # block scale per 64 rows wastes precision on the others unless the
    # rotation spreads the outliers over all dimensions first
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(350)
    B, N, H, d = 1, 512, 2, 128
    q = torch.randn(B, N, H, d, generator=g)
    k = torch.randn(B, N, H, d, generator=g)
    v = torch.randn(B, N, H, d, generator=g)
    q[..., :4] *= 8.0
    k[..., :4] *= 8.0
    q, k, v = (t.to(torch.bfloat16).to(dev) for t in (q, k, v))
    scale = float(np.float32(1.0 / math.sqrt(d)))
    ref, _ = O.attention(f64(q), f64(k), f64(v), False, scale)
    errs = {}
    for rot in (False, True):
        signs = SI.random_signs(d, seed=351).to(dev) if rot else None
        o, _ = _pipeline(q, k, v, False, signs)
        torch.cuda.synchronize()
        errs[rot] = float(np.sqrt(np.mean((f64(o) - ref) ** 2) / np.mean(ref ** 2)))
        note(f"  outliers, rotation={rot}: relative RMS error {errs[rot]:.4f}")
    assert errs[True] < errs[False]


def test_fp8_full_size_sampled():
    # the training-shape workload (B=8, H=16, N=2048, d=128, causal) in FP8,
    # sampled heads against the oracle on the same codes
    B, H, N, d = 8, 16, 2048, 128
    dev = torch.device("cuda")
    ins = SI.fp8_inputs(B, H, H, N, N, d, seed=360)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = fa().fa_fwd_fp8(*(t.to(dev) for t in ins), N, N, causal=True, scale=scale)
    torch.cuda.synchronize()
    q8, qs, k8, ks, vt8, vs = (t.numpy() for t in ins)
    for b, h in ((0, 0), (B - 1, H - 1), (3, 7)):
        sl = lambda t: t[b:b + 1, h:h + 1]
        o_ref, l_ref = F8.attention_fp8(sl(q8), sl(qs).astype(np.int64) - 127, sl(k8), sl(ks).astype(np.int64) - 127,
                                        np.swapaxes(sl(vt8), 2, 3), sl(vs).astype(np.int64) - 127, N, N, True, scale)
        eo = float(np.max(np.abs(f64(o[b:b + 1, :, h:h + 1]) - o_ref)))
        el = float(np.max(np.abs(f64(lse[b:b + 1, h:h + 1]) - l_ref)))
        note(f"  b={b} h={h}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
        assert eo <= TOL_O and el <= TOL_LSE
