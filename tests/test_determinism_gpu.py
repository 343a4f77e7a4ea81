"""Run-to-run bitwise reproducibility of every kernel family.

Each path runs several times on the same inputs into output buffers that
start as zeros, NaN and noise, and every run must match the first bit for
bit. The kernels use no atomics and fixed reduction orders, so any
difference means a read of data that is not yet (or no longer) valid: an
LDS read racing a ring refill, or a register read inside an MFMA's latency.
Such faults are timing-dependent and can hide under the parity tolerances
of a single run; the shapes here cross the loop boundaries where they showed
(causal tiles whose wavefronts run one unmasked tile and then masked ones,
ragged tails, GQA).
"""

import math

import numpy as np
import pytest
import torch

import seeded_inputs as SI

pytestmark = pytest.mark.gpu

FILLS = (0.0, float("nan"), None)  # None: noise
REPEATS = 2                        # rounds over the three fills


def fa():
    import exact_io_aware_online_amd as m
    m.lib()
    return m


def note(msg):
    print(msg, flush=True)


def _filled(like, fill, gen):
    if fill is None:
        return (torch.randn(like.shape, generator=gen, device=like.device) * 1e3).to(like.dtype)
    return torch.full_like(like, fill)


def _same(runs, what):
    ref = runs[0]
    for i, r in enumerate(runs[1:], 1):
        for a, b, name in zip(ref, r, what):
            if a is None:
                continue
            eq = torch.equal(a.view(torch.int8), b.view(torch.int8)) if a.dtype != torch.bool else torch.equal(a, b)
            assert eq, f"run {i}: {name} differs in {(a.view(torch.int8) != b.view(torch.int8)).sum().item()} bytes"


def _repeat(call, outs_like, what):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    runs = []
    for _ in range(REPEATS):
        for fill in FILLS:
            outs = [_filled(t, fill, gen) for t in outs_like]
            call(*outs)
            torch.cuda.synchronize()
            runs.append([t.clone() for t in outs])
    _same(runs, what)


# (B, Hq, Hkv, Nq, Nk, causal, d)
PREFILL = [
    (1, 2, 2, 128, 128, True, 128),
    (2, 4, 2, 1000, 1000, True, 128),
    (1, 4, 1, 200, 777, False, 128),
    (2, 4, 4, 1000, 1000, True, 64),
    (1, 2, 1, 300, 513, False, 64),
    (2, 2, 2, 700, 700, True, 256),
    (1, 2, 1, 130, 257, False, 256),
]
IDS = lambda c: "B{}H{}kv{}q{}k{}{}d{}".format(*c[:5], "c" if c[5] else "", c[6])


@pytest.mark.parametrize("case", PREFILL, ids=IDS)
def test_prefill_bf16_reproducible(case):
    B, Hq, Hkv, Nq, Nk, causal, d = case
    note(f"repro bf16 fwd {IDS(case)}")
    q, k, v = SI.prefill_inputs(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, seed=900 + Nq, device="cuda")
    o0 = torch.empty_like(q)
    l0 = torch.empty(B, Hq, Nq, dtype=torch.float32, device="cuda")
    scale = float(np.float32(1.0 / math.sqrt(d)))
    _repeat(lambda o, lse: fa().fa_fwd(q, k, v, o=o, lse=lse, causal=causal, scale=scale), [o0, l0], ["O", "LSE"])


@pytest.mark.parametrize("case", PREFILL, ids=IDS)
def test_fp8_forward_reproducible(case):
    B, Hq, Hkv, Nq, Nk, causal, d = case
    note(f"repro fp8 fwd {IDS(case)}")
    ins = [t.to("cuda") for t in SI.fp8_inputs(B, Hq, Hkv, Nq, Nk, d, seed=910 + Nq)]
    o0 = torch.empty(B, Nq, Hq, d, dtype=torch.bfloat16, device="cuda")
    l0 = torch.empty(B, Hq, Nq, dtype=torch.float32, device="cuda")
    scale = float(np.float32(1.0 / math.sqrt(d)))
    _repeat(lambda o, lse: fa().fa_fwd_fp8(*ins, Nq, Nk, causal=causal, scale=scale, o=o, lse=lse), [o0, l0],
            ["O", "LSE"])


@pytest.mark.parametrize("case", [c for c in PREFILL if c[6] in (64, 128)], ids=IDS)
def test_backward_reproducible(case):
    B, Hq, Hkv, Nq, Nk, causal, d = case
    note(f"repro bwd {IDS(case)}")
    q, k, v = SI.prefill_inputs(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, seed=920 + Nq, device="cuda")
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = fa().fa_fwd(q, k, v, causal=causal, scale=scale)
    g = torch.Generator(device="cuda")
    g.manual_seed(921)
    dout = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    _repeat(lambda dq, dk, dv: fa().fa_bwd(q, k, v, o, lse, dout, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv),
            [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)], ["dQ", "dK", "dV"])


@pytest.mark.parametrize("d", [64, 128, 256])
def test_decode_reproducible(d):
    note(f"repro decode d={d}")
    B, Hq, Hkv, cap = 16, 8, 2, 3000
    q, kc, vc, lens = (t.to("cuda") for t in SI.decode_inputs(B, Hq, Hkv, cap, d, seed=930 + d, len_lo=1))
    o0 = torch.empty_like(q)
    l0 = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
    _repeat(lambda o, lse: fa().fa_fwd_kvcache(q, kc, vc, lens, o=o, lse=lse), [o0, l0], ["O", "LSE"])
