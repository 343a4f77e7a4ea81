"""GPU parity on a seeded sweep of small random shapes.

The hand-picked parity cases fix particular tails; this sweep draws shapes
from a fixed numpy generator, including query and key counts around the
32-row wavefront, the 128-row workgroup tile and the 64-key tile, GQA groups
of 1 to 4, d = 64 / 128 / 256 and both masks. Each case goes through
`fa_fwd` and, where d and the mask allow, through `fa_bwd`, against the
float64 oracle with the tolerances of the other parity tests (O and the
gradients relative to their magnitude, LSE absolute).
"""

import math

import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import sdpa as O

pytestmark = pytest.mark.gpu

EDGE = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 191, 255, 257]


def _cases(n=24, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128, 256]))
        g = int(rng.choice([1, 2, 4]))
        hkv = int(rng.choice([1, 2]))
        nq = int(rng.choice(EDGE)) if rng.random() < 0.6 else int(rng.integers(1, 320))
        nk = int(rng.choice(EDGE)) if rng.random() < 0.6 else int(rng.integers(1, 320))
        causal = bool(rng.random() < 0.5)
        b = int(rng.choice([1, 2]))
        out.append((b, hkv * g, hkv, nq, nk, d, causal, 500 + i))
    return out


CASES = _cases()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


@pytest.mark.parametrize("case", CASES, ids=["B{}H{}kv{}q{}k{}d{}c{}s{}".format(*c) for c in CASES])
def test_forward_sweep(case):
    import exact_io_aware_online_amd as fa
    B, Hq, Hkv, Nq, Nk, d, causal, seed = case
    print(f"forward sweep B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} seed={seed}", flush=True)
    dev = torch.device("cuda")
    q, k, v = SI.prefill_inputs(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, dtype="bf16", seed=seed, device=dev)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = O.attention(f64(q), f64(k), f64(v), causal, scale)
    assert np.max(np.abs(f64(o) - o_ref)) <= 2e-2
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(f64(lse)), fin)
    if fin.any():
        assert np.max(np.abs(f64(lse)[fin] - l_ref[fin])) <= 1e-3


BWD_CASES = [c for c in CASES if c[5] in (64, 128)][:10]


@pytest.mark.parametrize("case", BWD_CASES, ids=["B{}H{}kv{}q{}k{}d{}c{}s{}".format(*c) for c in BWD_CASES])
def test_backward_sweep(case):
    import exact_io_aware_online_amd as fa
    B, Hq, Hkv, Nq, Nk, d, causal, seed = case
    print(f"backward sweep B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} seed={seed}", flush=True)
    dev = torch.device("cuda")
    q, k, v = SI.prefill_inputs(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, dtype="bf16", seed=seed, device=dev)
    g = torch.Generator(device=dev).manual_seed(seed + 1)
    do = torch.randn(q.shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv = O.attention_backward(f64(q), f64(k), f64(v), f64(do), causal, scale)
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        err = np.max(np.abs(f64(got) - ref)) if ref.size else 0.0
        assert err <= 2e-2 * max(1.0, float(np.max(np.abs(ref))) if ref.size else 1.0), err


# Batches whose (sequence, key/value head) pair count is a multiple of 16 run
# their causal tiles in two chunks of pairs; these cases cover that order for
# MHA and GQA, with a ragged last query tile.
CHUNKED = [(2, 8, 8, 300, 300, 128, 900), (4, 16, 4, 257, 257, 128, 901), (16, 4, 1, 129, 129, 64, 902)]


@pytest.mark.parametrize("case", CHUNKED, ids=["B{}H{}kv{}q{}k{}d{}s{}".format(*c) for c in CHUNKED])
def test_forward_chunked_order(case):
    import exact_io_aware_online_amd as fa
    B, Hq, Hkv, Nq, Nk, d, seed = case
    print(f"chunked order B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} seed={seed}", flush=True)
    q, k, v = SI.prefill_inputs(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, dtype="bf16", seed=seed,
                                device=torch.device("cuda"))
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = fa.fa_fwd(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = O.attention(f64(q), f64(k), f64(v), True, scale)
    assert np.max(np.abs(f64(o) - o_ref)) <= 2e-2
    assert np.max(np.abs(f64(lse) - l_ref)) <= 1e-3


@pytest.mark.parametrize("case", [(2, 4, 2, 300, 300, True), (1, 4, 1, 520, 520, True), (1, 2, 2, 333, 129, False),
                                  (2, 2, 2, 1, 77, False)], ids=lambda c: "B{}H{}kv{}q{}k{}{}".format(*c))
def test_pipelined_tile_shape_variant(case, monkeypatch):
    # FA_FWD_VARIANT=4 selects, at d = 128, the one-wavefront-per-SIMD
    # pipelined shape (two query blocks per wavefront, 32-key tiles); it
    # must agree with the oracle like the default shape, and with windows
    B, Hq, Hkv, Nq, Nk, causal = case
    monkeypatch.setenv("FA_FWD_VARIANT", "4")
    dev = torch.device("cuda")
    q, k, v = SI.prefill_inputs(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=128, seed=950 + Nq, device=dev)
    scale = float(np.float32(1.0 / math.sqrt(128)))
    import exact_io_aware_online_amd as m
    o, lse = m.fa_fwd(q, k, v, causal=causal, scale=scale)
    ow, lw = m.fa_fwd_window(q, k, v, 40, 0, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = O.attention(f64(q), f64(k), f64(v), causal, scale)
    ow_ref, lw_ref = O.attention_window(f64(q), f64(k), f64(v), 40, 0, scale)
    for got_o, got_l, ro, rl in ((o, lse, o_ref, l_ref), (ow, lw, ow_ref, lw_ref)):
        fin = np.isfinite(rl)
        assert np.array_equal(np.isfinite(f64(got_l)), fin)
        assert np.max(np.abs(f64(got_o) - ro)) <= 2e-2
        assert np.max(np.abs(f64(got_l)[fin] - rl[fin]), initial=0.0) <= 1e-3
