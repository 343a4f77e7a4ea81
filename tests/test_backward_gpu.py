"""GPU parity of the backward pass (fa_bwd) against the float64 oracle.

The oracle differentiates the forward definition (oracle.sdpa
.attention_backward, pinned in tests/oracle_pins.py). The GPU backward gets
the GPU forward's O and LSE, as a training step would. Bound: element-wise
max-abs error <= 2e-2 * max(1, max |reference|) per gradient (bf16 outputs,
bf16 probabilities and dS in the products, fp32 accumulation).
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


def run(B, Hq, Hkv, Nq, Nk, d, causal, seed):
    dev = torch.device("cuda")
    q, k, v = SI.prefill_inputs(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, seed=seed, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(seed + 1000)
    do = torch.randn(q.shape, generator=g, device=dev).to(torch.bfloat16)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    m = fa()
    o, lse = m.fa_fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = m.fa_bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return q, k, v, do, o, lse, dq, dk, dv, scale


# (B, Hq, Hkv, Nq, Nk, d, causal)
CASES = [
    (1, 2, 2, 128, 128, 128, False),
    (1, 2, 2, 128, 128, 128, True),
    (2, 3, 3, 300, 300, 128, True),     # ragged query and key tiles
    (2, 3, 3, 300, 300, 128, False),
    (1, 8, 2, 200, 200, 128, True),     # GQA: dK, dV summed over 4 query heads
    (1, 4, 1, 161, 161, 128, False),    # MQA
    (1, 2, 2, 100, 333, 128, False),    # Nq < Nk
    (1, 2, 2, 333, 100, 128, True),     # Nq > Nk, top-left causal
    (2, 4, 4, 257, 257, 64, True),      # d = 64
    (1, 4, 2, 190, 130, 64, False),
    (1, 2, 2, 1, 50, 128, False),       # one query
    (1, 2, 2, 40, 1, 128, False),       # one key
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}kv{}q{}k{}d{}{}".format(*c[:6], "c" if c[6] else ""))
def test_backward_small(case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    note(f"backward B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal}")
    q, k, v, do, o, lse, dq, dk, dv, scale = run(B, Hq, Hkv, Nq, Nk, d, causal, seed=71)
    rq, rk, rv = O.attention_backward(f64(q), f64(k), f64(v), f64(do), causal, scale)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        err = float(np.max(np.abs(f64(got) - ref))) if ref.size else 0.0
        note(f"  {name}: max|err|={err:.3e} (bound {tol(ref):.3e}, max|ref|={np.max(np.abs(ref)):.2f})")
        assert np.isfinite(f64(got)).all()
        assert err <= tol(ref), (name, err)


def test_backward_deterministic():
    a = run(1, 4, 2, 300, 300, 128, True, seed=72)
    b = run(1, 4, 2, 300, 300, 128, True, seed=72)
    for x, y in zip(a[6:9], b[6:9]):
        assert torch.equal(x, y)


def test_backward_constant_values_zero_dq_dk():
    # constant value rows: O does not depend on Q or K, so dQ = dK = 0 up to rounding
    dev = torch.device("cuda")
    q, k, v = SI.prefill_inputs(B=1, Hq=2, Hkv=2, Nq=150, Nk=150, d=128, seed=73, device=dev)
    v = v[:, :1].expand_as(v).contiguous()
    do = torch.randn(q.shape, generator=torch.Generator(device=dev).manual_seed(5), device=dev).to(torch.bfloat16)
    m = fa()
    o, lse = m.fa_fwd(q, k, v, causal=True)
    dq, dk, dv = m.fa_bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    note(f"  max|dq|={dq.abs().max().item():.3e} max|dk|={dk.abs().max().item():.3e}")
    assert dq.abs().max().item() <= 2e-2 and dk.abs().max().item() <= 2e-2
    # the value gradients sum (over keys) to the sum of dO over queries
    want = do.float().sum(dim=1)
    got = dv.float().sum(dim=1)
    assert (got - want).abs().max().item() <= 0.05 * max(1.0, want.abs().max().item())


def test_backward_abi_errors():
    m = fa()
    dev = torch.device("cuda")
    q, k, v = SI.prefill_inputs(B=1, Hq=2, Hkv=2, Nq=64, Nk=64, d=256, seed=74, device=dev)
    o, lse = m.fa_fwd(q, k, v)
    with pytest.raises(m.FAError) as e:
        m.fa_bwd(q, k, v, o, lse, o)
    assert e.value.status == m.FA_ERR_UNSUPPORTED


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mha_bf16_causal_b8_h16_n2048_d128", "gqa_bf16_causal_h32kv8_n16384_d128"])
def test_backward_full_size_sampled(name):
    # Both workloads at their real sizes (the 16K one at N = 16384). The
    # float64 reference materialises N x N matrices per query head, so it is
    # taken for a few key/value head groups: three of the training shape,
    # one (the last, all four of its query heads) of the 16K workload.
    w = dict(SI.PREFILL_WORKLOADS[name])
    note(f"full-size backward {name}")
    dev = torch.device("cuda")
    q, k, v = SI.prefill_inputs(device=dev, **w)
    do = torch.randn(q.shape, generator=torch.Generator(device=dev).manual_seed(9), device=dev).to(torch.bfloat16)
    scale = float(np.float32(1.0 / math.sqrt(w["d"])))
    m = fa()
    o, lse = m.fa_fwd(q, k, v, causal=w["causal"], scale=scale)
    dq, dk, dv = m.fa_bwd(q, k, v, o, lse, do, causal=w["causal"], scale=scale)
    torch.cuda.synchronize()
    assert all(torch.isfinite(t.float()).all() for t in (dq, dk, dv))
    G = w["Hq"] // w["Hkv"]
    rng = np.random.default_rng(w["seed"])
    if w["Nq"] > 4096:
        groups = [(0, w["Hkv"] - 1)]
    else:
        groups = {(0, 0), (w["B"] - 1, w["Hkv"] - 1), (int(rng.integers(w["B"])), int(rng.integers(w["Hkv"])))}
    from concurrent.futures import ThreadPoolExecutor
    for b, kvh in groups:
        qs, ks, vs, ds = (f64(t[b:b + 1]) for t in (q, k, v, do))
        rk = np.zeros((w["Nk"], w["d"]))
        rv = np.zeros((w["Nk"], w["d"]))
        with ThreadPoolExecutor(max_workers=G) as ex:
            grads = list(ex.map(lambda hq: O.attention_backward_rows(qs, ks, vs, ds, w["causal"], scale, 0, hq),
                                range(kvh * G, (kvh + 1) * G)))
        for hq, (gq, gk, gv) in zip(range(kvh * G, (kvh + 1) * G), grads):
            rk += gk
            rv += gv
            err = np.max(np.abs(f64(dq[b, :, hq]) - gq))
            assert err <= tol(gq), ("dq", b, hq, err)
        for n, got, ref in (("dk", dk[b, :, kvh], rk), ("dv", dv[b, :, kvh], rv)):
            err = np.max(np.abs(f64(got) - ref))
            note(f"  b={b} kvh={kvh} {n}: max|err|={err:.3e} (bound {tol(ref):.3e})")
            assert err <= tol(ref), (n, b, kvh, err)
