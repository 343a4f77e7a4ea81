"""Element-wise parity at the workloads' full sizes, in the launch
configuration bench.py times (same library calls, default tile shapes,
default split count): every O and LSE element of the causal training shape
(B=8, H=16, N=2048), of both variance-4 non-causal shapes (d=64 and d=256)
and of the GQA decode workload; for the 16K causal GQA prefill, all 16384
rows of one query head per key/value head (a different position in the
group for each), which covers every key/value head and every query tile
of the launch's work order.

The oracle materialises each (batch, head)'s score rows in float64; the
heads run on a thread pool with the BLAS threads split between workers.
Bars as everywhere: O max-abs 2e-2 (bf16), LSE max-abs 1e-3.
"""

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import sdpa as O

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 2e-2, 1e-3
WORKERS = max(1, min(8, (os.cpu_count() or 2) // 2))


def fa():
    import exact_io_aware_online_amd as m
    m.lib()
    return m


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def note(msg):
    print(msg, flush=True)


def pool_map(fn, items):
    try:
        from threadpoolctl import threadpool_limits
        limits = threadpool_limits(limits=max(1, (os.cpu_count() or 2) // WORKERS))
    except Exception:  # pragma: no cover - threadpoolctl missing
        limits = None
    try:
        with ThreadPoolExecutor(max_workers=WORKERS) as ex:
            return list(ex.map(fn, items))
    finally:
        if limits is not None:
            limits.restore_original_limits()


def run(name):
    w = SI.PREFILL_WORKLOADS[name]
    dev = torch.device("cuda")
    q, k, v = SI.prefill_inputs(device=dev, **w)
    scale = float(np.float32(1.0 / math.sqrt(w["d"])))
    o, lse = fa().fa_fwd(q, k, v, causal=w["causal"], scale=scale)
    torch.cuda.synchronize()
    return w, q.cpu(), k.cpu(), v.cpu(), o.cpu(), lse.cpu(), scale


def head_errors(w, q, k, v, o, lse, scale, b, h, block=2048):
    """Max-abs O and LSE errors of one (batch, query head) over all rows,
    computed in blocks of query rows (causal blocks see their key prefix)."""
    kv = O.kv_head_of(h, w["Hq"], w["Hkv"])
    kk = f64(k[b:b + 1, :, kv:kv + 1])
    vv = f64(v[b:b + 1, :, kv:kv + 1])
    eo = el = 0.0
    for r0 in range(0, w["Nq"], block):
        r1 = min(r0 + block, w["Nq"])
        if w["causal"]:
            nk = min(r1, w["Nk"])
            o_ref, l_ref = O.attention_rows(f64(q[b:b + 1, :r1, h:h + 1]), kk[:, :nk], vv[:, :nk], True, scale, 0, 0,
                                            rows=np.arange(r0, r1))
        else:
            o_ref, l_ref = O.attention_rows(f64(q[b:b + 1, r0:r1, h:h + 1]), kk, vv, False, scale, 0, 0)
        eo = max(eo, float(np.max(np.abs(f64(o[b, r0:r1, h]) - o_ref))))
        el = max(el, float(np.max(np.abs(f64(lse[b, h, r0:r1]) - l_ref))))
    return eo, el


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mha_bf16_causal_b8_h16_n2048_d128", "mha_bf16_b4_h16_n4096_d64_qkvar4",
                                  "mha_bf16_b2_h8_n4096_d256_qkvar4"])
def test_prefill_full_size_every_element(name):
    note(f"full-size prefill, every element: {name}")
    w, q, k, v, o, lse, scale = run(name)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    pairs = [(b, h) for b in range(w["B"]) for h in range(w["Hq"])]
    errs = pool_map(lambda bh: head_errors(w, q, k, v, o, lse, scale, *bh), pairs)
    eo = max(e[0] for e in errs)
    el = max(e[1] for e in errs)
    note(f"  {len(pairs)} (batch, head) slices, all rows: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O and el <= TOL_LSE


@pytest.mark.timeout(900)
def test_long_gqa_prefill_full_size_one_head_per_kv_head():
    name = "gqa_bf16_causal_h32kv8_n16384_d128"
    note(f"full-size prefill: {name}, all rows of one query head per key/value head")
    w, q, k, v, o, lse, scale = run(name)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    G = w["Hq"] // w["Hkv"]
    heads = [kv * G + kv % G for kv in range(w["Hkv"])]
    errs = pool_map(lambda h: head_errors(w, q, k, v, o, lse, scale, 0, h), heads)
    for h, (eo, el) in zip(heads, errs):
        note(f"  head {h}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert max(e[0] for e in errs) <= TOL_O and max(e[1] for e in errs) <= TOL_LSE


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(SI.DECODE_WORKLOADS))
def test_decode_full_size_every_element(name):
    w = SI.DECODE_WORKLOADS[name]
    dev = torch.device("cuda")
    note(f"full-size decode, every element: {name}")
    q, kc, vc, lens = SI.decode_inputs(device=dev, **w)
    scale = float(np.float32(1.0 / math.sqrt(w["d"])))
    m = fa()
    S = m.fa_kvcache_default_splits(w["B"], w["Hkv"], w["capacity"], w["d"])
    o, lse = m.fa_fwd_kvcache(q, kc, vc, lens, num_splits=S, scale=scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    qh, kh, vh, lh = q.cpu(), kc.cpu(), vc.cpu(), lens.cpu().numpy()
    oh, lsh = f64(o), f64(lse)

    def seq(b):
        n = int(lh[b])
        o_ref, l_ref = O.decode(f64(qh[b:b + 1]), f64(kh[b:b + 1, :n]), f64(vh[b:b + 1, :n]), [n], scale)
        return float(np.max(np.abs(oh[b, 0] - o_ref[0]))), float(np.max(np.abs(lsh[b] - l_ref[0])))
    errs = pool_map(seq, range(w["B"]))
    eo = max(e[0] for e in errs)
    el = max(e[1] for e in errs)
    note(f"  S={S}, {w['B']} sequences x {w['Hq']} heads: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O and el <= TOL_LSE
