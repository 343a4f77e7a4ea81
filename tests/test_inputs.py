"""Seeded input generator: determinism, shapes, dtypes, ranges (CPU only)."""

import torch

import seeded_inputs as SI


def test_same_seed_same_tensors():
    a = SI.prefill_inputs(B=2, Hq=4, Hkv=2, Nq=33, Nk=17, d=16, dtype="bf16", seed=7)
    b = SI.prefill_inputs(B=2, Hq=4, Hkv=2, Nq=33, Nk=17, d=16, dtype="bf16", seed=7)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    c = SI.prefill_inputs(B=2, Hq=4, Hkv=2, Nq=33, Nk=17, d=16, dtype="bf16", seed=8)
    assert not torch.equal(a[0], c[0])


def test_shapes_and_dtypes():
    q, k, v = SI.prefill_inputs(B=2, Hq=6, Hkv=3, Nq=5, Nk=9, d=8, dtype="f32", seed=1)
    assert q.shape == (2, 5, 6, 8) and k.shape == (2, 9, 3, 8) and v.shape == (2, 9, 3, 8)
    assert q.dtype == torch.float32 and q.is_contiguous()
    q, kc, vc, lens = SI.decode_inputs(B=5, Hq=8, Hkv=2, capacity=64, d=16, seed=3, len_lo=10, len_hi=64)
    assert q.shape == (5, 1, 8, 16) and kc.shape == (5, 64, 2, 16) and vc.dtype == torch.bfloat16
    assert lens.dtype == torch.int32 and int(lens.min()) >= 10 and int(lens.max()) <= 64


def test_bf16_cast_is_round_to_nearest_even():
    # the draw is fp32 then .to(bfloat16); check that cast against an
    # integer-arithmetic RNE on the fp32 bit patterns
    x = torch.randn(4096, generator=torch.Generator().manual_seed(0)) * 3
    x = torch.cat([x, torch.tensor([1.0 + 2**-8, 1.0 + 3 * 2**-8, -(1.0 + 2**-8)])])
    bits = x.view(torch.int32).to(torch.int64) & 0xFFFFFFFF
    lsb = (bits >> 16) & 1
    rne = ((bits + 0x7FFF + lsb) >> 16) & 0xFFFF
    got = x.to(torch.bfloat16).view(torch.int16).to(torch.int64) & 0xFFFF
    assert torch.equal(got, rne)


def test_std_scaling_is_exact():
    q1, _, _ = SI.prefill_inputs(B=1, Hq=1, Hkv=1, Nq=64, Nk=1, d=8, dtype="f32", seed=4, std_qk=1.0)
    q2, _, _ = SI.prefill_inputs(B=1, Hq=1, Hkv=1, Nq=64, Nk=1, d=8, dtype="f32", seed=4, std_qk=2.0)
    assert torch.equal(q1 * 2, q2)


def test_poison_tail():
    q, kc, vc, lens = SI.decode_inputs(B=3, Hq=2, Hkv=1, capacity=8, d=4, seed=2, len_lo=1, len_hi=8)
    SI.poison_cache_tail(kc, vc, lens)
    for b, n in enumerate(lens.tolist()):
        assert torch.all(kc[b, n:] == 1.0e4)
        assert torch.all(torch.isnan(vc[b, n:]).logical_or(torch.tensor(n == 8)))
        assert not torch.any(torch.isnan(vc[b, :n]))


def test_workload_tables_are_consistent():
    for name, w in SI.PREFILL_WORKLOADS.items():
        assert w["Hq"] % w["Hkv"] == 0, name
    for name, w in SI.DECODE_WORKLOADS.items():
        assert w["Hq"] % w["Hkv"] == 0 and w["len_hi"] <= w["capacity"], name
