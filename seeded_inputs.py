"""Seeded synthetic inputs shared by the oracle-side tests and the HIP path.

This module holds no attention arithmetic: it only draws normal variates from
a seeded torch generator, scales them by a power-of-two standard deviation
(exact in fp32), casts them to the working dtype (round-to-nearest-even for
bf16) and lays them out as (batch, sequence, heads, head_dim). Both sides of
every parity check receive the same tensors from here.

Draw order for a seed: Q, then K, then V, then (decode only) the cache
lengths. The generator lives on the device the tensors are made on, so the
same seed gives different (but each time identical) values on CPU and GPU.
"""

import torch

__all__ = [
    "PREFILL_WORKLOADS",
    "DECODE_WORKLOADS",
    "prefill_inputs",
    "decode_inputs",
    "poison_cache_tail",
    "fp8_inputs",
    "random_signs",
]

# Workloads, named by what they are. "std" is the standard deviation of the
# normal draw (variance std**2).
PREFILL_WORKLOADS = {
    "mha_f32_n256_d64": dict(B=1, Hq=2, Hkv=2, Nq=256, Nk=256, d=64, dtype="f32", causal=False,
                             std_qk=1.0, std_v=1.0, seed=1),
    "mha_bf16_causal_b8_h16_n2048_d128": dict(B=8, Hq=16, Hkv=16, Nq=2048, Nk=2048, d=128, dtype="bf16",
                                              causal=True, std_qk=1.0, std_v=1.0, seed=2),
    "gqa_bf16_causal_h32kv8_n16384_d128": dict(B=1, Hq=32, Hkv=8, Nq=16384, Nk=16384, d=128, dtype="bf16",
                                               causal=True, std_qk=1.0, std_v=1.0, seed=3),
    "mha_bf16_b4_h16_n4096_d64_qkvar4": dict(B=4, Hq=16, Hkv=16, Nq=4096, Nk=4096, d=64, dtype="bf16",
                                             causal=False, std_qk=2.0, std_v=1.0, seed=5),
    "mha_bf16_b2_h8_n4096_d256_qkvar4": dict(B=2, Hq=8, Hkv=8, Nq=4096, Nk=4096, d=256, dtype="bf16",
                                             causal=False, std_qk=2.0, std_v=1.0, seed=6),
}

DECODE_WORKLOADS = {
    "gqa_bf16_decode_b64_h32kv8_cap8192_d128": dict(B=64, Hq=32, Hkv=8, capacity=8192, d=128,
                                                    len_lo=1024, len_hi=8192, seed=4),
}

_DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def _dtype(dt):
    return _DTYPES[dt] if isinstance(dt, str) else dt


def _normal(shape, std, gen, device):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def prefill_inputs(B, Hq, Hkv, Nq, Nk, d, dtype="bf16", seed=0, std_qk=1.0, std_v=1.0,
                   device="cpu", **_unused):
    """q (B, Nq, Hq, d), k and v (B, Nk, Hkv, d), contiguous, in ``dtype``."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    dt = _dtype(dtype)
    q = _normal((B, Nq, Hq, d), std_qk, gen, device).to(dt)
    k = _normal((B, Nk, Hkv, d), std_qk, gen, device).to(dt)
    v = _normal((B, Nk, Hkv, d), std_v, gen, device).to(dt)
    return q, k, v


def decode_inputs(B, Hq, Hkv, capacity, d, seed=0, len_lo=1, len_hi=None, device="cpu",
                  std_qk=1.0, std_v=1.0, **_unused):
    """q (B, 1, Hq, d), kcache and vcache (B, capacity, Hkv, d) bf16, and
    cache_seqlens (B,) int32 drawn uniformly from [len_lo, len_hi] inclusive."""
    if len_hi is None:
        len_hi = capacity
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    q = _normal((B, 1, Hq, d), std_qk, gen, device).to(torch.bfloat16)
    kc = _normal((B, capacity, Hkv, d), std_qk, gen, device).to(torch.bfloat16)
    vc = _normal((B, capacity, Hkv, d), std_v, gen, device).to(torch.bfloat16)
    lens = torch.randint(int(len_lo), int(len_hi) + 1, (B,), generator=gen, device=device,
                         dtype=torch.int64).to(torch.int32)
    return q, kc, vc, lens


def poison_cache_tail(kcache, vcache, seqlens, k_value=1.0e4, v_value=float("nan")):
    """Overwrite every cache row at or beyond seqlens[b] (in place).

    A kernel that reads past the valid length then sees keys that dominate
    the softmax, or values that turn the output into NaN.
    """
    for b, n in enumerate(seqlens.tolist()):
        kcache[b, n:] = k_value
        vcache[b, n:] = v_value
    return kcache, vcache


def _codes(shape, std, gen, device):
    # random e4m3 codes: normal draws (clipped to the format's +-448) cast by
    # torch to float8_e4m3fn, viewed as bytes
    x = _normal(shape, std, gen, device).clamp_(-448.0, 448.0)
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def fp8_inputs(B, Hq, Hkv, Nq, Nk, d, seed=0, device="cpu", code_std=64.0, exp_lo=-7, exp_hi=-6):
    """Random e4m3 operands in the layout of the FP8 forward: q8 (B, Hq, Nqp,
    d), k8 (B, Hkv, Nkp, d), vt8 (B, Hkv, d, Nkp) uint8 codes (rows past Nq /
    Nk are code 0; Nqp, Nkp = lengths rounded up to 64) and per-64-row scale
    bytes 127 + e, e uniform in [exp_lo, exp_hi] (by default values of
    standard deviation 0.5 to 1, the scale of the N(0, 1) workloads). Draw
    order: q, k, v codes, then q, k, v exponents."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    Nqp, Nkp = -(-Nq // 64) * 64, -(-Nk // 64) * 64
    q8 = torch.zeros((B, Hq, Nqp, d), dtype=torch.uint8, device=device)
    k8 = torch.zeros((B, Hkv, Nkp, d), dtype=torch.uint8, device=device)
    vt8 = torch.zeros((B, Hkv, d, Nkp), dtype=torch.uint8, device=device)
    q8[:, :, :Nq] = _codes((B, Hq, Nq, d), code_std, gen, device)
    k8[:, :, :Nk] = _codes((B, Hkv, Nk, d), code_std, gen, device)
    vt8[:, :, :, :Nk] = _codes((B, Hkv, d, Nk), code_std, gen, device)
    exps = [torch.randint(exp_lo, exp_hi + 1, (B, H, n // 64), generator=gen, device=device, dtype=torch.int32)
            for H, n in ((Hq, Nqp), (Hkv, Nkp), (Hkv, Nkp))]
    qs, ks, vs = ((e + 127).to(torch.uint8) for e in exps)
    return q8, qs, k8, ks, vt8, vs


def random_signs(d, seed=0, device="cpu"):
    """(d,) float32 of independent +-1 (the random diagonal of a rotation)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return (torch.randint(0, 2, (d,), generator=gen, device=device, dtype=torch.int32) * 2 - 1).to(torch.float32)
