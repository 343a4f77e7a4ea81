"""GPU checks of properties the exact result must have, beyond element-wise
parity with the oracle: invariants that hold at any size (constant values,
joint permutation of keys and values, reconstruction of O from the returned
LSE), limits with closed forms (large scale -> the arg-max row, two equal
scores -> the rounded mean), the causal row as attention over a prefix, and
the error of the tiled kernel against a one-pass bf16 emulation.

The attention being computed (FlashAttention: Part 2, sections 1.1 and
6.2): O_i = sum_j softmax_j(scale q_i . k_j) v_j over the visible keys,
LSE_i = ln sum_j exp(scale q_i . k_j).
"""

import math

import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import sdpa as O

pytestmark = pytest.mark.gpu

TOL_O = 2e-2
TOL_LSE = 1e-3


def fa():
    import exact_io_aware_online_amd as m
    m.lib()
    return m


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def note(msg):
    print(msg, flush=True)


def inputs(B, Hq, Hkv, Nq, Nk, d, seed, causal=False, dtype="bf16"):
    return SI.prefill_inputs(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, dtype=dtype, seed=seed,
                             device=torch.device("cuda"))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_give_that_value(d, causal):
    # every value row equal to u: any convex combination of them is u
    note(f"constant V d={d} causal={causal}")
    q, k, v = inputs(2, 4, 2, 190, 190, d, seed=61)
    u = v[0, 0, 0].clone()
    v = u.expand_as(v).contiguous()
    o, lse = fa().fa_fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    err = (o.float() - u.float()).abs().max().item()
    note(f"  max|O - u|={err:.3e}")
    assert err <= TOL_O


def test_constant_values_decode():
    dev = torch.device("cuda")
    q, kc, vc, _ = SI.decode_inputs(B=3, Hq=8, Hkv=2, capacity=300, d=128, seed=62, device=dev)
    u = vc[0, 0, 0].clone()
    vc = u.expand_as(vc).contiguous()
    lens = torch.tensor([300, 17, 129], dtype=torch.int32, device=dev)
    for S in (1, 3):
        o, _ = fa().fa_fwd_kvcache(q, kc, vc, lens, num_splits=S)
        torch.cuda.synchronize()
        err = (o.float() - u.float()).abs().max().item()
        note(f"  decode S={S} max|O - u|={err:.3e}")
        assert err <= TOL_O


@pytest.mark.parametrize("d", [64, 128])
def test_joint_key_value_permutation(d):
    # non-causal attention is a function of the set of (key, value) pairs
    note(f"permutation d={d}")
    q, k, v = inputs(1, 4, 4, 160, 333, d, seed=63)
    perm = torch.randperm(333, generator=torch.Generator().manual_seed(7)).to(q.device)
    m = fa()
    o1, l1 = m.fa_fwd(q, k, v)
    o2, l2 = m.fa_fwd(q, k[:, perm].contiguous(), v[:, perm].contiguous())
    torch.cuda.synchronize()
    eo = (o1.float() - o2.float()).abs().max().item()
    el = (l1 - l2).abs().max().item()
    note(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O and el <= TOL_LSE


@pytest.mark.parametrize("causal", [False, True])
def test_lse_reconstructs_output(causal):
    # with the returned LSE, O_i = sum_j exp(s_ij - LSE_i) v_j and the weights sum to 1
    q, k, v = inputs(1, 2, 1, 150, 200, 128, seed=64)
    scale = float(np.float32(1 / math.sqrt(128)))
    o, lse = fa().fa_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    Q, K, V = f64(q), f64(k), f64(v)
    L = f64(lse)
    worst_w = worst_o = 0.0
    for h in range(2):
        s = scale * Q[0, :, h] @ K[0, :, 0].T
        if causal:
            s = np.where(np.tril(np.ones_like(s, dtype=bool)), s, -np.inf)
        w = np.exp(s - L[0, h][:, None])
        worst_w = max(worst_w, np.max(np.abs(w.sum(axis=1) - 1.0)))
        worst_o = max(worst_o, np.max(np.abs(w @ V[0, :, 0] - f64(o)[0, :, h])))
    note(f"  max|sum w - 1|={worst_w:.3e} max|O_rec - O|={worst_o:.3e}")
    assert worst_w <= 2 * TOL_LSE
    assert worst_o <= TOL_O


def test_large_scale_selects_argmax_row():
    # as scale grows with distinct scores, softmax -> one-hot on the arg max
    note("large scale")
    q, k, v = inputs(1, 2, 2, 70, 90, 128, seed=65)
    scale = 64.0
    o, lse = fa().fa_fwd(q, k, v, scale=scale)
    torch.cuda.synchronize()
    Q, K, V = f64(q), f64(k), f64(v)
    for h in range(2):
        s = Q[0, :, h] @ K[0, :, h].T
        top2 = np.sort(s, axis=1)[:, -2:]
        rows = np.nonzero((top2[:, 1] - top2[:, 0]) * scale > 40)[0]  # runner-up weight < e^-40
        assert len(rows) >= 35, "too few rows with a clear maximum"
        am = np.argmax(s, axis=1)[rows]
        err = np.max(np.abs(f64(o)[0, rows, h] - V[0, am, h]))
        smax = scale * s.max(axis=1)[rows]
        el = np.max(np.abs(f64(lse)[0, h, rows] - smax) / np.maximum(1.0, np.abs(smax)))
        note(f"  head {h}: {len(rows)} rows, max|O - v_argmax|={err:.3e} rel|LSE - max s|={el:.3e}")
        assert err <= TOL_O
        assert el <= TOL_LSE


def test_causal_row_is_prefix_attention():
    # row i of top-left causal attention = non-causal attention over keys 0..i
    q, k, v = inputs(1, 4, 2, 300, 300, 128, seed=66)
    m = fa()
    oc, lc = m.fa_fwd(q, k, v, causal=True)
    for i in (0, 1, 31, 32, 63, 64, 127, 128, 200, 299):
        op, lp = m.fa_fwd(q[:, i:i + 1].contiguous(), k[:, :i + 1].contiguous(), v[:, :i + 1].contiguous())
        torch.cuda.synchronize()
        eo = (oc[:, i:i + 1].float() - op.float()).abs().max().item()
        el = (lc[:, :, i:i + 1] - lp).abs().max().item()
        assert eo <= TOL_O and el <= TOL_LSE, (i, eo, el)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_output_rounding_is_nearest_even(d):
    # Q = 0 and two keys: O = (v0 + v1) / 2 exactly in fp32, so the bf16
    # output must equal the round-to-nearest-even cast of that mean,
    # ties included (a mean of two bf16 values needs 9 significant bits)
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(67)
    B, H, Nq = 1, 8, 5
    v = torch.randn(B, 2, H, d, generator=g).to(torch.bfloat16)
    k = torch.randn(B, 2, H, d, generator=g).to(torch.bfloat16)
    q = torch.zeros(B, Nq, H, d, dtype=torch.bfloat16)
    o, lse = fa().fa_fwd(q.to(dev), k.to(dev), v.to(dev))
    torch.cuda.synchronize()
    mean = (v[:, 0].float() + v[:, 1].float()) / 2
    want = mean.to(torch.bfloat16)
    ties = ((mean.view(torch.int32) & 0xFFFF) == 0x8000).sum().item()
    note(f"  d={d}: {ties} exact ties among {mean.numel()} outputs")
    got = o.cpu()
    assert torch.equal(got.view(torch.int16), want[:, None].expand_as(got).contiguous().view(torch.int16))
    assert (lse.cpu() - math.log(2)).abs().max().item() <= 1e-6


def test_decode_output_rounding_is_nearest_even():
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(68)
    B, Hq, Hkv, cap, d = 2, 8, 2, 64, 128
    q = torch.zeros(B, 1, Hq, d, dtype=torch.bfloat16)
    kc = torch.randn(B, cap, Hkv, d, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, cap, Hkv, d, generator=g).to(torch.bfloat16)
    lens = torch.tensor([2, 2], dtype=torch.int32)
    o, _ = fa().fa_fwd_kvcache(q.to(dev), kc.to(dev), vc.to(dev), lens.to(dev), num_splits=1)
    torch.cuda.synchronize()
    mean = ((vc[:, 0].float() + vc[:, 1].float()) / 2).to(torch.bfloat16)  # (B, Hkv, d)
    want = mean.repeat_interleave(Hq // Hkv, dim=1)[:, None]
    assert torch.equal(o.cpu().view(torch.int16), want.contiguous().view(torch.int16))


def test_error_within_twice_a_one_pass_bf16_emulation():
    # a plain non-tiled emulation of the same precisions (fp32 scores, bf16
    # probabilities, fp32 accumulation, bf16 output) sets the error scale
    q, k, v = inputs(1, 4, 4, 256, 256, 128, seed=69)
    scale = float(np.float32(1 / math.sqrt(128)))
    o, _ = fa().fa_fwd(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    ref, _ = O.attention(f64(q), f64(k), f64(v), True, scale)
    qc, kc, vc = (t.cpu().float() for t in (q, k, v))
    s = torch.einsum("bihd,bjhd->bhij", qc, kc) * scale
    s = s.masked_fill(~torch.ones(256, 256, dtype=torch.bool).tril(), -math.inf)
    p = torch.exp(s - s.amax(-1, keepdim=True))
    emu = torch.einsum("bhij,bjhd->bihd", p.to(torch.bfloat16).float(), vc) / p.sum(-1).permute(0, 2, 1)[..., None]
    emu = emu.to(torch.bfloat16)
    e_gpu = np.max(np.abs(f64(o) - ref))
    e_emu = np.max(np.abs(f64(emu) - ref))
    note(f"  err gpu={e_gpu:.3e} err one-pass emulation={e_emu:.3e}")
    assert e_gpu <= 2 * e_emu + 1e-6
