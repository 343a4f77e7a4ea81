"""Parity with tensors of more than 2^31 elements (over 4 GiB in bf16).

Every kernel forms its global addresses as a 64-bit base per (sequence,
head) plus a 32-bit offset inside a tile; these cases put rows of q, k, v,
o, the gradients and the KV cache past 2^31 elements (and 2^32 bytes) so
that a 32-bit product anywhere on that path would read or write the wrong
rows. The oracle is taken for the (batch, head) slices and sequences at the
far end of each tensor plus a few others; bars as everywhere (O 2e-2, LSE
1e-3; gradients 2e-2 x max(1, max|ref|)).
"""

import math

import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import sdpa as O

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 2e-2, 1e-3
ELEMS_32 = 2 ** 31

# causal MHA, 130 x 2048 x 64 x 128 = 2.18e9 elements in each of q, k, v, o
BIG_PREFILL = dict(B=130, Hq=64, Hkv=64, Nq=2048, Nk=2048, d=128, causal=True)
# GQA decode over a 64 x 36864 x 8 x 128 = 2.42e9-element cache per K and V
BIG_DECODE = dict(B=64, Hq=32, Hkv=8, capacity=36864, d=128)


def fa():
    import exact_io_aware_online_amd as m
    m.lib()
    return m


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def note(msg):
    print(msg, flush=True)


def gtol(ref):
    return 2e-2 * max(1.0, float(np.max(np.abs(ref))) if ref.size else 1.0)


def release():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_prefill_and_backward_past_2_31_elements():
    w = BIG_PREFILL
    B, H, N, d = w["B"], w["Hq"], w["Nq"], w["d"]
    assert B * N * H * d > ELEMS_32 and (B - 2) * N * H * d >= ELEMS_32
    note(f"prefill + backward, {B}x{N}x{H}x{d} per tensor ({B * N * H * d / 2**31:.3f} x 2^31 elements)")
    dev = torch.device("cuda")
    m = fa()
    q, k, v = SI.prefill_inputs(device=dev, seed=41, **w)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = m.fa_fwd(q, k, v, causal=True, scale=scale)
    do = torch.randn(q.shape, generator=torch.Generator(device=dev).manual_seed(42), device=dev).to(torch.bfloat16)
    dq, dk, dv = m.fa_bwd(q, k, v, o, lse, do, causal=True, scale=scale)
    torch.cuda.synchronize()
    # the last two batches lie wholly past element 2^31
    heads = [(B - 1, H - 1), (B - 1, 0), (B - 2, 17), (B // 2, H // 2), (0, 0)]
    for b, h in heads:
        qs, ks, vs, ds = (f64(t[b:b + 1, :, h:h + 1]) for t in (q, k, v, do))
        o_ref, l_ref = O.attention_rows(qs, ks, vs, True, scale, 0, 0)
        eo = float(np.max(np.abs(f64(o[b, :, h]) - o_ref)))
        el = float(np.max(np.abs(f64(lse[b, h]) - l_ref)))
        gq, gk, gv = O.attention_backward_rows(qs, ks, vs, ds, True, scale, 0, 0)
        errs = {n: float(np.max(np.abs(f64(t[b, :, h]) - r))) for n, t, r in
                (("dq", dq, gq), ("dk", dk, gk), ("dv", dv, gv))}
        note(f"  b={b} h={h}: max|dO|={eo:.3e} max|dLSE|={el:.3e} " +
             " ".join(f"max|{n}|={e:.3e}" for n, e in errs.items()))
        assert eo <= TOL_O and el <= TOL_LSE, (b, h, eo, el)
        for n, r in (("dq", gq), ("dk", gk), ("dv", gv)):
            assert errs[n] <= gtol(r), (n, b, h, errs[n])
    del q, k, v, o, lse, do, dq, dk, dv
    release()


def _decode_check(o, lse, q, seq_cache, lens, scale, seqs):
    worst = (0.0, 0.0)
    for b in seqs:
        n = int(lens[b])
        kb, vb = seq_cache(b, n)
        o_ref, l_ref = O.decode(f64(q[b:b + 1]), kb, vb, [n], scale)
        eo = float(np.max(np.abs(f64(o[b, 0]) - o_ref[0])))
        el = float(np.max(np.abs(f64(lse[b]) - l_ref[0])))
        assert eo <= TOL_O and el <= TOL_LSE, (b, n, eo, el)
        worst = (max(worst[0], eo), max(worst[1], el))
    return worst


@pytest.mark.timeout(600)
def test_decode_contiguous_and_paged_past_2_31_elements():
    w = BIG_DECODE
    B, Hq, Hkv, cap, d = w["B"], w["Hq"], w["Hkv"], w["capacity"], w["d"]
    assert B * cap * Hkv * d > ELEMS_32
    note(f"decode over a {B}x{cap}x{Hkv}x{d} cache ({B * cap * Hkv * d / 2**31:.3f} x 2^31 elements)")
    dev = torch.device("cuda")
    m = fa()
    q, kc, vc, lens = SI.decode_inputs(B, Hq, Hkv, cap, d, seed=43, len_lo=1, device=dev)
    lens[-1] = cap  # the last sequence reaches the end of the cache
    lens[-2] = cap - 1
    lh = lens.cpu().numpy()
    scale = float(np.float32(1.0 / math.sqrt(d)))
    seqs = [B - 1, B - 2, B // 2, 0]

    S = m.fa_kvcache_default_splits(B, Hkv, cap, d)
    for splits in sorted({S, 1, 8}):
        o, lse = m.fa_fwd_kvcache(q, kc, vc, lens, num_splits=splits, scale=scale)
        torch.cuda.synchronize()
        eo, el = _decode_check(o, lse, q, lambda b, n: (f64(kc[b:b + 1, :n]), f64(vc[b:b + 1, :n])), lh, scale, seqs)
        note(f"  contiguous, S={splits}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")

    # the same buffers as a pool of 256-row pages, every sequence's pages
    # scattered over the whole pool
    page = 256
    pps = cap // page
    kp = kc.view(B * pps, page, Hkv, d)
    vp = vc.view(B * pps, page, Hkv, d)
    perm = torch.randperm(B * pps, generator=torch.Generator().manual_seed(44)).to(torch.int32)
    bt = perm.view(B, pps).to(dev)
    assert int(bt[B - 1].max()) >= (B * pps * 15) // 16  # far pages in use

    def paged_seq(b, n):
        rows = bt[b].long()
        return (f64(kp[rows].reshape(1, pps * page, Hkv, d)[:, :n]),
                f64(vp[rows].reshape(1, pps * page, Hkv, d)[:, :n]))
    o, lse = m.fa_fwd_kvcache_paged(q, kp, vp, bt, lens, num_splits=S, scale=scale)
    torch.cuda.synchronize()
    eo, el = _decode_check(o, lse, q, paged_seq, lh, scale, seqs)
    note(f"  paged (256-row pages), S={S}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    del q, kc, vc, lens, kp, vp, bt, o, lse
    release()


@pytest.mark.timeout(600)
def test_fp8_forward_past_2_31_bytes():
    # The e4m3 codes of q, k and v^T cross 2^31 bytes. Each sampled (batch,
    # head) slice is quantised and attended again as a tensor of its own: the
    # arithmetic of an element does not depend on where its head sits, so
    # codes, scales, O and LSE must match bit for bit (the small path is
    # checked against the FP8 oracle elsewhere).
    w = BIG_PREFILL
    B, H, N, d = w["B"], w["Hq"], w["Nq"], w["d"]
    note(f"FP8 forward, {B}x{N}x{H}x{d} codes per tensor ({B * N * H * d / 2**31:.3f} x 2^31 bytes)")
    dev = torch.device("cuda")
    m = fa()
    q, k, v = SI.prefill_inputs(device=dev, seed=45, **w)
    signs = SI.random_signs(d, seed=46, device=dev)
    scale = float(np.float32(1.0 / math.sqrt(d)))

    def fp8(qq, kk, vv):
        q8, qs = m.fa_quantize_fp8(qq, signs)
        k8, ks = m.fa_quantize_fp8(kk, signs)
        v8, vs = m.fa_quantize_fp8(vv, transpose=True)
        o, lse = m.fa_fwd_fp8(q8, qs, k8, ks, v8, vs, qq.shape[1], kk.shape[1], causal=True, scale=scale)
        return (q8, qs, k8, ks, v8, vs), o, lse
    codes, o, lse = fp8(q, k, v)
    torch.cuda.synchronize()
    assert codes[0].numel() > ELEMS_32
    for b, h in [(B - 1, H - 1), (B - 2, 17), (B // 2, H // 2), (0, 0)]:
        sl = [t[b:b + 1, :, h:h + 1].contiguous() for t in (q, k, v)]
        c1, o1, l1 = fp8(*sl)
        torch.cuda.synchronize()
        for name, big, small in zip(("q8", "q_scales", "k8", "k_scales", "vt8", "v_scales"), codes, c1):
            assert torch.equal(big[b:b + 1, h:h + 1], small), (name, b, h)
        assert torch.equal(o[b:b + 1, :, h:h + 1].view(torch.int16), o1.view(torch.int16)), ("O", b, h)
        assert torch.equal(lse[b:b + 1, h:h + 1], l1), ("LSE", b, h)
        note(f"  b={b} h={h}: codes, scales, O and LSE equal to the slice run")
    del q, k, v, codes, o, lse
    release()
