"""Pins that tie the oracle to something other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
an independent source: a pure-Python brute force on tiny inputs (math.fsum,
math.exp), a library routine (scipy.special, PyTorch CPU float64
scaled_dot_product_attention), a closed form, or an invariant the
definition implies. ``tests/test_oracle.py`` runs them against the real
oracle; ``tests/test_oracle_mutations.py`` plants plausible mistakes in the
oracle and checks that some pin fails for each.

Functions are looked up on ``oracle.sdpa`` at call time so a planted mistake
in any helper reaches every caller.
"""

import json
import math
import os

import numpy as np

from oracle import fp8 as F8
from oracle import sdpa as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# independent pure-Python brute force (no numpy arithmetic)
# ---------------------------------------------------------------------------
def brute_attention(q, k, v, causal, scale):
    """Triple loop over (batch, query head, query); exact sums via math.fsum."""
    q = np.asarray(q, dtype=np.float64).tolist()
    k = np.asarray(k, dtype=np.float64).tolist()
    v = np.asarray(v, dtype=np.float64).tolist()
    B, Nq, Hq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Nk, Hkv, dv = len(k[0]), len(k[0][0]), len(v[0][0][0])
    out = np.zeros((B, Nq, Hq, dv))
    lse = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            g = (h * Hkv) // Hq
            for i in range(Nq):
                keys = [j for j in range(Nk) if (not causal) or j <= i]
                if not keys:
                    lse[b, h, i] = -math.inf
                    continue
                s = [scale * math.fsum(q[b][i][h][t] * k[b][j][g][t] for t in range(d)) for j in keys]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                den = math.fsum(e)
                lse[b, h, i] = mx + math.log(den)
                for t in range(dv):
                    out[b, i, h, t] = math.fsum(e[n] * v[b][j][g][t] for n, j in enumerate(keys)) / den
    return out, lse


def rng_case(seed, B, Nq, Nk, Hq, Hkv, d, std=1.0):
    r = np.random.default_rng(seed)
    q = r.normal(0.0, std, (B, Nq, Hq, d))
    k = r.normal(0.0, std, (B, Nk, Hkv, d))
    v = r.normal(0.0, 1.0, (B, Nk, Hkv, d))
    return q, k, v


TINY_SHAPES = [
    # (B, Nq, Nk, Hq, Hkv, d)
    (1, 5, 5, 1, 1, 3),
    (2, 4, 7, 2, 2, 4),
    (1, 8, 8, 4, 2, 2),
    (2, 3, 6, 6, 3, 3),
    (1, 7, 3, 4, 1, 4),
    (1, 6, 6, 2, 1, 1),
]


def pin_brute_force(tol=1e-12):
    for n, (B, Nq, Nk, Hq, Hkv, d) in enumerate(TINY_SHAPES):
        for causal in (False, True):
            q, k, v = rng_case(100 + n, B, Nq, Nk, Hq, Hkv, d, std=1.5)
            scale = 1.0 / math.sqrt(d) * 1.3
            o_ref, l_ref = brute_attention(q, k, v, causal, scale)
            o, l = O.attention(q, k, v, causal, scale)
            assert np.max(np.abs(o - o_ref)) <= tol, ("O vs brute force", causal, (B, Nq, Nk, Hq, Hkv, d))
            assert np.max(np.abs(l - l_ref)) <= tol, ("LSE vs brute force", causal, (B, Nq, Nk, Hq, Hkv, d))


def pin_torch_sdpa(tol=1e-12):
    """PyTorch CPU float64 scaled_dot_product_attention (is_causal is top-left,
    enable_gqa repeats each KV head over a contiguous block of query heads)."""
    import torch
    import torch.nn.functional as F
    for n, (B, Nq, Nk, Hq, Hkv, d) in enumerate([(2, 9, 9, 4, 2, 8), (1, 16, 16, 8, 2, 16),
                                                 (1, 5, 12, 3, 3, 4), (2, 12, 12, 2, 1, 5)]):
        for causal in (False, True):
            q, k, v = rng_case(200 + n, B, Nq, Nk, Hq, Hkv, d)
            scale = 0.37
            o, _ = O.attention(q, k, v, causal, scale)
            tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))) for x in (q, k, v))
            ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale,
                                                 enable_gqa=(Hq != Hkv))
            ref = ref.numpy().transpose(0, 2, 1, 3)
            assert np.max(np.abs(o - ref)) <= tol, ("O vs torch SDPA", causal, (B, Nq, Nk, Hq, Hkv, d))


def pin_scipy_rows(tol=1e-12):
    from scipy.special import logsumexp, softmax
    q, k, v = rng_case(300, 1, 10, 13, 1, 1, 6, std=3.0)
    scale = 0.8
    S = scale * np.einsum("id,jd->ij", q[0, :, 0], k[0, :, 0])
    o, l = O.attention(q, k, v, False, scale)
    assert np.max(np.abs(l[0, 0] - logsumexp(S, axis=1))) <= tol, "LSE vs scipy logsumexp"
    assert np.max(np.abs(o[0, :, 0] - softmax(S, axis=1) @ v[0, :, 0])) <= tol, "O vs scipy softmax"


def pin_golden_closed_forms(tol=1e-13):
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        fixtures = json.load(f)["fixtures"]
    env = {"e": math.e, "log": math.log, "exp": math.exp, "tanh": math.tanh}
    for fx in fixtures:
        q, k, v = (np.array(fx[n], dtype=np.float64) for n in ("q", "k", "v"))
        o, l = O.attention(q, k, v, fx["causal"], fx["scale"])
        for ent in fx["o"]:
            want = eval(ent["expr"], {"__builtins__": {}}, env)  # noqa: S307 - fixed local expressions
            assert abs(want - ent["value"]) <= 1e-15 * max(1.0, abs(want)), ("fixture typo", fx["name"])
            assert abs(o[tuple(ent["index"])] - want) <= tol, ("golden O", fx["name"], ent["index"])
        for ent in fx["lse"]:
            want = eval(ent["expr"], {"__builtins__": {}}, env)  # noqa: S307
            assert abs(want - ent["value"]) <= 1e-15 * max(1.0, abs(want)), ("fixture typo", fx["name"])
            assert abs(l[tuple(ent["index"])] - want) <= tol, ("golden LSE", fx["name"], ent["index"])


def pin_row_stochastic(tol=1e-12):
    q, k, _ = rng_case(400, 1, 12, 12, 1, 1, 5, std=2.0)
    for causal in (False, True):
        S = O.scores(q[0, :, 0], k[0, :, 0], 0.7)
        P, _ = O.softmax_rows(S, O.visible_mask(12, 12, causal))
        assert np.all(P >= 0.0), "P negative"
        assert np.max(np.abs(P.sum(axis=1) - 1.0)) <= tol, "rows of P do not sum to 1"
        if causal:
            assert np.all(P[np.triu_indices(12, 1)] == 0.0), "causal P leaks future keys"


def pin_constant_values(tol=1e-12):
    q, k, v = rng_case(500, 2, 9, 9, 4, 2, 3, std=2.0)
    c = np.array([1.25, -3.0, 0.5])
    v[:] = c
    for causal in (False, True):
        o, _ = O.attention(q, k, v, causal, 0.9)
        assert np.max(np.abs(o - c)) <= tol, "constant V not reproduced"


def pin_key_permutation(tol=1e-12):
    q, k, v = rng_case(600, 1, 6, 11, 2, 1, 4)
    perm = np.random.default_rng(601).permutation(11)
    o1, l1 = O.attention(q, k, v, False, 0.6)
    o2, l2 = O.attention(q, k[:, perm], v[:, perm], False, 0.6)
    assert np.max(np.abs(o1 - o2)) <= tol and np.max(np.abs(l1 - l2)) <= tol, "not key-permutation equivariant"


def pin_zero_query_closed_form(tol=1e-12):
    _, k, v = rng_case(700, 1, 7, 7, 2, 2, 3)
    q = np.zeros((1, 7, 2, 3))
    for causal in (False, True):
        o, l = O.attention(q, k, v, causal, 1.0)
        for i in range(7):
            n = i + 1 if causal else 7
            assert np.max(np.abs(o[0, i] - v[0, :n].mean(axis=0))) <= tol, ("q=0 mean", causal, i)
            assert np.max(np.abs(l[0, :, i] - math.log(n))) <= tol, ("q=0 LSE", causal, i)


def pin_single_key(tol=1e-12):
    q, k, v = rng_case(800, 2, 4, 1, 2, 1, 5)
    for causal in (False, True):
        o, l = O.attention(q, k, v, causal, 0.45)
        for h in range(2):
            assert np.max(np.abs(o[:, :, h] - v[:, 0:1, 0])) <= tol, "Nk=1: O != v0"
            s = 0.45 * np.einsum("bnd,bd->bn", q[:, :, h], k[:, 0, 0])
            assert np.max(np.abs(l[:, h] - s)) <= tol, "Nk=1: LSE != s00"


def pin_large_scale_argmax(tol=1e-9):
    q, k, v = rng_case(900, 1, 5, 8, 1, 1, 4)
    o, _ = O.attention(q, k, v, False, 1.0e4)
    S = q[0, :, 0] @ k[0, :, 0].T
    assert np.max(np.abs(o[0, :, 0] - v[0, S.argmax(axis=1), 0])) <= tol, "hard-max limit"


def pin_causal_prefix(tol=1e-12):
    q, k, v = rng_case(1000, 1, 8, 8, 2, 2, 3)
    oc, lc = O.attention(q, k, v, True, 0.5)
    for i in range(8):
        on, ln = O.attention(q[:, i:i + 1], k[:, :i + 1], v[:, :i + 1], False, 0.5)
        assert np.max(np.abs(oc[:, i:i + 1] - on)) <= tol and np.max(np.abs(lc[:, :, i:i + 1] - ln)) <= tol, (
            "causal row i != full attention over keys 0..i", i)


def pin_gqa_repeat(tol=1e-15):
    q, k, v = rng_case(1100, 2, 6, 6, 6, 2, 3)
    for causal in (False, True):
        o1, l1 = O.attention(q, k, v, causal, 0.7)
        o2, l2 = O.attention(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), causal, 0.7)
        assert np.max(np.abs(o1 - o2)) <= tol and np.max(np.abs(l1 - l2)) <= tol, "GQA != repeat-interleaved MHA"


def pin_split_combine(tol=1e-12):
    """Parts over disjoint key sets, each from the brute force, merge to the full result."""
    q, k, v = rng_case(1200, 1, 5, 13, 2, 1, 4)
    o_full, l_full = brute_attention(q, k, v, False, 0.8)
    cuts = [0, 4, 4, 9, 13]  # includes an empty part
    parts_o, parts_l = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        if b > a:
            po, pl = brute_attention(q, k[:, a:b], v[:, a:b], False, 0.8)
        else:
            po, pl = np.zeros_like(o_full), np.full_like(l_full, -np.inf)
        parts_o.append(po)
        parts_l.append(pl.transpose(0, 2, 1))  # (B, Nq, Hq) to match O's leading dims
    o, l = O.merge_partials(np.stack(parts_o), np.stack(parts_l))
    assert np.max(np.abs(o - o_full)) <= tol, "merged O != full"
    assert np.max(np.abs(l - l_full.transpose(0, 2, 1))) <= tol, "merged LSE != full"
    o0, l0 = O.merge_partials(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.all(o0 == 0.0) and np.all(l0 == -np.inf), "all-empty merge"


def pin_decode(tol=1e-12):
    r = np.random.default_rng(1300)
    B, cap, Hq, Hkv, d = 3, 9, 4, 2, 5
    q = r.normal(size=(B, 1, Hq, d))
    kc = r.normal(size=(B, cap, Hkv, d))
    vc = r.normal(size=(B, cap, Hkv, d))
    lens = [1, 9, 4]
    o, l = O.decode(q, kc, vc, lens, 0.45)
    for b, n in enumerate(lens):
        ob, lb = brute_attention(q[b:b + 1], kc[b:b + 1, :n], vc[b:b + 1, :n], False, 0.45)
        assert np.max(np.abs(o[b] - ob[0, 0])) <= tol, ("decode O", b)
        assert np.max(np.abs(l[b] - lb[0, :, 0])) <= tol, ("decode LSE", b)


def pin_decode_paged(tol=1e-12):
    """Pages gathered by hand (plain loops) give the brute-force decode."""
    r = np.random.default_rng(1350)
    B, P, pps, Hq, Hkv, d = 2, 3, 3, 4, 2, 5
    num_pages = 8
    q = r.normal(size=(B, 1, Hq, d))
    kp = r.normal(size=(num_pages, P, Hkv, d))
    vp = r.normal(size=(num_pages, P, Hkv, d))
    bt = np.array([[5, 0, 7], [2, 6, 1]])
    lens = [7, 4]
    o, l = O.decode_paged(q, kp, vp, bt, lens, 0.55)
    for b, n in enumerate(lens):
        rows_k = [kp[bt[b][i // P]][i % P] for i in range(n)]
        rows_v = [vp[bt[b][i // P]][i % P] for i in range(n)]
        kc = np.array(rows_k)[None]
        vc = np.array(rows_v)[None]
        ob, lb = brute_attention(q[b:b + 1], kc, vc, False, 0.55)
        assert np.max(np.abs(o[b] - ob[0, 0])) <= tol, ("paged O", b)
        assert np.max(np.abs(l[b] - lb[0, :, 0])) <= tol, ("paged LSE", b)


def pin_online_recurrence(tol=1e-12):
    """The tiled (m, l, a) recurrence reaches the brute-force result."""
    q, k, v = rng_case(1400, 1, 11, 11, 1, 1, 4, std=3.0)
    for causal in (False, True):
        ob, lb = brute_attention(q, k, v, causal, 0.9)
        for bq, bk in ((4, 3), (11, 11), (1, 5)):
            o, l = O.online_softmax_attention(q[0, :, 0], k[0, :, 0], v[0, :, 0], causal, 0.9, bq, bk)
            assert np.max(np.abs(o - ob[0, :, 0])) <= tol, ("recurrence O", causal, bq, bk)
            assert np.max(np.abs(l - lb[0, 0])) <= tol, ("recurrence LSE", causal, bq, bk)


# ---------------------------------------------------------------------------
# backward pass
# ---------------------------------------------------------------------------
def _bwd_case(seed, B, Nq, Nk, Hq, Hkv, d):
    q, k, v = rng_case(seed, B, Nq, Nk, Hq, Hkv, d)
    do = np.random.default_rng(seed + 1).normal(size=q.shape[:3] + (v.shape[3],))
    return q, k, v, do


def pin_backward_torch_autograd(tol=1e-12):
    """PyTorch CPU float64 autograd through scaled_dot_product_attention."""
    import torch

    q, k, v, do = _bwd_case(1500, 2, 7, 9, 4, 2, 5)
    for causal in (False, True):
        dq, dk, dv = O.attention_backward(q, k, v, do, causal, 0.6)
        Q, K, V = (torch.tensor(x).permute(0, 2, 1, 3).requires_grad_() for x in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=causal, scale=0.6,
                                                             enable_gqa=True)
        o.backward(torch.tensor(do).permute(0, 2, 1, 3))
        for mine, ref, n in ((dq, Q.grad, "dq"), (dk, K.grad, "dk"), (dv, V.grad, "dv")):
            assert np.max(np.abs(mine - ref.permute(0, 2, 1, 3).numpy())) <= tol, (n, causal)


def pin_backward_finite_differences(tol=2e-7):
    """Central differences of sum(O * dO) through the forward oracle."""
    q, k, v, do = _bwd_case(1600, 1, 4, 5, 2, 1, 3)
    h = 1e-5
    for causal in (False, True):
        grads = O.attention_backward(q, k, v, do, causal, 0.9)
        for which, x in enumerate((q, k, v)):
            for idx in [(0, 0, 0, 0), (0, 2, 0, 1), (0, 3, x.shape[2] - 1, 2)]:
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = [q, k, v]
                args_m = [q, k, v]
                args_p[which], args_m[which] = xp, xm
                fp = np.sum(O.attention(*args_p, causal, 0.9)[0] * do)
                fm = np.sum(O.attention(*args_m, causal, 0.9)[0] * do)
                fd = (fp - fm) / (2 * h)
                assert abs(fd - grads[which][idx]) <= tol, ("finite difference", which, idx, causal)


def pin_backward_constant_values(tol=1e-13):
    """Constant value rows make O independent of Q and K: dQ = dK = 0."""
    q, k, v, do = _bwd_case(1700, 1, 6, 6, 2, 2, 4)
    v[:] = v[:, :1]
    for causal in (False, True):
        dq, dk, dv = O.attention_backward(q, k, v, do, causal, 1.1)
        assert np.max(np.abs(dq)) <= tol and np.max(np.abs(dk)) <= tol, ("constant V", causal)
        # every query's weights sum to one, so the value gradients sum to dO
        assert np.max(np.abs(dv.sum(axis=1) - do.reshape(1, 6, 2, 1, 4).sum(axis=(1, 3)))) <= 1e-12


def pin_backward_gqa_sum(tol=1e-13):
    """A grouped head's gradients are the sums over its repeated MHA heads."""
    q, k, v, do = _bwd_case(1800, 1, 5, 5, 6, 2, 3)
    for causal in (False, True):
        dq, dk, dv = O.attention_backward(q, k, v, do, causal, 0.5)
        dq2, dk2, dv2 = O.attention_backward(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), do, causal, 0.5)
        assert np.max(np.abs(dq - dq2)) <= tol, "GQA dq"
        assert np.max(np.abs(dk - dk2.reshape(1, 5, 2, 3, 3).sum(axis=3))) <= tol, "GQA dk"
        assert np.max(np.abs(dv - dv2.reshape(1, 5, 2, 3, 3).sum(axis=3))) <= tol, "GQA dv"


# ---------------------------------------------------------------------------
# local windows, bottom-right alignment, variable-length packing
# ---------------------------------------------------------------------------
def brute_window(q, k, v, wl, wr, scale):
    """Plain loops: key j visible to query i iff i+off-wl <= j <= i+off+wr."""
    q = np.asarray(q, dtype=np.float64).tolist()
    k = np.asarray(k, dtype=np.float64).tolist()
    v = np.asarray(v, dtype=np.float64).tolist()
    B, Nq, Hq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Nk, Hkv, dv = len(k[0]), len(k[0][0]), len(v[0][0][0])
    off = Nk - Nq
    out = np.zeros((B, Nq, Hq, dv))
    lse = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            g = (h * Hkv) // Hq
            for i in range(Nq):
                keys = [j for j in range(Nk) if (wl < 0 or j >= i + off - wl) and (wr < 0 or j <= i + off + wr)]
                if not keys:
                    lse[b, h, i] = -math.inf
                    continue
                s = [scale * math.fsum(q[b][i][h][t] * k[b][j][g][t] for t in range(d)) for j in keys]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                den = math.fsum(e)
                lse[b, h, i] = mx + math.log(den)
                for t in range(dv):
                    out[b, i, h, t] = math.fsum(e[n] * v[b][j][g][t] for n, j in enumerate(keys)) / den
    return out, lse


def pin_window_brute_force(tol=1e-12):
    for (Nq, Nk, wl, wr) in ((5, 9, 2, 0), (9, 5, -1, 0), (7, 7, 1, 2), (6, 6, -1, -1), (4, 8, 0, -1), (8, 3, 3, 1)):
        q, k, v = rng_case(1900 + Nq * 10 + Nk, 1, Nq, Nk, 4, 2, 3, std=1.5)
        o, l = O.attention_window(q, k, v, wl, wr, 0.6)
        ob, lb = brute_window(q, k, v, wl, wr, 0.6)
        fin = np.isfinite(lb)
        assert np.max(np.abs(o - ob)) <= tol, ("window O", Nq, Nk, wl, wr)
        assert np.array_equal(fin, np.isfinite(l)) and np.max(np.abs(l[fin] - lb[fin]), initial=0.0) <= tol


def pin_window_torch_mask(tol=1e-12):
    """PyTorch float64 SDPA with the window as an explicit boolean mask."""
    import torch

    q, k, v = rng_case(2000, 2, 6, 10, 4, 4, 5)
    for wl, wr in ((3, 0), (-1, 0), (2, 2)):
        o, _ = O.attention_window(q, k, v, wl, wr, 0.45)
        i = torch.arange(6)[:, None] + 4
        j = torch.arange(10)[None, :]
        m = torch.ones(6, 10, dtype=torch.bool)
        if wl >= 0:
            m &= j >= i - wl
        if wr >= 0:
            m &= j <= i + wr
        ref = torch.nn.functional.scaled_dot_product_attention(
            *(torch.tensor(x).permute(0, 2, 1, 3) for x in (q, k, v)), attn_mask=m, scale=0.45)
        assert np.max(np.abs(o - ref.permute(0, 2, 1, 3).numpy())) <= tol, ("torch mask", wl, wr)


def pin_window_special_cases(tol=0.0):
    """No window = non-causal; (-1, 0) on square inputs = top-left causal."""
    q, k, v = rng_case(2100, 1, 7, 7, 2, 1, 4)
    o1, l1 = O.attention_window(q, k, v, -1, -1, 0.8)
    o2, l2 = O.attention(q, k, v, False, 0.8)
    assert np.max(np.abs(o1 - o2)) <= tol and np.max(np.abs(l1 - l2)) <= tol, "no window"
    o1, l1 = O.attention_window(q, k, v, -1, 0, 0.8)
    o2, l2 = O.attention(q, k, v, True, 0.8)
    assert np.max(np.abs(o1 - o2)) <= tol and np.max(np.abs(l1 - l2)) <= tol, "square causal"


def pin_varlen_concatenation(tol=0.0):
    """A packed batch is its sequences' results laid end to end."""
    r = np.random.default_rng(2200)
    lq, lk = [3, 0, 5, 2], [4, 2, 5, 6]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q = r.normal(size=(cu_q[-1], 4, 3))
    k = r.normal(size=(cu_k[-1], 2, 3))
    v = r.normal(size=(cu_k[-1], 2, 3))
    for wl, wr in ((-1, -1), (-1, 0), (1, 1)):
        o, l = O.attention_varlen(q, k, v, cu_q, cu_k, wl, wr, 0.7)
        for b in range(4):
            if lq[b] == 0:
                continue
            ob, lb = brute_window(q[None, cu_q[b]:cu_q[b + 1]], k[None, cu_k[b]:cu_k[b + 1]],
                                  v[None, cu_k[b]:cu_k[b + 1]], wl, wr, 0.7)
            assert np.max(np.abs(o[cu_q[b]:cu_q[b + 1]] - ob[0])) <= 1e-12, ("varlen O", b, wl, wr)
            fin = np.isfinite(lb[0])
            lv = l[:, cu_q[b]:cu_q[b + 1]]
            assert np.array_equal(np.isfinite(lv), fin)
            assert np.max(np.abs(lv[fin] - lb[0][fin]), initial=0.0) <= 1e-12, ("varlen LSE", b)


# ---------------------------------------------------------------------------
# decode step with in-place cache append
# ---------------------------------------------------------------------------
def _append_case(seed, B, cap, Nq, Hq, Hkv, d):
    r = np.random.default_rng(seed)
    return (r.normal(size=(B, Nq, Hq, d)), r.normal(size=(B, cap, Hkv, d)), r.normal(size=(B, cap, Hkv, d)),
            r.normal(size=(B, Nq, Hkv, d)), r.normal(size=(B, Nq, Hkv, d)))


def pin_decode_append_brute_force(tol=1e-12):
    """Cache rows gathered by hand, then the new rows, attended by the
    bottom-right brute force (plain loops)."""
    B, cap, Nq, Hq, Hkv, d = 3, 9, 3, 4, 2, 3
    q, kc, vc, kn, vn = _append_case(2300, B, cap, Nq, Hq, Hkv, d)
    lens = [2, 0, 6]
    for append in (True, False):
        for causal in (True, False):
            k2, v2, o, l = O.decode_append(q, kc, vc, lens, kn if append else None, vn if append else None,
                                           causal, 0.6)
            for b in range(B):
                rows_k = [kc[b, j] for j in range(lens[b])] + ([kn[b, i] for i in range(Nq)] if append else [])
                rows_v = [vc[b, j] for j in range(lens[b])] + ([vn[b, i] for i in range(Nq)] if append else [])
                if not rows_k:  # nothing to attend: O = 0, LSE = -inf
                    assert not np.any(o[b]) and np.all(l[b] == -np.inf), ("empty cache", append, causal, b)
                    continue
                ob, lb = brute_window(q[b:b + 1], np.array(rows_k)[None], np.array(rows_v)[None], -1,
                                      0 if causal else -1, 0.6)
                assert np.max(np.abs(o[b] - ob[0])) <= tol, ("append O", append, causal, b)
                fin = np.isfinite(lb[0])
                assert np.array_equal(np.isfinite(l[b]), fin), ("rows without keys", append, causal, b)
                assert np.max(np.abs(l[b][fin] - lb[0][fin]), initial=0.0) <= tol, ("append LSE", b)


def pin_decode_append_cache_update(tol=0.0):
    """New rows land at [len, len + Nq); every other row, and the inputs,
    stay as they were; rows at or past capacity are dropped."""
    B, cap, Nq, Hq, Hkv, d = 3, 6, 3, 2, 1, 2
    q, kc, vc, kn, vn = _append_case(2310, B, cap, Nq, Hq, Hkv, d)
    kc0, vc0 = kc.copy(), vc.copy()
    lens = [1, 4, 6]
    k2, v2, _, _ = O.decode_append(q, kc, vc, lens, kn, vn, True, 1.0)
    assert np.array_equal(kc, kc0) and np.array_equal(vc, vc0), "inputs modified"
    for b in range(B):
        for j in range(cap):
            i = j - lens[b]
            want_k = kn[b, i] if 0 <= i < Nq else kc0[b, j]
            want_v = vn[b, i] if 0 <= i < Nq else vc0[b, j]
            assert np.array_equal(k2[b, j], want_k) and np.array_equal(v2[b, j], want_v), ("cache row", b, j)


def pin_decode_append_reduces_to_decode(tol=1e-12):
    """One query: without new rows this is the plain decode; with one new
    row it is the plain decode of the grown cache at length + 1."""
    B, cap, Hq, Hkv, d = 2, 8, 4, 2, 3
    q, kc, vc, kn, vn = _append_case(2320, B, cap, 1, Hq, Hkv, d)
    lens = [5, 7]
    _, _, o, l = O.decode_append(q, kc, vc, lens, None, None, True, 0.8)
    od, ld = O.decode(q, kc, vc, lens, 0.8)
    assert np.max(np.abs(o[:, 0] - od)) <= tol and np.max(np.abs(l[:, :, 0] - ld)) <= tol
    k2, v2, o, l = O.decode_append(q, kc, vc, lens, kn, vn, True, 0.8)
    od, ld = O.decode(q, k2, v2, [n + 1 for n in lens], 0.8)
    assert np.max(np.abs(o[:, 0] - od)) <= tol and np.max(np.abs(l[:, :, 0] - ld)) <= tol


def pin_decode_append_capacity_overflow(tol=1e-12):
    """Length cap - 1 plus three new rows: only the first is written and all
    three queries see the full cache (their causal limits lie past it)."""
    B, cap, Nq, Hq, Hkv, d = 1, 5, 3, 2, 1, 3
    q, kc, vc, kn, vn = _append_case(2330, B, cap, Nq, Hq, Hkv, d)
    k2, v2, o, l = O.decode_append(q, kc, vc, [cap - 1], kn, vn, True, 0.9)
    assert np.array_equal(k2[0, cap - 1], kn[0, 0]) and np.array_equal(v2[0, cap - 1], vn[0, 0])
    rows_k = np.array([kc[0, j] for j in range(cap - 1)] + [kn[0, 0]])[None]
    rows_v = np.array([vc[0, j] for j in range(cap - 1)] + [vn[0, 0]])[None]
    ob, lb = brute_attention(q, rows_k, rows_v, False, 0.9)
    assert np.max(np.abs(o - ob)) <= tol and np.max(np.abs(l - lb)) <= tol


# ---------------------------------------------------------------------------
# FP8: e4m3 codes, the randomised Hadamard rotation, block quantisation and
# attention on quantised operands
# ---------------------------------------------------------------------------
def _torch_e4m3(x):
    import torch
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_e4m3_against_torch(tol=0.0):
    """Encoding and decoding agree with torch's float8_e4m3fn cast on every
    code, every midpoint between neighbours and random values."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F8.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    fin = np.unique(np.abs(ref[np.isfinite(ref)]))
    mids = (fin[1:] + fin[:-1]) / 2
    r = np.random.default_rng(2400)
    x = np.concatenate([fin, -fin, mids, -mids, r.normal(size=4000) * 40,
                        r.uniform(-1, 1, 4000) * 2.0 ** r.integers(-12, 8, 4000)])
    x = np.clip(x, -448, 448).astype(np.float32).astype(np.float64)  # exact in float32 for torch
    assert np.array_equal(F8.e4m3_encode(x), _torch_e4m3(x)), "e4m3 encoding"


def pin_hadamard_rotation(tol=1e-12):
    """H_d equals scipy's Hadamard matrix; R = H diag(s) / sqrt(d) is
    orthogonal, so rotating Q and K keeps every score."""
    import scipy.linalg
    for d in (1, 2, 8, 64, 128):
        assert np.array_equal(F8.hadamard(d), scipy.linalg.hadamard(d))
    r = np.random.default_rng(2410)
    d = 64
    s = r.choice([-1.0, 1.0], size=d)
    R = F8.rotate(np.eye(d), s).T
    assert np.max(np.abs(R @ R.T - np.eye(d))) <= tol
    q, k = r.normal(size=(5, d)), r.normal(size=(7, d))
    assert np.max(np.abs(F8.rotate(q, s) @ F8.rotate(k, s).T - q @ k.T)) <= 1e-11
    # sign flips act before the transform: rotating the unit vector e_i gives
    # s_i times column i of scipy's H, over sqrt(d)
    Hs = scipy.linalg.hadamard(d)
    for i in range(d):
        ei = np.zeros(d)
        ei[i] = 1.0
        assert np.max(np.abs(F8.rotate(ei, s) - s[i] * Hs[:, i] / 8.0)) <= tol, ("rotation column", i)


def pin_block_exponent(tol=0.0):
    """Closed forms and the defining inequality amax <= 448 2^e < 2 amax."""
    cases = {448.0: 0, 449.0: 1, 224.0: -1, 224.5: 0, 1.0: -8, 0.0: 0, 448.0 * 2.0 ** 40: 40,
             2.0 ** -200: -127, 1e30: 91}
    for a, e in cases.items():
        assert F8.block_exponent(a) == e, (a, F8.block_exponent(a), e)
    r = np.random.default_rng(2420)
    for a in np.abs(r.normal(size=500)) * 2.0 ** r.integers(-60, 60, 500):
        e = F8.block_exponent(float(a))
        assert a <= 448.0 * 2.0 ** e and a > 448.0 * 2.0 ** (e - 1)


def pin_quantize_rows(tol=0.0):
    """Codes round each value to the nearest multiple the block's scale
    allows (half an e4m3 step), padding rows are zero, and scaling one block
    by a power of two moves only its exponent."""
    r = np.random.default_rng(2430)
    x = r.normal(size=(150, 16)) * 3.0
    x[70:128] *= 1000.0
    codes, exps = F8.quantize_rows(x)
    assert codes.shape == (192, 16) and exps.shape == (3,)
    assert not codes[150:].any()
    xh = F8.e4m3_decode(codes) * np.repeat(2.0 ** exps, 64)[:, None]
    for blk in range(3):
        rows = slice(64 * blk, min(64 * blk + 64, 150))
        amax = np.max(np.abs(x[rows]))
        assert amax <= 448.0 * 2.0 ** exps[blk] < 2 * amax
        step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(x[rows]), 1e-300))) - 3),
                          2.0 ** (exps[blk] - 9))
        assert np.all(np.abs(xh[rows] - x[rows]) <= step / 2 * (1 + 1e-12))
    y = x.copy()
    y[64:128] *= 2.0 ** 5
    c2, e2 = F8.quantize_rows(y)
    assert np.array_equal(c2, codes) and list(e2 - exps) == [0, 5, 0]


def _fp8_case(seed, B, Nq, Nk, Hq, Hkv, d, integer_scores=False):
    r = np.random.default_rng(seed)
    q = r.normal(size=(B, Nq, Hq, d))
    k = r.normal(size=(B, Nk, Hkv, d))
    v = r.normal(size=(B, Nk, Hkv, d))
    if integer_scores:  # every score an integer: q rows one-hot times small integers, k small integers
        q = np.zeros((B, Nq, Hq, d))
        q[..., 0] = 1.0
        k = r.integers(-6, 4, size=(B, Nk, Hkv, d)).astype(np.float64)
    qc, qe = F8.quantize_bhnd(q)
    kc, ke = F8.quantize_bhnd(k)
    vc, ve = F8.quantize_bhnd(v)
    return qc, qe, kc, ke, vc, ve


def pin_attention_fp8_exact_probabilities(tol=1e-12):
    """When every score (in base-2 units) is an integer, each quantised
    probability 2^(t - M + 6) is exactly an e4m3 value, so the FP8 model
    equals exact attention on the dequantised operands."""
    B, Nq, Nk, Hq, Hkv, d = 1, 70, 70, 4, 2, 8
    qc, qe, kc, ke, vc, ve = _fp8_case(2440, B, Nq, Nk, Hq, Hkv, d, integer_scores=True)
    scale = 1.0 / math.log2(math.e)  # t = q . k exactly up to one rounding of the product
    deq = lambda c, e, n: np.transpose(F8.dequantize_bhnd(c, e)[:, :, :n], (0, 2, 1, 3))
    for causal in (False, True):
        o, l = F8.attention_fp8(qc, qe, kc, ke, vc, ve, Nq, Nk, causal, scale)
        oe, le = brute_attention(deq(qc, qe, Nq), deq(kc, ke, Nk), deq(vc, ve, Nk), causal, scale)
        assert np.max(np.abs(o - oe)) <= tol, ("fp8 exact probabilities O", causal)
        assert np.max(np.abs(l - le)) <= tol, ("fp8 exact probabilities LSE", causal)


def pin_attention_fp8_error_bound(tol=1e-12):
    """On random operands the FP8 model stays within the bound its
    probability rounding allows around exact attention on the dequantised
    operands: |dO| <= (2^-4 sum_j p_j |v_j| + 2^-16 sum_j |v_j|) / sum_j p_j
    (relative half-step of a normal e4m3 value, half a subnormal step), and
    its LSE is the exact one (the denominator is not quantised)."""
    B, Nq, Nk, Hq, Hkv, d = 1, 90, 130, 2, 1, 16
    qc, qe, kc, ke, vc, ve = _fp8_case(2450, B, Nq, Nk, Hq, Hkv, d)
    scale = 0.3
    o, l = F8.attention_fp8(qc, qe, kc, ke, vc, ve, Nq, Nk, False, scale)
    Q = F8.dequantize_bhnd(qc, qe)[0, :, :Nq]
    K = F8.dequantize_bhnd(kc, ke)[0, :, :Nk]
    V = F8.dequantize_bhnd(vc, ve)[0, :, :Nk]
    worst = 0.0
    for h in range(Hq):
        s = scale * Q[h] @ K[0].T
        p = np.exp(s - s.max(axis=1, keepdims=True))
        oe = p @ V[0] / p.sum(axis=1, keepdims=True)
        le = np.log(p.sum(axis=1)) + s.max(axis=1)
        bound = (2.0 ** -4 * p @ np.abs(V[0]) + 2.0 ** -16 * np.abs(V[0]).sum(axis=0)[None, :]) / p.sum(axis=1)[:, None]
        err = np.abs(o[0, :, h] - oe)
        assert np.all(err <= bound * (1 + 1e-9)), "fp8 error bound"
        assert np.max(np.abs(l[0, h] - le)) <= tol, "fp8 LSE"
        worst = max(worst, float(np.max(err)))
    assert worst > 0.0  # the probabilities really were rounded


def pin_attention_fp8_brute_force(tol=1e-12):
    """Plain loops with torch's e4m3 cast for the probabilities."""
    B, Nq, Nk, Hq, Hkv, d = 1, 5, 7, 2, 1, 4
    qc, qe, kc, ke, vc, ve = _fp8_case(2460, B, Nq, Nk, Hq, Hkv, d)
    scale = 0.7
    Q = F8.dequantize_bhnd(qc, qe)
    K = F8.dequantize_bhnd(kc, ke)
    V = F8.dequantize_bhnd(vc, ve)
    import torch
    for causal in (False, True):
        o, l = F8.attention_fp8(qc, qe, kc, ke, vc, ve, Nq, Nk, causal, scale)
        for h in range(Hq):
            for i in range(Nq):
                keys = [j for j in range(Nk) if not causal or j <= i]
                t = [scale / math.log(2.0) * math.fsum(Q[0, h, i, x] * K[0, 0, j, x] for x in range(d)) for j in keys]
                M = math.ceil(max(t))
                den = math.fsum(2.0 ** (x - M) for x in t)
                pq = [float(torch.tensor(2.0 ** (x - M + 6), dtype=torch.float32).to(torch.float8_e4m3fn).float())
                      for x in t]
                for x in range(d):
                    want = 2.0 ** -6 * math.fsum(pq[n] * V[0, 0, j, x] for n, j in enumerate(keys)) / den
                    assert abs(o[0, i, h, x] - want) <= tol, ("fp8 brute O", causal, h, i, x)
                assert abs(l[0, h, i] - math.log(2.0) * (M + math.log2(den))) <= tol, ("fp8 brute LSE", causal)


# ---------------------------------------------------------------------------
# backward under windows and packed variable-length batches
# ---------------------------------------------------------------------------
def _torch_masked_grads(q, k, v, do, mask, scale):
    """PyTorch float64 autograd of softmax(scale Q K^T + mask) V for one
    head; rows without a visible key are zeroed before the product."""
    import torch
    Q, K, V = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    S = scale * Q @ K.T
    S = S.masked_fill(~torch.tensor(mask), float("-inf"))
    P = torch.softmax(S, dim=1)
    P = torch.where(torch.isnan(P), torch.zeros_like(P), P)
    O = P @ V
    O.backward(torch.tensor(do, dtype=torch.float64))
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


def pin_backward_window_torch_autograd(tol=1e-10):
    """Bottom-right windows (causal and sliding, Nq != Nk, rows with no key)
    against PyTorch float64 autograd with an explicit mask (built here by
    plain loops)."""
    r = np.random.default_rng(2500)
    B, Hq, Hkv, d = 1, 4, 2, 5
    for Nq, Nk, wl, wr in ((6, 9, -1, 0), (9, 6, -1, 0), (8, 8, 2, 1), (7, 10, 3, -1), (5, 5, 0, 0)):
        q = r.normal(size=(B, Nq, Hq, d))
        k = r.normal(size=(B, Nk, Hkv, d))
        v = r.normal(size=(B, Nk, Hkv, d))
        do = r.normal(size=(B, Nq, Hq, d))
        gq, gk, gv = O.attention_backward_window(q, k, v, do, wl, wr, 0.6)
        off = Nk - Nq
        mask = np.array([[(wl < 0 or j >= i + off - wl) and (wr < 0 or j <= i + off + wr) for j in range(Nk)]
                         for i in range(Nq)])
        rk = np.zeros_like(gk)
        rv = np.zeros_like(gv)
        for h in range(Hq):
            kv = (h * Hkv) // Hq
            tq, tk, tv = _torch_masked_grads(q[0, :, h], k[0, :, kv], v[0, :, kv], do[0, :, h], mask, 0.6)
            assert np.max(np.abs(gq[0, :, h] - tq)) <= tol, ("window dq", Nq, Nk, wl, wr)
            rk[0, :, kv] += tk
            rv[0, :, kv] += tv
        assert np.max(np.abs(gk - rk)) <= tol and np.max(np.abs(gv - rv)) <= tol, ("window dk/dv", Nq, Nk, wl, wr)


def pin_backward_varlen_concatenation(tol=1e-12):
    """A packed batch's gradients are its sequences' own, laid end to end
    (sequences pinned one by one against autograd above)."""
    r = np.random.default_rng(2510)
    lq, lk = [3, 0, 5, 2], [4, 2, 5, 6]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q = r.normal(size=(cu_q[-1], 2, 3))
    k = r.normal(size=(cu_k[-1], 1, 3))
    v = r.normal(size=(cu_k[-1], 1, 3))
    do = r.normal(size=(cu_q[-1], 2, 3))
    for wl, wr in ((-1, -1), (-1, 0), (1, 1)):
        gq, gk, gv = O.attention_backward_varlen(q, k, v, do, cu_q, cu_k, wl, wr, 0.7)
        for b in range(4):
            qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
            if lq[b] == 0:
                assert not gk[ks].any() and not gv[ks].any(), "keys of a sequence without queries"
                continue
            mask = np.array([[(wl < 0 or j >= i + lk[b] - lq[b] - wl) and (wr < 0 or j <= i + lk[b] - lq[b] + wr)
                              for j in range(lk[b])] for i in range(lq[b])])
            tq, tk, tv = _torch_masked_grads(q[qs, :, :].transpose(1, 0, 2)[0], k[ks, 0], v[ks, 0],
                                             do[qs].transpose(1, 0, 2)[0], mask, 0.7)
            tq1, tk1, tv1 = _torch_masked_grads(q[qs, 1], k[ks, 0], v[ks, 0], do[qs, 1], mask, 0.7)
            assert np.max(np.abs(gq[qs, 0] - tq)) <= 1e-10 and np.max(np.abs(gq[qs, 1] - tq1)) <= 1e-10
            assert np.max(np.abs(gk[ks, 0] - (tk + tk1))) <= 1e-10 and np.max(np.abs(gv[ks, 0] - (tv + tv1))) <= 1e-10


ALL_PINS = [
    pin_brute_force,
    pin_torch_sdpa,
    pin_scipy_rows,
    pin_golden_closed_forms,
    pin_row_stochastic,
    pin_constant_values,
    pin_key_permutation,
    pin_zero_query_closed_form,
    pin_single_key,
    pin_large_scale_argmax,
    pin_causal_prefix,
    pin_gqa_repeat,
    pin_split_combine,
    pin_decode,
    pin_decode_paged,
    pin_online_recurrence,
    pin_backward_torch_autograd,
    pin_backward_finite_differences,
    pin_backward_constant_values,
    pin_backward_gqa_sum,
    pin_window_brute_force,
    pin_window_torch_mask,
    pin_window_special_cases,
    pin_varlen_concatenation,
    pin_decode_append_brute_force,
    pin_decode_append_cache_update,
    pin_decode_append_reduces_to_decode,
    pin_decode_append_capacity_overflow,
    pin_e4m3_against_torch,
    pin_hadamard_rotation,
    pin_block_exponent,
    pin_quantize_rows,
    pin_attention_fp8_exact_probabilities,
    pin_attention_fp8_error_bound,
    pin_attention_fp8_brute_force,
    pin_backward_window_torch_autograd,
    pin_backward_varlen_concatenation,
]
