"""Plant plausible mistakes in the oracle (on the CPU) and check a pin fails.

Each mutation replaces one helper of ``oracle.sdpa`` for the duration of the
test; the pin suite must reject every one of them, which shows the pins
constrain each part of the oracle rather than echo it.
"""

import numpy as np
import pytest

import oracle_pins as P
from oracle import fp8 as F8
from oracle import sdpa as O

_orig = {n: getattr(O, n) for n in ("kv_head_of", "visible_mask", "scores", "softmax_rows",
                                    "attention_rows", "decode", "merge_partials",
                                    "online_softmax_attention", "attention_backward_rows", "decode_paged",
                                    "window_mask", "attention_varlen", "decode_append",
                                    "attention_backward_window", "attention_backward_varlen")}


def _interleaved_groups(hq, Hq, Hkv):
    _orig["kv_head_of"](hq, Hq, Hkv)
    return hq % Hkv


def _strict_causal(Nq, Nk, causal, rows=None):
    i = np.arange(Nq) if rows is None else np.asarray(rows)
    j = np.arange(Nk)
    return (j[None, :] < i[:, None]) if causal else np.ones((i.shape[0], Nk), dtype=bool)


def _reversed_causal(Nq, Nk, causal, rows=None):
    i = np.arange(Nq) if rows is None else np.asarray(rows)
    j = np.arange(Nk)
    return (j[None, :] >= i[:, None]) if causal else np.ones((i.shape[0], Nk), dtype=bool)


def _bottom_right_causal(Nq, Nk, causal, rows=None):
    i = np.arange(Nq) if rows is None else np.asarray(rows)
    j = np.arange(Nk)
    return (j[None, :] <= i[:, None] + (Nk - Nq)) if causal else np.ones((i.shape[0], Nk), dtype=bool)


def _no_scale(q_rows, k_rows, scale):
    return _orig["scores"](q_rows, k_rows, 1.0)


def _sqrt_scale(q_rows, k_rows, scale):
    return _orig["scores"](q_rows, k_rows, scale / np.sqrt(np.asarray(q_rows).shape[-1]))


def _transposed_scores(q_rows, k_rows, scale):
    S = _orig["scores"](q_rows, k_rows, scale)
    return S.T if S.shape[0] == S.shape[1] else S[:, ::-1]


def _lse_without_max(S, mask):
    P_, lse = _orig["softmax_rows"](S, mask)
    S = np.where(mask, np.asarray(S, float), -np.inf)
    mx = S.max(axis=1)
    return P_, lse - np.where(np.isfinite(mx), mx, 0.0)


def _unnormalised(S, mask):
    P_, lse = _orig["softmax_rows"](S, mask)
    return P_ * np.exp(lse)[:, None] / np.exp(np.where(np.isfinite(lse), lse.max(), 0.0)), lse


def _column_softmax(S, mask):
    P_, lse = _orig["softmax_rows"](np.asarray(S).T, np.asarray(mask).T)
    if P_.shape[0] != P_.shape[1]:
        return _orig["softmax_rows"](S, mask)[0][:, ::-1], lse[: np.asarray(S).shape[0]]
    return P_.T, lse


def _values_from_keys(q, k, v, causal, scale, b, hq, rows=None):
    return _orig["attention_rows"](q, k, k if np.asarray(k).shape == np.asarray(v).shape else v,
                                   causal, scale, b, hq, rows)


def _decode_off_by_one(q, kcache, vcache, seqlens, scale, heads=None):
    cap = np.asarray(kcache).shape[1]
    return _orig["decode"](q, kcache, vcache, [min(int(n) + 1, cap) if int(n) < cap else int(n) - 1
                                               for n in seqlens], scale, heads)


def _merge_plain_mean(o_parts, lse_parts):
    o, lse = _orig["merge_partials"](o_parts, lse_parts)
    return np.asarray(o_parts, float).mean(axis=0), lse


def _recurrence_wrong_alpha(q_rows, k_rows, v_rows, causal, scale, block_q, block_k):
    # alpha = e^(m' - m) instead of e^(m - m'): emulate by running the
    # recurrence with the opposite rescale through a local copy.
    Q, K, V = (np.asarray(x, float) for x in (q_rows, k_rows, v_rows))
    Nq, Nk = Q.shape[0], K.shape[0]
    Oo = np.zeros((Nq, V.shape[1]))
    L = np.zeros(Nq)
    for i0 in range(0, Nq, block_q):
        rows = np.arange(i0, min(i0 + block_q, Nq))
        m = np.full(len(rows), -np.inf)
        l = np.zeros(len(rows))
        a = np.zeros((len(rows), V.shape[1]))
        for j0 in range(0, Nk, block_k):
            cols = np.arange(j0, min(j0 + block_k, Nk))
            S = scale * Q[rows] @ K[cols].T
            if causal:
                S = np.where(cols[None, :] <= rows[:, None], S, -np.inf)
            m_new = np.maximum(m, S.max(axis=1))
            mu = np.where(np.isfinite(m_new), m_new, 0.0)
            alpha = np.where(np.isfinite(m), np.exp(np.minimum(mu - m, 50.0)), 0.0)
            E = np.exp(S - mu[:, None])
            l = alpha * l + E.sum(axis=1)
            a = alpha[:, None] * a + E @ V[cols]
            m = m_new
        Oo[rows] = a / l[:, None]
        L[rows] = m + np.log(l)
    return Oo, L


def _bwd_variant(kind):
    def f(q, k, v, do, causal, scale, b, hq):
        q, k, v, do = (np.asarray(x) for x in (q, k, v, do))
        _, Nq, Hq, _ = q.shape
        Nk, Hkv = k.shape[1], k.shape[2]
        kv = O.kv_head_of(hq, Hq, Hkv)
        Q, K, V, dO = (np.asarray(x, float) for x in (q[b, :, hq], k[b, :, kv], v[b, :, kv], do[b, :, hq]))
        P_, _ = O.softmax_rows(O.scores(Q, K, scale), O.visible_mask(Nq, Nk, causal))
        dP = dO @ V.T
        dS = P_ * (dP - np.sum(P_ * dP, axis=1, keepdims=True))
        dQ, dK, dV = scale * (dS @ K), scale * (dS.T @ Q), P_.T @ dO
        if kind == "no_softmax_correction":
            dS = P_ * dP
            dQ, dK = scale * (dS @ K), scale * (dS.T @ Q)
        elif kind == "unscaled_dk":
            dK = dS.T @ Q
        elif kind == "dq_from_values":
            dQ = scale * (dS @ V) if V.shape == K.shape else dQ * 2
        elif kind == "dv_untransposed":
            dV = (P_ @ dO[: P_.shape[1]]) if P_.shape[0] >= P_.shape[1] else np.zeros_like(dV)
        return dQ, dK, dV
    f.__name__ = "_bwd_" + kind
    return f


def _paged_identity_table(q, kpages, vpages, block_table, seqlens, scale, heads=None):
    bt = np.asarray(block_table)
    return _orig["decode_paged"](q, kpages, vpages, np.sort(bt, axis=1), seqlens, scale, heads)


def _window_top_left(Nq, Nk, window_left, window_right, rows=None):
    i = np.arange(Nq) if rows is None else np.asarray(rows)
    j = np.arange(Nk)
    m = np.ones((i.shape[0], Nk), dtype=bool)
    if window_left >= 0:
        m &= j[None, :] >= i[:, None] - window_left
    if window_right >= 0:
        m &= j[None, :] <= i[:, None] + window_right
    return m


def _window_exclusive(Nq, Nk, window_left, window_right, rows=None):
    m = _orig["window_mask"](Nq, Nk, window_left, window_right, rows)
    i = np.arange(Nq) if rows is None else np.asarray(rows)
    j = np.arange(Nk)
    if window_left >= 0:
        m &= j[None, :] > (i + Nk - Nq)[:, None] - window_left
    return m


def _varlen_shared_keys(q, k, v, cu_q, cu_k, window_left, window_right, scale):
    return _orig["attention_varlen"](q, k, v, cu_q, cu_q if len(cu_q) == len(cu_k) and cu_q[-1] <= cu_k[-1]
                                     else cu_k, window_left, window_right, scale)


def _append_variant(kind):
    """decode_append with one planted mistake."""
    def f(q, kcache, vcache, seqlens, k_new, v_new, causal, scale):
        q = np.asarray(q, dtype=np.float64)
        kc = np.array(kcache, dtype=np.float64)
        vc = np.array(vcache, dtype=np.float64)
        B, Nq, Hq, _ = q.shape
        cap, Hkv = kc.shape[1], kc.shape[2]
        n_new = 0 if k_new is None else Nq
        O_ = np.zeros((B, Nq, Hq, vc.shape[3]))
        L_ = np.zeros((B, Hq, Nq))
        for b in range(B):
            base = min(max(int(seqlens[b]), 0), cap)
            at = base + 1 if kind == "shifted_write" else base
            for i in range(n_new):
                if at + i < cap:
                    kc[b, at + i] = k_new[b, i]
                    vc[b, at + i] = v_new[b, i]
            n = base + n_new
            avail = min(n, cap) if kind != "old_length" else base
            j = np.arange(avail)
            mask = np.ones((Nq, avail), dtype=bool)
            if causal:
                lim = np.arange(Nq) if kind == "top_left" else n - Nq + np.arange(Nq)
                mask &= j[None, :] <= lim[:, None]
            for hq in range(Hq):
                kv = O.kv_head_of(hq, Hq, Hkv)
                P_, lse = O.softmax_rows(O.scores(q[b, :, hq], kc[b, :avail, kv], scale), mask)
                O_[b, :, hq] = P_ @ vc[b, :avail, kv]
                L_[b, hq] = lse
        return kc, vc, O_, L_
    f.__name__ = f"_append_{kind}"
    return f


def _bwd_window_top_left(q, k, v, do, window_left, window_right, scale):
    # windows aligned to the top-left corner: pretend Nk = Nq for the offset
    saved = O.window_mask
    O.window_mask = lambda Nq, Nk, wl, wr, rows=None: _window_top_left(Nq, Nk, wl, wr, rows)
    try:
        return _orig["attention_backward_window"](q, k, v, do, window_left, window_right, scale)
    finally:
        O.window_mask = saved


def _bwd_varlen_keys_of_next(q, k, v, do, cu_q, cu_k, window_left, window_right, scale):
    # off by one sequence in the key offsets
    cu_k2 = np.concatenate([cu_k[1:], [cu_k[-1]]]) if len(cu_k) > 2 else cu_k
    cu_k2 = np.maximum.accumulate(np.concatenate([[0], cu_k2[1:]]))
    return _orig["attention_backward_varlen"](q, k, v, do, cu_q, cu_k2, window_left, window_right, scale)


MUTATIONS = [
    ("kv_head_of", _interleaved_groups),
    ("visible_mask", _strict_causal),
    ("visible_mask", _reversed_causal),
    ("visible_mask", _bottom_right_causal),
    ("scores", _no_scale),
    ("scores", _sqrt_scale),
    ("scores", _transposed_scores),
    ("softmax_rows", _lse_without_max),
    ("softmax_rows", _unnormalised),
    ("softmax_rows", _column_softmax),
    ("attention_rows", _values_from_keys),
    ("decode", _decode_off_by_one),
    ("merge_partials", _merge_plain_mean),
    ("online_softmax_attention", _recurrence_wrong_alpha),
    ("attention_backward_rows", _bwd_variant("no_softmax_correction")),
    ("attention_backward_rows", _bwd_variant("unscaled_dk")),
    ("attention_backward_rows", _bwd_variant("dq_from_values")),
    ("attention_backward_rows", _bwd_variant("dv_untransposed")),
    ("decode_paged", _paged_identity_table),
    ("window_mask", _window_top_left),
    ("window_mask", _window_exclusive),
    ("attention_varlen", _varlen_shared_keys),
    ("decode_append", _append_variant("shifted_write")),
    ("decode_append", _append_variant("old_length")),
    ("decode_append", _append_variant("top_left")),
    ("attention_backward_window", _bwd_window_top_left),
    ("attention_backward_varlen", _bwd_varlen_keys_of_next),
]


_orig_fp8 = {n: getattr(F8, n) for n in ("e4m3_encode", "block_exponent", "rotate", "attention_fp8",
                                          "dequantize_bhnd", "quantize_rows")}


def _e4m3_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    vals = F8.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    idx = np.searchsorted(vals, np.abs(x), side="right") - 1
    code = idx.astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def _e4m3_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    c = _orig_fp8["e4m3_encode"](x)
    vals = F8.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    a = np.abs(x)
    hi = np.clip(np.searchsorted(vals, a), 0, len(vals) - 1)
    tie = (hi > 0) & (vals[hi] - a == a - vals[np.maximum(hi - 1, 0)])
    up = np.where(np.signbit(x), hi.astype(np.uint8) | 0x80, hi.astype(np.uint8))
    return np.where(tie, up, c).astype(np.uint8)


def _exponent_plus_one(amax):
    return min(127, _orig_fp8["block_exponent"](amax) + 1) if amax else 0


def _rotate_no_signs(x, signs):
    return _orig_fp8["rotate"](x, np.ones_like(np.asarray(signs, dtype=np.float64)))


def _fp8_unquantised_p(qc, qe, kc, ke, vc, ve, Nq, Nk, causal, scale):
    saved = F8.e4m3_encode
    F8.e4m3_encode = lambda x: x  # decode(x) then sees values, not codes: give it a float path
    try:
        dec = F8.e4m3_decode
        F8.e4m3_decode = lambda c: np.asarray(c, dtype=np.float64) if np.asarray(c).dtype != np.uint8 else dec(c)
        return _orig_fp8["attention_fp8"](qc, qe, kc, ke, vc, ve, Nq, Nk, causal, scale)
    finally:
        F8.e4m3_encode = saved
        F8.e4m3_decode = dec


def _fp8_bias_zero(qc, qe, kc, ke, vc, ve, Nq, Nk, causal, scale):
    saved = F8.P_BIAS
    F8.P_BIAS = 0
    try:
        return _orig_fp8["attention_fp8"](qc, qe, kc, ke, vc, ve, Nq, Nk, causal, scale)
    finally:
        F8.P_BIAS = saved


def _dequantize_without_exponents(codes, exps):
    return _orig_fp8["dequantize_bhnd"](codes, np.zeros_like(np.asarray(exps)))


def _quantize_rows_32(x):
    saved = F8.BLOCK
    F8.BLOCK = 32
    try:
        return _orig_fp8["quantize_rows"](x)
    finally:
        F8.BLOCK = saved


MUTATIONS_FP8 = [
    ("e4m3_encode", _e4m3_truncate),
    ("e4m3_encode", _e4m3_ties_away),
    ("block_exponent", _exponent_plus_one),
    ("rotate", _rotate_no_signs),
    ("attention_fp8", _fp8_unquantised_p),
    ("attention_fp8", _fp8_bias_zero),
    ("dequantize_bhnd", _dequantize_without_exponents),
    ("quantize_rows", _quantize_rows_32),
]


@pytest.mark.parametrize("name,bad", MUTATIONS_FP8, ids=[f"{n}:{f.__name__}" for n, f in MUTATIONS_FP8])
def test_some_pin_rejects_fp8_mutation(monkeypatch, name, bad):
    monkeypatch.setattr(F8, name, bad)
    failed = []
    for pin in P.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except AssertionError:
            failed.append(pin.__name__)
        except Exception as exc:
            failed.append(f"{pin.__name__}({type(exc).__name__})")
    assert failed, f"no pin caught the planted mistake {name}:{bad.__name__}"


@pytest.mark.parametrize("name,bad", MUTATIONS, ids=[f"{n}:{f.__name__}" for n, f in MUTATIONS])
def test_some_pin_rejects_mutation(monkeypatch, name, bad):
    monkeypatch.setattr(O, name, bad)
    failed = []
    for pin in P.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except AssertionError:
            failed.append(pin.__name__)
        except Exception as exc:  # a crash also counts as caught, but say so
            failed.append(f"{pin.__name__}({type(exc).__name__})")
    assert failed, f"no pin caught the planted mistake {name}:{bad.__name__}"
