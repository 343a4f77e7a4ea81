"""CPU float64 oracle: attention written out from its definition.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Sources (the pages this follows; cited by page title and section):

* FlashAttention: Part 2, section 2.1 "PyTorch Scaled-Dot-Product Attention
  Today": the function is softmax(Q K^T / sqrt(d)) V.
* FlashAttention: Part 2, section 3.2 and section 1.6: dense FlashAttention
  evaluates that function for every required query/key pair, no pair
  skipped, so the tiled method is exact up to rounding order and the oracle
  is simply the definition.
* FlashAttention: Part 2, section 1.3: one row-wise log-sum-exp per query row
  is the per-row statistic kept next to the output.
* pyshine.com FlashAttention code tour, "Why You Need This": grouped-query
  attention lets K and V carry fewer heads than Q when the counts divide
  evenly; decode with query length one splits the cache over thread blocks
  and combines the partial results.
* FlashAttention: Part 2, section 4.1: decode is one query row against the
  whole key/value cache.
* FlashAttention: Part 2, section 6.2 "FlashAttention Summary": the online
  softmax state (m, l, a) and the rescale factor alpha = e^(m - m').

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):

* LSE is the natural log of the sum of e^(s) over the visible keys of the
  *scaled* scores s = scale * <q, k>.
* Causal is top-left aligned: key j is visible to query i iff j <= i.
* Grouped heads are contiguous: query head hq reads key/value head
  hq // (Hq // Hkv).
* A row with no visible key has O = 0 and LSE = -inf.
* Layout is (batch, sequence, heads, head_dim) for q, k, v and o; LSE is
  (batch, heads, queries).

Everything is float64. Inputs of any real dtype are converted with
``numpy.asarray(..., dtype=float64)``, which is exact for bf16/fp32 values.
"""

import numpy as np

__all__ = [
    "kv_head_of",
    "visible_mask",
    "scores",
    "softmax_rows",
    "attention",
    "attention_rows",
    "decode",
    "decode_paged",
    "merge_partials",
    "online_softmax_attention",
    "attention_backward_rows",
    "attention_backward",
    "window_mask",
    "attention_window",
    "attention_varlen",
    "decode_append",
    "attention_backward_window",
    "attention_backward_varlen",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def kv_head_of(hq, Hq, Hkv):
    """Key/value head read by query head ``hq`` (contiguous groups of Hq/Hkv).

    pyshine.com FlashAttention code tour, "Why You Need This": K and V may
    carry fewer heads than Q when the counts divide evenly. The grouping
    order is not stated; contiguous groups are the reading taken here.
    """
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a positive multiple of Hkv")
    return hq // (Hq // Hkv)


def visible_mask(Nq, Nk, causal, rows=None):
    """Boolean (len(rows), Nk) mask of the key positions each query sees.

    Non-causal: every key. Causal (top-left): key j is visible to query i
    iff j <= i. ``rows`` selects query indices (default: all Nq).
    """
    i = np.arange(Nq) if rows is None else np.asarray(rows)
    j = np.arange(Nk)
    if causal:
        return j[None, :] <= i[:, None]
    return np.ones((i.shape[0], Nk), dtype=bool)


def scores(q_rows, k_rows, scale):
    """Scaled scores s_ij = scale * <q_i, k_j> for (n, d) and (m, d) inputs.

    FlashAttention: Part 2, section 2.1: the argument of the softmax is
    Q K^T scaled (by 1/sqrt(d) by default; here by the caller's scale).
    """
    return float(scale) * (_f64(q_rows) @ _f64(k_rows).T)


def softmax_rows(S, mask):
    """Row softmax over visible entries; returns (P, LSE) in float64.

    P_ij = e^(s_ij - LSE_i) on visible entries and 0 elsewhere, with
    LSE_i = ln sum_{visible j} e^(s_ij) computed as max + ln(sum e^(s - max)).
    A row with no visible entry gets P = 0 and LSE = -inf.
    """
    S = _f64(S)
    Sm = np.where(mask, S, -np.inf)
    row_max = Sm.max(axis=1, keepdims=True) if S.shape[1] > 0 else np.full((S.shape[0], 1), -np.inf)
    empty = ~np.isfinite(row_max)
    safe_max = np.where(empty, 0.0, row_max)
    E = np.where(mask, np.exp(Sm - safe_max), 0.0)
    denom = E.sum(axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        P = np.where(empty, 0.0, E / np.where(empty, 1.0, denom))
        lse = np.where(empty, -np.inf, safe_max + np.log(np.where(empty, 1.0, denom)))
    return P, lse[:, 0]


def attention_rows(q, k, v, causal, scale, b, hq, rows=None):
    """O and LSE for query head ``hq`` of batch ``b`` at the given rows.

    q: (B, Nq, Hq, d); k, v: (B, Nk, Hkv, d). Returns (O (n, d), LSE (n,)).
    The full score row block is materialised, masked, softmaxed and
    multiplied by V (the naive execution the method avoids).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    _, Nq, Hq, _ = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    kv = kv_head_of(hq, Hq, Hkv)
    rows = np.arange(Nq) if rows is None else np.asarray(rows)
    S = scores(q[b, rows, hq, :], k[b, :, kv, :], scale)
    P, lse = softmax_rows(S, visible_mask(Nq, Nk, causal, rows))
    O = P @ _f64(v[b, :, kv, :])
    return O, lse


def attention(q, k, v, causal, scale):
    """Full attention: O (B, Nq, Hq, dv) float64 and LSE (B, Hq, Nq) float64."""
    q = np.asarray(q)
    B, Nq, Hq, _ = q.shape
    dv = np.asarray(v).shape[3]
    O = np.zeros((B, Nq, Hq, dv), dtype=np.float64)
    L = np.zeros((B, Hq, Nq), dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            o, lse = attention_rows(q, k, v, causal, scale, b, hq)
            O[b, :, hq, :] = o
            L[b, hq, :] = lse
    return O, L


def decode(q, kcache, vcache, seqlens, scale, heads=None):
    """One new query per sequence against the first ``seqlens[b]`` cache rows.

    FlashAttention: Part 2, section 4.1: decode has one query row and reads
    the whole existing cache. q: (B, 1, Hq, d) or (B, Hq, d);
    kcache, vcache: (B, capacity, Hkv, d); seqlens: (B,) integers.
    Returns O (B, Hq, dv) and LSE (B, Hq); optional ``heads`` restricts the
    query heads computed (others are left as NaN).
    """
    q = np.asarray(q)
    if q.ndim == 4:
        q = q[:, 0]
    B, Hq, _ = q.shape
    Hkv = np.asarray(kcache).shape[2]
    dv = np.asarray(vcache).shape[3]
    O = np.full((B, Hq, dv), np.nan)
    L = np.full((B, Hq), np.nan)
    heads = range(Hq) if heads is None else heads
    for b in range(B):
        n = int(seqlens[b])
        for hq in heads:
            kv = kv_head_of(hq, Hq, Hkv)
            S = scores(q[b, hq][None, :], np.asarray(kcache)[b, :n, kv, :], scale)
            P, lse = softmax_rows(S, np.ones((1, n), dtype=bool))
            O[b, hq] = (P @ _f64(np.asarray(vcache)[b, :n, kv, :]))[0]
            L[b, hq] = lse[0]
    return O, L


def decode_paged(q, kpages, vpages, block_table, seqlens, scale, heads=None):
    """``decode`` over a paged cache.

    pyshine.com FlashAttention code tour (the paged KV cache of the
    with-kvcache entry point, after PagedAttention): sequence b's cache rows
    are its pages block_table[b, 0], block_table[b, 1], ... laid end to end.
    kpages, vpages: (num_pages, page_size, Hkv, d); block_table:
    (B, pages_per_seq) page indices.
    """
    kp = np.asarray(kpages)
    vp = np.asarray(vpages)
    bt = np.asarray(block_table)
    B, pps = bt.shape
    _, P, Hkv, d = kp.shape
    kc = kp[bt].reshape(B, pps * P, Hkv, d)
    vc = vp[bt].reshape(B, pps * P, Hkv, vp.shape[3])
    return decode(q, kc, vc, seqlens, scale, heads)


def merge_partials(o_parts, lse_parts):
    """Combine results over disjoint key sets into the result over their union.

    pyshine.com FlashAttention code tour, "Why You Need This": decode splits
    the cache across thread blocks and combines partial results. The combine
    is not printed; with the per-row log-sum-exp of FlashAttention: Part 2,
    section 1.3, the exact combine of parts s is
        LSE = ln sum_s e^(LSE_s),  O = sum_s e^(LSE_s - LSE) O_s.
    o_parts: (S, ..., d); lse_parts: (S, ...). Parts with LSE = -inf carry no
    weight; if every part is empty the result is O = 0, LSE = -inf.
    """
    o_parts = _f64(o_parts)
    lse_parts = _f64(lse_parts)
    m = lse_parts.max(axis=0)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lse_parts - m_safe[None])
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, tot)))
        O = (w[..., None] * o_parts).sum(axis=0) / np.where(empty, 1.0, tot)[..., None]
    O = np.where(empty[..., None], 0.0, O)
    return O, lse


def online_softmax_attention(q_rows, k_rows, v_rows, causal, scale, block_q, block_k):
    """The tiled online-softmax recurrence, one (batch, head) at a time.

    FlashAttention: Part 2, section 6.2: Q is split into tiles Q_i and K, V
    into tiles K_j, V_j; for each score tile the state (m, l, a) = (running
    maximum, running sum of exponentials, running unnormalised value sum) is
    updated, the old state rescaled by alpha = e^(m - m') when the maximum
    grows, and the tile discarded. The update equations are lost in the
    page's text; the plainest recurrence consistent with that state is
        m' = max(m, rowmax S_ij)
        l' = e^(m - m') l + sum_j e^(S_ij - m')
        a' = e^(m - m') a + e^(S_ij - m') V_j
    and at the end O = a / l and LSE = m + ln l (deferred normalisation,
    FlashAttention: Part 2, section 1.3 and the post on tracing
    FlashAttention's evolution through plain PyTorch code).
    q_rows: (Nq, d); k_rows, v_rows: (Nk, d). Returns (O, LSE).
    """
    Q = _f64(q_rows)
    K = _f64(k_rows)
    V = _f64(v_rows)
    Nq, Nk = Q.shape[0], K.shape[0]
    O = np.zeros((Nq, V.shape[1]))
    LSE = np.full(Nq, -np.inf)
    for i0 in range(0, Nq, block_q):
        rows = np.arange(i0, min(i0 + block_q, Nq))
        m = np.full(rows.shape[0], -np.inf)
        l = np.zeros(rows.shape[0])
        a = np.zeros((rows.shape[0], V.shape[1]))
        for j0 in range(0, Nk, block_k):
            cols = np.arange(j0, min(j0 + block_k, Nk))
            S = scores(Q[rows], K[cols], scale)
            vis = visible_mask(Nq, Nk, causal, rows)[:, cols]
            S = np.where(vis, S, -np.inf)
            m_new = np.maximum(m, S.max(axis=1))
            m_use = np.where(np.isfinite(m_new), m_new, 0.0)
            alpha = np.exp(m - m_use)
            E = np.exp(S - m_use[:, None])
            l = alpha * l + E.sum(axis=1)
            a = alpha[:, None] * a + E @ V[cols]
            m = m_new
        done = l > 0
        with np.errstate(divide="ignore", invalid="ignore"):
            O[rows] = np.where(done[:, None], a / np.where(done, l, 1.0)[:, None], 0.0)
            LSE[rows] = np.where(done, m + np.log(np.where(done, l, 1.0)), -np.inf)
    return O, LSE


def attention_backward_rows(q, k, v, do, causal, scale, b, hq):
    """Gradients of one (batch, query head) block for an upstream gradient dO.

    FlashAttention: Part 2, section 1.3: the backward pass keeps only the
    row-wise log-sum-exp from the forward pass and recomputes the score
    tiles (the pyshine.com code tour, on the kernel sources, describes the
    same recompute-then-accumulate backward). What it computes is the
    derivative of the forward definition (FlashAttention: Part 2, section
    2.1, O = softmax(scale Q K^T) V), written out by the chain rule:

        dV = P^T dO
        dP = dO V^T
        dS_ij = P_ij (dP_ij - sum_l P_il dP_il)      (softmax Jacobian)
        dQ = scale dS K,   dK = scale dS^T Q

    Returns (dq (Nq, d), dk (Nk, d), dv (Nk, dv)) for this query head; the
    key/value gradients of a grouped head are the sums over its group.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    do = np.asarray(do)
    _, Nq, Hq, _ = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    kv = kv_head_of(hq, Hq, Hkv)
    Q, K, V = _f64(q[b, :, hq, :]), _f64(k[b, :, kv, :]), _f64(v[b, :, kv, :])
    dO = _f64(do[b, :, hq, :])
    P, _ = softmax_rows(scores(Q, K, scale), visible_mask(Nq, Nk, causal))
    dV = P.T @ dO
    dP = dO @ V.T
    dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
    dQ = float(scale) * (dS @ K)
    dK = float(scale) * (dS.T @ Q)
    return dQ, dK, dV


def attention_backward(q, k, v, do, causal, scale):
    """dq (B, Nq, Hq, d), dk and dv (B, Nk, Hkv, d) in float64.

    Grouped query heads (pyshine.com code tour, "Why You Need This") read
    the same key/value head, so that head's gradients sum over the group.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    B, Nq, Hq, _ = q.shape
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(np.asarray(v).shape, dtype=np.float64)
    Hkv = k.shape[2]
    for b in range(B):
        for hq in range(Hq):
            kv = kv_head_of(hq, Hq, Hkv)
            gq, gk, gv = attention_backward_rows(q, k, v, do, causal, scale, b, hq)
            dq[b, :, hq, :] = gq
            dk[b, :, kv, :] += gk
            dv[b, :, kv, :] += gv
    return dq, dk, dv


def window_mask(Nq, Nk, window_left, window_right, rows=None):
    """Boolean (len(rows), Nk) mask of a bottom-right aligned local window.

    pyshine.com FlashAttention code tour: causal masking is aligned to the
    bottom right since version 2.1 (the last query sees the last key) and
    sliding windows arrived in 2.3. With off = Nk - Nq, key j is visible to
    query i iff i + off - window_left <= j <= i + off + window_right; a
    negative bound means no limit on that side. Causal (bottom-right) is
    window_left < 0, window_right = 0.
    """
    i = np.arange(Nq) if rows is None else np.asarray(rows)
    j = np.arange(Nk)
    c = (i + (Nk - Nq))[:, None]
    m = np.ones((i.shape[0], Nk), dtype=bool)
    if window_left >= 0:
        m &= j[None, :] >= c - window_left
    if window_right >= 0:
        m &= j[None, :] <= c + window_right
    return m


def attention_window(q, k, v, window_left, window_right, scale):
    """Attention under ``window_mask``: O (B, Nq, Hq, dv), LSE (B, Hq, Nq).

    Rows that see no key get O = 0 and LSE = -inf (as ``softmax_rows``).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, Nq, Hq, _ = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    O = np.zeros((B, Nq, Hq, v.shape[3]))
    L = np.zeros((B, Hq, Nq))
    mask = window_mask(Nq, Nk, window_left, window_right)
    for b in range(B):
        for hq in range(Hq):
            kv = kv_head_of(hq, Hq, Hkv)
            P, lse = softmax_rows(scores(q[b, :, hq], k[b, :, kv], scale), mask)
            O[b, :, hq] = P @ _f64(v[b, :, kv])
            L[b, hq] = lse
    return O, L


def attention_varlen(q, k, v, cu_q, cu_k, window_left, window_right, scale):
    """Packed variable-length batch: sequence b is rows cu_q[b]:cu_q[b+1] of
    q (total_q, Hq, d) against rows cu_k[b]:cu_k[b+1] of k and v
    (total_k, Hkv, d) (pyshine.com code tour: variable-length batches
    since 2.0, the padded batch flattened into packed token arrays).
    Returns O (total_q, Hq, dv) and LSE (Hq, total_q).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    O = np.zeros(q.shape[:2] + (v.shape[2],))
    L = np.zeros((q.shape[1], q.shape[0]))
    for b in range(len(cu_q) - 1):
        qa, qb, ka, kb = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if qb == qa:
            continue
        o, lse = attention_window(q[None, qa:qb], k[None, ka:kb], v[None, ka:kb], window_left, window_right, scale)
        O[qa:qb] = o[0]
        L[:, qa:qb] = lse[0]
    return O, L


def decode_append(q, kcache, vcache, seqlens, k_new, v_new, causal, scale):
    """A decode step that first writes the new tokens' keys and values into
    the cache, then attends to the grown cache.

    pyshine.com FlashAttention code tour, "Why You Need This" and its usage
    example: the with-kvcache entry point takes a preallocated cache with
    per-sequence lengths and updates it in place with the new tokens; causal
    masking is bottom-right aligned (version 2.1). FlashAttention: Part 2,
    section 4.1: the step then reads the whole cache.

    q: (B, Nq, Hq, d); kcache, vcache: (B, capacity, Hkv, d); seqlens: (B,)
    rows already in the cache; k_new, v_new: (B, Nq, Hkv, d) or both None
    (nothing appended). Readings where the pages are silent: a length is
    clamped to [0, capacity]; new rows at or past capacity are dropped;
    with n = length + appended rows, query i sees key j iff j < min(n,
    capacity) and, when causal, j <= n - Nq + i; a query that sees no key
    gets O = 0 and LSE = -inf.
    Returns (kcache', vcache', O (B, Nq, Hq, dv), LSE (B, Hq, Nq)); the
    inputs are not modified.
    """
    q = _f64(q)
    kc = _f64(kcache).copy()
    vc = _f64(vcache).copy()
    B, Nq, Hq, _ = q.shape
    cap, Hkv = kc.shape[1], kc.shape[2]
    n_new = 0 if k_new is None else Nq
    O = np.zeros((B, Nq, Hq, vc.shape[3]))
    L = np.zeros((B, Hq, Nq))
    for b in range(B):
        base = min(max(int(seqlens[b]), 0), cap)
        for i in range(n_new):
            if base + i < cap:
                kc[b, base + i] = _f64(k_new)[b, i]
                vc[b, base + i] = _f64(v_new)[b, i]
        n = base + n_new
        avail = min(n, cap)
        j = np.arange(avail)
        mask = np.ones((Nq, avail), dtype=bool)
        if causal:
            mask &= j[None, :] <= (n - Nq + np.arange(Nq))[:, None]
        for hq in range(Hq):
            kv = kv_head_of(hq, Hq, Hkv)
            P, lse = softmax_rows(scores(q[b, :, hq], kc[b, :avail, kv], scale), mask)
            O[b, :, hq] = P @ vc[b, :avail, kv]
            L[b, hq] = lse
    return kc, vc, O, L


def attention_backward_window(q, k, v, do, window_left, window_right, scale):
    """Gradients of ``attention_window``: dq (B, Nq, Hq, d), dk and dv
    (B, Nk, Hkv, d) in float64.

    The chain rule of ``attention_backward_rows`` applied under the
    bottom-right aligned window of ``window_mask`` (pyshine.com code tour:
    bottom-right causal since 2.1, sliding windows since 2.3). A query that
    sees no key has P = 0 in its row, so it contributes no gradient.
    """
    q, k, v, do = (np.asarray(x) for x in (q, k, v, do))
    B, Nq, Hq, _ = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    mask = window_mask(Nq, Nk, window_left, window_right)
    for b in range(B):
        for hq in range(Hq):
            kv = kv_head_of(hq, Hq, Hkv)
            Q, K, V = _f64(q[b, :, hq]), _f64(k[b, :, kv]), _f64(v[b, :, kv])
            dO = _f64(do[b, :, hq])
            P, _ = softmax_rows(scores(Q, K, scale), mask)
            dP = dO @ V.T
            dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
            dq[b, :, hq] = float(scale) * (dS @ K)
            dk[b, :, kv] += float(scale) * (dS.T @ Q)
            dv[b, :, kv] += P.T @ dO
    return dq, dk, dv


def attention_backward_varlen(q, k, v, do, cu_q, cu_k, window_left, window_right, scale):
    """Gradients of ``attention_varlen`` for packed q, do (total_q, Hq, d)
    and k, v (total_k, Hkv, d): each sequence's block is
    ``attention_backward_window`` of its own rows."""
    q, k, v, do = (np.asarray(x) for x in (q, k, v, do))
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(len(cu_q) - 1):
        qa, qb, ka, kb = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if qb == qa or kb == ka:
            continue
        gq, gk, gv = attention_backward_window(q[None, qa:qb], k[None, ka:kb], v[None, ka:kb], do[None, qa:qb],
                                               window_left, window_right, scale)
        dq[qa:qb] = gq[0]
        dk[ka:kb] = gk[0]
        dv[ka:kb] = gv[0]
    return dq, dk, dv
