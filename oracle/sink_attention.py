"""Plain fp64 CPU oracle for attention with a learnable per-head sink logit.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Every function takes
NumPy arrays (bf16 inputs arrive as their exact float values), upcasts them to
float64 and returns float64 (or int64 for index work).  Nothing here is
blocked, fused or reordered beyond the definition it states.

Sources (web pages; cited by title and section):
  [FA-sink]  flash-attention PR #1819 "feat: Implement Sink Attention",
             section "Description": the sink is a tensor of shape (nheads,),
             one learnable value per head, entered as an extra logit into the
             attention scores before the softmax; the backward pass returns
             its gradient.
  [trtllm]   sglang PR #8825 "feat: openai oss attention sink support with
             trtllm-gen backend", bot "Summary of Changes": the sink is an
             additional per-head value in the softmax denominator; it is None
             when the layer has no sink; decode and extend both receive it.
  [window]   sglang PR #12504 "To implement attention-sink": "Motivation"
             (keep a first window of 1024 and a last window of 7168 tokens),
             "Modifications" (the page table becomes the first-window slice
             followed by the last-window slice), the bot "Code Review" (the
             window applies only when the sequence is longer than 1024+7168;
             otherwise the whole prefix is used; the kernel length becomes
             1024+7168) and the maintainer's comment that the last 7168 tokens
             are kept for each sequence.

  [dsa]      "SGLang dsa" (s1mplewind blog), sections "layer0" and "Other
             Layers": the lightning indexer selects, per query, a list of KV
             entries (sink-like absolute positions plus relative/local ones);
             the lists of 128 adjacent queries overlap by about a third of
             their size; the first 2048 tokens are attended densely.

Readings where the pages are silent (each also listed in the design doc):
  * the sink is in the units of the already-scaled scores (not multiplied by
    the softmax scale), indexed by query head;
  * "no sink" (None) is the same as a sink of -inf;
  * LSE is the natural log of the full softmax denominator, sink included;
  * causal masking is bottom-right aligned: query row i of Sq sits at
    absolute key position Sk - Sq + i;
  * the first/last window keeps key j for query position p iff
    j < W1 or j > p - W2 (with j <= p); this reproduces both branches of the
    page's selection code for every length;
  * GQA: query head h reads KV head h // (Hq / Hkv);
  * a row that sees no key and has no sink gets O = 0, LSE = -inf;
  * extend (chunked prefill): a sequence's new tokens are the last nq of its
    L cached tokens, so new token i sits at position L - nq + i and sees keys
    by the prefill rule above, the window included (the pages define the
    window for decode only; the per-query rule is its prefill form).
  * index-list selection: one list of token positions serves a block of
    block_q consecutive query rows of a sequence; a row attends to the
    listed tokens at or before its own position (plus the sink); entries
    < 0 or >= L are empty slots; a list names each token at most once;
  * variable-length (packed) forward and backward: each sequence is its own
    attention problem with its own Sq and Sk (bottom-right causal inside the
    sequence); no key of one sequence is visible to a query of another; the
    sink gradient sums over all sequences' rows.

Parity status: every function below is pinned by tests that do not retype
its formula (closed forms, library special cases, brute force, finite
differences, the page's own slicing rule); see tests/test_oracle_*.py.
"""

import math

import numpy as np

NEG_INF = float("-inf")


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _sink_vector(sink, Hq):
    # [trtllm] Summary: the sink is None when the layer has none -> -inf.
    if sink is None:
        return np.full(Hq, NEG_INF, dtype=np.float64)
    s = _f64(sink)
    assert s.shape == (Hq,), "sink must have shape (nheads,) [FA-sink]"
    return s


def visible(i, j, Sq, Sk, causal, window):
    """Is key j visible to query row i?  (scalar form, used by brute force)

    Causal: bottom-right alignment, query i at position p = Sk - Sq + i.
    Window (W1, W2): [window] Code Review keeps the first W1 tokens and the
    last W2 tokens ending at the current one, i.e. j < W1 or j > p - W2.
    """
    p = Sk - Sq + i
    if causal and j > p:
        return False
    if window is not None:
        w1, w2 = window
        if not (j < w1 or j > p - w2):
            return False
    return True


def _visible_matrix(pos, nkeys, causal, window):
    """Vectorised `visible` for query positions `pos` against keys 0..nkeys-1."""
    j = np.arange(nkeys)[None, :]
    p = np.asarray(pos)[:, None]
    ok = np.ones((len(pos), nkeys), dtype=bool)
    if causal:
        ok &= j <= p
    if window is not None:
        w1, w2 = window
        ok &= (j < w1) | (j > p - w2)
    return ok


def prefill(q, k, v, sink, scale, causal=True, window=None, row_block=1024):
    """Sink-attention forward.  q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D], sink [Hq]|None.

    For query head h (KV head h // g) and row i with visible key set V_i:
        s_ij = scale * <q_i, k_j>
        Z_i  = exp(sink_h) + sum_{j in V_i} exp(s_ij)     [FA-sink], [trtllm]
        O_i  = sum_{j in V_i} exp(s_ij) v_j / Z_i          (sink has no value row)
        LSE_i = ln Z_i
    evaluated with the usual max shift m_i = max(sink_h, max_j s_ij).
    Returns (o [B,Sq,Hq,D], lse [B,Hq,Sq]) in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, _ = k.shape
    assert Hq % Hkv == 0
    g = Hq // Hkv
    sig = _sink_vector(sink, Hq)
    o = np.zeros((B, Sq, Hq, D))
    lse = np.full((B, Hq, Sq), NEG_INF)
    for b in range(B):
        for h in range(Hq):
            K = k[b, :, h // g, :]
            V = v[b, :, h // g, :]
            for i0 in range(0, Sq, row_block):
                i1 = min(Sq, i0 + row_block)
                pos = Sk - Sq + np.arange(i0, i1)
                # keys past the last row's causal bound are masked for the
                # whole block; leaving them out changes no value
                nk = Sk if not causal else max(0, min(Sk, int(pos[-1]) + 1))
                s = scale * (q[b, i0:i1, h, :] @ K[:nk].T)
                s = np.where(_visible_matrix(pos, nk, causal, window), s, NEG_INF)
                rowmax = s.max(axis=1) if nk > 0 else np.full(i1 - i0, NEG_INF)
                m = np.maximum(sig[h], rowmax)
                live = np.isfinite(m)
                mm = np.where(live, m, 0.0)
                e = np.where(np.isfinite(s), np.exp(s - mm[:, None]), 0.0)
                z = np.exp(sig[h] - mm) + e.sum(axis=1)
                out = (e @ V[:nk]) / np.where(live, z, 1.0)[:, None]
                o[b, i0:i1, h, :] = np.where(live[:, None], out, 0.0)
                lse[b, h, i0:i1] = np.where(live, mm + np.log(np.where(live, z, 1.0)), NEG_INF)
    return o, lse


def prefill_bruteforce(q, k, v, sink, scale, causal=True, window=None):
    """The same definition written as scalar loops; for tiny inputs only."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, _ = k.shape
    g = Hq // Hkv
    sig = _sink_vector(sink, Hq)
    o = np.zeros((B, Sq, Hq, D))
    lse = np.full((B, Hq, Sq), NEG_INF)
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            for i in range(Sq):
                logits = []
                rows = []
                for j in range(Sk):
                    if visible(i, j, Sq, Sk, causal, window):
                        dot = 0.0
                        for d in range(D):
                            dot += q[b, i, h, d] * k[b, j, kh, d]
                        logits.append(scale * dot)
                        rows.append(j)
                m = max([sig[h]] + logits)
                if m == NEG_INF:
                    continue
                z = math.exp(sig[h] - m) if sig[h] != NEG_INF else 0.0
                acc = [0.0] * D
                for s, j in zip(logits, rows):
                    e = math.exp(s - m)
                    z += e
                    for d in range(D):
                        acc[d] += e * v[b, j, kh, d]
                for d in range(D):
                    o[b, i, h, d] = acc[d] / z
                lse[b, h, i] = m + math.log(z)
    return o, lse


def select_tokens(L, window):
    """Logical KV selection of one sequence of length L (current token included).

    [window] Code Review: if L > W1 + W2 keep tokens [0, W1) followed by
    [L - W2, L); otherwise keep the whole prefix [0, L).  The maintainer asks
    for this per sequence, so L is the sequence's own length.
    """
    L = int(L)
    if window is None:
        return np.arange(L, dtype=np.int64)
    w1, w2 = window
    if L <= w1 + w2:
        return np.arange(L, dtype=np.int64)
    return np.concatenate([np.arange(w1, dtype=np.int64),
                           np.arange(L - w2, L, dtype=np.int64)])


def select_slots(block_table, seqlens, page_size, window):
    """Physical KV slots of the selected tokens, per sequence (list of int64 arrays).

    Token t of sequence b lives in page block_table[b, t // P] at offset t % P,
    i.e. slot = block_table[b, t // P] * P + t % P ([window] Code Review maps
    token positions to KV slots through the request's token table; with page
    size P the table holds one entry per page).
    """
    bt = np.asarray(block_table, dtype=np.int64)
    out = []
    for b, L in enumerate(np.asarray(seqlens).tolist()):
        t = select_tokens(L, window)
        out.append(bt[b, t // page_size] * page_size + t % page_size)
    return out


def gather_kv(k_cache, v_cache, block_table, seqlens, page_size, window):
    """Rows of the paged caches [num_pages, P, Hkv, D] at the selected slots."""
    nP, P, Hkv, D = k_cache.shape
    assert P == page_size
    kf = np.asarray(k_cache).reshape(nP * P, Hkv, D)
    vf = np.asarray(v_cache).reshape(nP * P, Hkv, D)
    ks, vs = [], []
    for slots in select_slots(block_table, seqlens, page_size, window):
        ks.append(kf[slots])
        vs.append(vf[slots])
    return ks, vs


def decode_paged(q, k_cache, v_cache, block_table, seqlens, sink, scale, window=None):
    """One new query token per sequence against its paged KV cache.

    q [B,Hq,D]; the current token's K/V is already in the cache and counted in
    seqlens.  The selected rows (all of them visible to the newest token) are
    gathered and the forward definition is applied to them.
    [trtllm] Summary: the decode path receives the same sink.
    Returns (o [B,Hq,D], lse [B,Hq]).
    """
    q = _f64(q)
    B, Hq, D = q.shape
    ks, vs = gather_kv(k_cache, v_cache, block_table, seqlens, k_cache.shape[1], window)
    o = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        ob, lb = prefill(q[b][None, None], ks[b][None], vs[b][None], sink, scale,
                         causal=False, window=None)
        o[b] = ob[0, 0]
        lse[b] = lb[0, :, 0]
    return o, lse


def extend_paged(q, cu_seqlens_q, k_cache, v_cache, block_table, seqlens, sink, scale,
                 window=None):
    """Chunked prefill (extend): packed new queries against a paged KV cache.

    The extend path receives the same sink as decode ([trtllm] Summary of
    Changes), and the variable-length functions take it too ([FA-sink]
    Description).  Sequence b's queries are rows cu_seqlens_q[b] ..
    cu_seqlens_q[b+1]-1 of q [total_q, Hq, D].  They are the last nq_b tokens
    of a context of L_b = seqlens[b] tokens whose K/V (theirs included) are
    already in the cache, so query i of b sits at position L_b - nq_b + i and
    sees keys by the prefill rule: bottom-right causal and, with a window, the
    first W1 and last W2 positions relative to itself.
    Returns (o [total_q, Hq, D], lse [Hq, total_q]).
    """
    q = _f64(q)
    total, Hq, D = q.shape
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    ks, vs = gather_kv(k_cache, v_cache, block_table, seqlens, k_cache.shape[1], None)
    o = np.zeros((total, Hq, D))
    lse = np.full((Hq, total), NEG_INF)
    for b in range(len(ks)):
        a, e = int(cu[b]), int(cu[b + 1])
        if e == a:
            continue
        ob, lb = prefill(q[a:e][None], ks[b][None], vs[b][None], sink, scale, causal=True,
                         window=window)
        o[a:e] = ob[0]
        lse[:, a:e] = lb[0]
    return o, lse


def backward(q, k, v, sink, dout, scale, causal=True, window=None, row_block=1024):
    """Gradients of L = sum(dout * O) for the forward above.

    With P_ij = exp(s_ij - LSE_i) (sink-inclusive LSE) and Di = <dO_i, O_i>:
        dV_j  = sum_{h in group, i} P_ij dO_i
        dS_ij = P_ij (<dO_i, v_j> - Di)
        dQ_i  = scale * sum_j dS_ij k_j
        dK_j  = scale * sum_{h in group, i} dS_ij q_i
        dSink_h = -sum_{b,i} exp(sink_h - LSE_i) Di
    The last line follows from dO_i/dsink = -exp(sink - LSE_i) O_i
    ([FA-sink] Description: the backward returns the sink's gradient).
    Returns (dq, dk, dv, dsink, o, lse), float64.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, _ = k.shape
    g = Hq // Hkv
    sig = _sink_vector(sink, Hq)
    o, lse = prefill(q, k, v, sink, scale, causal, window, row_block)
    di = np.einsum("bshd,bshd->bhs", dout, o)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dsink = np.zeros(Hq)
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            K = k[b, :, kh, :]
            V = v[b, :, kh, :]
            for i0 in range(0, Sq, row_block):
                i1 = min(Sq, i0 + row_block)
                pos = Sk - Sq + np.arange(i0, i1)
                nk = Sk if not causal else max(0, min(Sk, int(pos[-1]) + 1))
                L = lse[b, h, i0:i1]
                live = np.isfinite(L)
                Ls = np.where(live, L, 0.0)
                s = scale * (q[b, i0:i1, h, :] @ K[:nk].T)
                vis = _visible_matrix(pos, nk, causal, window) & live[:, None]
                p = np.where(vis, np.exp(np.where(vis, s, 0.0) - Ls[:, None]), 0.0)
                dO = dout[b, i0:i1, h, :]
                dv[b, :nk, kh, :] += p.T @ dO
                dp = dO @ V[:nk].T
                ds = p * (dp - di[b, h, i0:i1][:, None])
                dq[b, i0:i1, h, :] = scale * (ds @ K[:nk])
                dk[b, :nk, kh, :] += scale * (ds.T @ q[b, i0:i1, h, :])
            if np.isfinite(sig[h]):
                L = lse[b, h, :]
                psink = np.where(np.isfinite(L), np.exp(sig[h] - np.where(np.isfinite(L), L, 0.0)), 0.0)
                dsink[h] -= np.sum(psink * di[b, h, :])
    return dq, dk, dv, dsink, o, lse


def _cu(cu):
    cu = np.asarray(cu, dtype=np.int64)
    assert cu[0] == 0 and np.all(np.diff(cu) >= 0), "cu_seqlens must start at 0 and not decrease"
    return cu


def prefill_varlen(q, cu_seqlens_q, k, v, cu_seqlens_k, sink, scale, causal=True, window=None):
    """Packed variable-length forward ([FA-sink] Description: the variable-
    length counterparts take the sink too).

    q [total_q, Hq, D], k/v [total_k, Hkv, D].  Sequence b owns query rows
    cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows cu_seqlens_k[b] ..
    cu_seqlens_k[b+1]-1 and is the prefill problem on those slices alone.
    Returns (o [total_q, Hq, D], lse [Hq, total_q]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    cq, ck = _cu(cu_seqlens_q), _cu(cu_seqlens_k)
    assert len(cq) == len(ck) and cq[-1] == q.shape[0] and ck[-1] == k.shape[0]
    total, Hq, D = q.shape
    o = np.zeros((total, Hq, D))
    lse = np.full((Hq, total), NEG_INF)
    for b in range(len(cq) - 1):
        a, e = int(cq[b]), int(cq[b + 1])
        if e == a:
            continue
        ka, ke = int(ck[b]), int(ck[b + 1])
        ob, lb = prefill(q[a:e][None], k[ka:ke][None], v[ka:ke][None], sink, scale, causal,
                         window)
        o[a:e] = ob[0]
        lse[:, a:e] = lb[0]
    return o, lse


def backward_varlen(q, cu_seqlens_q, k, v, cu_seqlens_k, sink, dout, scale, causal=True,
                    window=None):
    """Gradients of L = sum(dout * O) for prefill_varlen ([FA-sink]
    Description: the backward returns the sink's gradient).

    The sequences share no score, so each sequence's dq, dk, dv are the
    backward above on its own slices, and dsink is the sum of the
    per-sequence sink gradients.
    Returns (dq, dk, dv, dsink, o [total_q, Hq, D], lse [Hq, total_q]).
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    cq, ck = _cu(cu_seqlens_q), _cu(cu_seqlens_k)
    assert len(cq) == len(ck) and cq[-1] == q.shape[0] and ck[-1] == k.shape[0]
    total, Hq, D = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dsink = np.zeros(Hq)
    o = np.zeros((total, Hq, D))
    lse = np.full((Hq, total), NEG_INF)
    for b in range(len(cq) - 1):
        a, e = int(cq[b]), int(cq[b + 1])
        ka, ke = int(ck[b]), int(ck[b + 1])
        if e == a:
            continue  # no query row: no score, every gradient of the slice is 0
        r = backward(q[a:e][None], k[ka:ke][None], v[ka:ke][None], sink, dout[a:e][None], scale,
                     causal, window)
        dq[a:e], dk[ka:ke], dv[ka:ke] = r[0][0], r[1][0], r[2][0]
        dsink += r[3]
        o[a:e] = r[4][0]
        lse[:, a:e] = r[5][0]
    return dq, dk, dv, dsink, o, lse


def _attend(s, sig, V):
    """Softmax with the sink over masked logits s [rows, n] (-inf = not
    visible) and values V [n, D]; the same definition as prefill's."""
    rowmax = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], NEG_INF)
    m = np.maximum(sig, rowmax)
    live = np.isfinite(m)
    mm = np.where(live, m, 0.0)
    e = np.where(np.isfinite(s), np.exp(s - mm[:, None]), 0.0)
    z = np.exp(sig - mm) + e.sum(axis=1)
    o = np.where(live[:, None], (e @ V) / np.where(live, z, 1.0)[:, None], 0.0)
    lse = np.where(live, mm + np.log(np.where(live, z, 1.0)), NEG_INF)
    return o, lse


def index_paged(q, cu_seqlens_q, k_cache, v_cache, block_table, seqlens, kv_index, cu_blocks,
                block_q, sink, scale):
    """Sink attention over per-query-block KV index lists ([dsa] layer0,
    Other Layers; the sink as in [trtllm] Summary of Changes).

    Sequence b's new queries are rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
    of q [total_q, Hq, D], the last nq_b of its L_b = seqlens[b] cached tokens
    (row i at position p = L_b - nq_b + i).  Row i reads list
    kv_index[cu_blocks[b] + i // block_q] (token positions; entries < 0 or
    >= L_b are empty) and attends to its tokens t <= p.
    Returns (o [total_q, Hq, D], lse [Hq, total_q]).
    """
    q = _f64(q)
    total, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    g = Hq // Hkv
    sig = _sink_vector(sink, Hq)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    cb = np.asarray(cu_blocks, dtype=np.int64)
    idx_all = np.asarray(kv_index, dtype=np.int64)
    ks, vs = gather_kv(k_cache, v_cache, block_table, seqlens, k_cache.shape[1], None)
    ks, vs = [_f64(x) for x in ks], [_f64(x) for x in vs]
    o = np.zeros((total, Hq, D))
    lse = np.full((Hq, total), NEG_INF)
    for b in range(len(ks)):
        a, e = int(cu[b]), int(cu[b + 1])
        nq, L = e - a, len(ks[b])
        for i0 in range(0, nq, block_q):
            i1 = min(nq, i0 + block_q)
            idx = idx_all[cb[b] + i0 // block_q]
            idx = idx[(idx >= 0) & (idx < L)]
            pos = L - nq + np.arange(i0, i1)
            vis = idx[None, :] <= pos[:, None]
            for h in range(Hq):
                K = ks[b][idx, h // g, :]
                V = vs[b][idx, h // g, :]
                sc = np.where(vis, scale * (q[a + i0:a + i1, h, :] @ K.T), NEG_INF)
                o[a + i0:a + i1, h, :], lse[h, a + i0:a + i1] = _attend(sc, sig[h], V)
    return o, lse
