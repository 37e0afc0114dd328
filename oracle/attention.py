"""float64 reference implementations (test infrastructure only; see the package docstring).

Sources, cited by page title and section:

* "FlashAttention" (shubhamtatvamasi.com, LLM inference course), opening display formula:
  O = softmax(Q K^T / sqrt(d) + M) V with an additive mask M.
* same page, "The trick: tiles and an online softmax": the running (m, l, O) update for a
  new tile of scores s with values v, and the final division O / l.
* same page, "Decode is a different problem": one query row per sequence against its whole
  K/V cache; partial (m, l, O) results of KV chunks are merged with the same rule.
* same page, "The FlashAttention family" table (the paged variants, which read K/V through
  a block table): the newest tokens of a sequence attend to its whole cached history.
* "FlashAttention, explained." (vibeengines.com), the worked example of the rescaling
  trick, and the forward-pass statement (Q, K, V are N x d per head, 1/sqrt(d) scale and
  masking fused, the statistics m and l are kept alongside O); its block-sparse section: a
  block mask over (query block, key block) pairs removes whole blocks of scores; its
  backward-pass section: the gradients are recomputed from Q, K, V with the saved m, l and
  D_i = rowsum(dO_i * O_i).

Conventions (readings of points the pages leave open):

* ``scale`` is passed explicitly (the pages use 1/sqrt(d)).
* causal: query i may attend key j iff j <= i (diagonal included); -inf elsewhere.
* GQA: query head h reads key/value head h // (Hq // Hkv).
* m is the row maximum of the scaled scores in natural-log units; l = sum_j exp(s_j - m).
* A row with no admissible key has O = 0, m = -inf, l = 0.
* Partials handed to :func:`merge` carry a normalised O_s (O_s = sum p v / l_s) with its
  (m_s, l_s); a partial with l_s = 0 carries no weight.
"""

from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _softmax_stats(s: np.ndarray, allowed: np.ndarray):
    """Safe softmax of each row of ``s`` restricted to ``allowed``.

    Subtract the row maximum before exponentiating, then divide by the row sum (the
    "safe" softmax the worked example on "FlashAttention, explained." starts from).
    Returns the unnormalised weights p = exp(s - m), the row maxima m and sums l.
    """
    s_masked = np.where(allowed, s, -np.inf)
    m = s_masked.max(axis=-1) if s.shape[-1] > 0 else np.full(s.shape[:-1], -np.inf)
    finite = np.isfinite(m)
    shift = np.where(finite, m, 0.0)
    p = np.where(allowed, np.exp(s_masked - shift[..., None]), 0.0)
    l = p.sum(axis=-1)
    return p, m, l


def attention_head(q, k, v, scale, causal, rows=None, row_block=256):
    """Exact attention for one head: O = softmax(scale * q k^T + M) v.

    q: [N, d]; k, v: [N_k, d]. ``rows`` selects query rows (default: all). The score matrix
    is materialised in full-width row blocks of ``row_block`` rows (every block sees all of
    its admissible keys; nothing is tiled over keys). Causal masking compares the query
    row index i with the key index j (j <= i admissible).

    Returns O [len(rows), d], m [len(rows)], l [len(rows)].
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    n_keys = k.shape[0]
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, v.shape[1]))
    m_out = np.full(rows.size, -np.inf)
    l_out = np.zeros(rows.size)
    for r0 in range(0, rows.size, row_block):
        idx = rows[r0:r0 + row_block]
        kend = min(n_keys, int(idx.max()) + 1) if causal and idx.size else n_keys
        s = scale * (q[idx] @ k[:kend].T)
        if causal:
            allowed = np.arange(kend)[None, :] <= idx[:, None]
        else:
            allowed = np.ones(s.shape, dtype=bool)
        p, m, l = _softmax_stats(s, allowed)
        num = p @ v[:kend]
        safe_l = np.where(l > 0, l, 1.0)
        out[r0:r0 + idx.size] = np.where(l[:, None] > 0, num / safe_l[:, None], 0.0)
        m_out[r0:r0 + idx.size] = m
        l_out[r0:r0 + idx.size] = l
    return out, m_out, l_out


def attention(q, k, v, scale, causal, row_block=256):
    """Exact multi-head attention over [B, H, N, d] tensors.

    q: [B, Hq, N, d]; k, v: [B, Hkv, N, d] with Hq % Hkv == 0; query head h reads key/value
    head h // (Hq // Hkv). Returns O [B, Hq, N, d], m [B, Hq, N], l [B, Hq, N], float64.
    """
    q = _f64(q)
    b_, hq, n, d = q.shape
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = hq // hkv
    out = np.zeros((b_, hq, n, v.shape[-1]))
    m = np.zeros((b_, hq, n))
    l = np.zeros((b_, hq, n))
    for b in range(b_):
        for h in range(hq):
            kh = h // group
            out[b, h], m[b, h], l[b, h] = attention_head(
                q[b, h], k[b, kh], v[b, kh], scale, causal, row_block=row_block)
    return out, m, l


def attention_probs(q, k, scale, causal):
    """The normalised probability matrix P = softmax(scale * q k^T + M) for one head.

    Only for small inputs: it returns the full [N, N_k] matrix.
    """
    q = _f64(q)
    k = _f64(k)
    s = scale * (q @ k.T)
    if causal:
        allowed = np.arange(k.shape[0])[None, :] <= np.arange(q.shape[0])[:, None]
    else:
        allowed = np.ones(s.shape, dtype=bool)
    p, _, l = _softmax_stats(s, allowed)
    safe_l = np.where(l > 0, l, 1.0)
    return np.where(l[:, None] > 0, p / safe_l[:, None], 0.0)


def decode(q, k_seqs, v_seqs, scale):
    """Single-query decode attention over each sequence's whole (logical) K/V.

    q: [B, Hq, d]; k_seqs[b], v_seqs[b]: [Hkv, L_b, d] (the logical, unpaged cache of
    sequence b). The one query of a sequence is its newest token, so every one of its L_b
    keys is admissible. Returns O [B, Hq, d], m [B, Hq], l [B, Hq].
    """
    q = _f64(q)
    b_, hq, d = q.shape
    out = np.zeros((b_, hq, d))
    m = np.full((b_, hq), -np.inf)
    l = np.zeros((b_, hq))
    for b in range(b_):
        kb = _f64(k_seqs[b])
        vb = _f64(v_seqs[b])
        group = hq // kb.shape[0]
        for h in range(hq):
            o_bh, m_bh, l_bh = attention_head(
                q[b, h][None, :], kb[h // group], vb[h // group], scale, causal=False)
            out[b, h], m[b, h], l[b, h] = o_bh[0], m_bh[0], l_bh[0]
    return out, m, l


def prefill_paged(q, k_seqs, v_seqs, scale, causal, row_block=256, q_lens=None):
    """Attention of each sequence's newest query rows against its whole (logical) K/V.

    q: [B, Hq, Nq, d]; k_seqs[b], v_seqs[b]: [Hkv, L_b, d]; q_lens: optional per-sequence
    query counts n_b <= Nq (default: Nq for every sequence). The n_b queries of sequence b are
    its last n_b tokens, in rows 0 .. n_b - 1: query i sits at position pos_i = L_b - n_b + i,
    so the causal mask admits key j iff j <= pos_i (the diagonal aligned to the bottom right of
    the L_b x n_b score block); without the mask every j < L_b is admissible. A query with no
    admissible key (pos_i < 0 when n_b > L_b, or L_b = 0) has O = 0, m = -inf, l = 0. Rows
    i >= n_b are not queries: they come back as O = 0, m = -inf, l = 0. S and P are
    materialised in full-width blocks of ``row_block`` rows over all L_b keys.

    Returns O [B, Hq, Nq, d], m [B, Hq, Nq], l [B, Hq, Nq], float64.
    """
    q = _f64(q)
    b_, hq, nq_all, d = q.shape
    out = np.zeros((b_, hq, nq_all, d))
    m_out = np.full((b_, hq, nq_all), -np.inf)
    l_out = np.zeros((b_, hq, nq_all))
    for b in range(b_):
        kb = _f64(k_seqs[b])
        vb = _f64(v_seqs[b])
        n_keys = kb.shape[1]
        group = hq // kb.shape[0]
        nq = nq_all if q_lens is None else int(min(max(int(q_lens[b]), 0), nq_all))
        pos = n_keys - nq + np.arange(nq)
        for h in range(hq):
            for r0 in range(0, nq, row_block):
                rows = slice(r0, min(nq, r0 + row_block))
                s = scale * (q[b, h, rows] @ kb[h // group].T)
                if causal:
                    allowed = np.arange(n_keys)[None, :] <= pos[rows, None]
                else:
                    allowed = np.ones(s.shape, dtype=bool)
                p, m, l = _softmax_stats(s, allowed)
                safe_l = np.where(l > 0, l, 1.0)
                num = p @ vb[h // group]
                out[b, h, rows] = np.where(l[:, None] > 0, num / safe_l[:, None], 0.0)
                m_out[b, h, rows] = m
                l_out[b, h, rows] = l
    return out, m_out, l_out


def attention_block_sparse(q, k, v, scale, causal, block_offsets, block_indices, block_q,
                           block_k, row_block=256):
    """Exact attention restricted by a block mask.

    q: [B, Hq, N, d]; k, v: [B, Hkv, N, d]. Query i and key j of head (b, h) may attend iff
    key block j // block_k is listed for query block i // block_q of that head and, when
    ``causal``, j <= i. The lists are compressed rows: the key blocks of query block qb of
    head (b, h) are block_indices[block_offsets[r] : block_offsets[r + 1]] with
    r = (b * Hq + h) * ceil(N / block_q) + qb. Indices outside [0, ceil(N / block_k)) name no
    key. Everything else is the definition: O = softmax(scale * q k^T + M) v with M = -inf
    outside the admitted set; a row with no admissible key has O = 0, m = -inf, l = 0.
    S and P are materialised in full-width blocks of ``row_block`` rows.

    Returns O [B, Hq, N, d], m [B, Hq, N], l [B, Hq, N], float64.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    b_, hq, n, d = q.shape
    group = hq // k.shape[1]
    nqb = -(-n // block_q)
    nkb = -(-n // block_k)
    offsets = np.asarray(block_offsets, dtype=np.int64)
    indices = np.asarray(block_indices, dtype=np.int64)
    out = np.zeros((b_, hq, n, d))
    m_out = np.full((b_, hq, n), -np.inf)
    l_out = np.zeros((b_, hq, n))
    key_block = np.arange(n) // block_k
    for b in range(b_):
        for h in range(hq):
            # admitted (query block, key block) pairs of this head
            blocks = np.zeros((nqb, nkb), dtype=bool)
            for qb in range(nqb):
                r = (b * hq + h) * nqb + qb
                sel = indices[offsets[r]:offsets[r + 1]]
                sel = sel[(sel >= 0) & (sel < nkb)]
                blocks[qb, sel] = True
            kh = h // group
            for r0 in range(0, n, row_block):
                rows = np.arange(r0, min(n, r0 + row_block))
                s = scale * (q[b, h, rows] @ k[b, kh].T)
                allowed = blocks[rows // block_q][:, key_block]
                if causal:
                    allowed &= np.arange(n)[None, :] <= rows[:, None]
                p, m, l = _softmax_stats(s, allowed)
                safe_l = np.where(l > 0, l, 1.0)
                num = p @ v[b, kh]
                out[b, h, rows] = np.where(l[:, None] > 0, num / safe_l[:, None], 0.0)
                m_out[b, h, rows] = m
                l_out[b, h, rows] = l
    return out, m_out, l_out


def attention_backward(q, k, v, dout, scale, causal):
    """Gradients of O = softmax(scale * q k^T + M) v with respect to q, k and v.

    q, dout: [B, Hq, N, d]; k, v: [B, Hkv, N, d]. Per head, with P the normalised
    probabilities and D_i = sum_c dO_ic O_ic:
        dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   dQ = scale dS K,   dK = scale dS^T Q
    (the chain rule through the row-wise softmax: dS_ij = P_ij (dP_ij - sum_t P_it dP_it), and
    sum_t P_it dP_it = D_i). A key/value head shared by several query heads receives the sum
    of their gradients. P is materialised in full for each head (small inputs only).

    Returns dQ [B, Hq, N, d], dK [B, Hkv, N, d], dV [B, Hkv, N, d], float64.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    dout = _f64(dout)
    b_, hq, n, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    dq = np.zeros_like(q)
    dk = np.zeros((b_, hkv, n, d))
    dv = np.zeros((b_, hkv, n, v.shape[-1]))
    for b in range(b_):
        for h in range(hq):
            kh = h // group
            p = attention_probs(q[b, h], k[b, kh], scale, causal)
            o = p @ v[b, kh]
            dvv = p.T @ dout[b, h]
            dp = dout[b, h] @ v[b, kh].T
            dd = (dout[b, h] * o).sum(axis=1)
            ds = p * (dp - dd[:, None])
            dq[b, h] = scale * (ds @ k[b, kh])
            dk[b, kh] += scale * (ds.T @ q[b, h])
            dv[b, kh] += dvv
    return dq, dk, dv


def merge(o_parts, m_parts, l_parts):
    """Merge S partial results over disjoint key sets into one.

    o_parts: [S, R, d] normalised partial outputs; m_parts, l_parts: [S, R]. With
    m = max_s m_s and w_s = l_s * exp(m_s - m): l = sum_s w_s and O = sum_s w_s O_s / l.
    This is the online-softmax rescale of "The trick: tiles and an online softmax" applied
    to whole partials, as "Decode is a different problem" prescribes for split KV chunks.
    Returns O [R, d], m [R], l [R]; a row whose partials are all empty gives O = 0,
    m = -inf, l = 0.
    """
    o_parts = _f64(o_parts)
    m_parts = _f64(m_parts)
    l_parts = _f64(l_parts)
    live = l_parts > 0
    m = np.where(live, m_parts, -np.inf).max(axis=0)
    shift = np.where(np.isfinite(m), m, 0.0)
    w = np.where(live, l_parts * np.exp(np.where(live, m_parts, 0.0) - shift[None, :]), 0.0)
    l = w.sum(axis=0)
    num = (w[:, :, None] * np.where(live[:, :, None], o_parts, 0.0)).sum(axis=0)
    safe_l = np.where(l > 0, l, 1.0)
    out = np.where(l[:, None] > 0, num / safe_l[:, None], 0.0)
    return out, m, l


def online_softmax(score_blocks, value_blocks):
    """The running (m, l, O) recurrence, one tile of scores at a time, in float64.

    For each tile of scores s (shape [T]) with values v (shape [T, d]), following the
    update rule of "The trick: tiles and an online softmax":
        m' = max(m, max_j s_j)
        l' = l * exp(m - m') + sum_j exp(s_j - m')
        O' = O * exp(m - m') + sum_j exp(s_j - m') v_j
    and the result is O / l. Starts from m = -inf, l = 0, O = 0.

    Returns (O / l, m, l, trace) where trace lists (m, l) after every tile. This models
    how the tiled kernels reach the oracle's result; tests use it to pin the recurrence
    against the pages' worked example and against :func:`attention_head`.
    """
    m = -np.inf
    l = 0.0
    acc = None
    trace = []
    for s, v in zip(score_blocks, value_blocks):
        s = _f64(s)
        v = _f64(v)
        if acc is None:
            acc = np.zeros(v.shape[1:])
        if s.size == 0:
            trace.append((m, l))
            continue
        m_new = max(m, float(s.max()))
        if m_new == -np.inf:
            trace.append((m, l))
            continue
        alpha = np.exp(m - m_new) if m != -np.inf else 0.0
        e = np.exp(s - m_new)
        l = l * alpha + e.sum()
        acc = acc * alpha + e @ v
        m = m_new
        trace.append((m, l))
    if acc is None or l == 0.0:
        return (np.zeros_like(acc) if acc is not None else None), m, l, trace
    return acc / l, m, l, trace
