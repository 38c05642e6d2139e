"""Plain fp64 attention: the definition, the chunked running-max method, and
the textbook gradient. TEST INFRASTRUCTURE ONLY (see the package docstring).

Shapes: q, k, v, do are float arrays of shape [..., n, d] (any number of
leading batch/head axes, identical across the four). Every computation is in
float64. No function here blocks, fuses or reorders arithmetic beyond what
its docstring states.
"""

import math

import numpy as np


def softmax_scale(d):
    """The score scale 1/sqrt(d_k).

    "Fast and memory-efficient exact attention 分析", section 数学表达形式:
    scores are QK^T divided by the square root of the key dimension d_k.
    Here d_k is the common head dimension of Q and K.
    """
    return 1.0 / math.sqrt(float(d))


def _as_slices(x):
    x = np.asarray(x, dtype=np.float64)
    if x.ndim < 2:
        raise ValueError("expected [..., n, d]")
    lead = x.shape[:-2]
    return x.reshape((int(np.prod(lead, dtype=np.int64)),) + x.shape[-2:]), lead


def naive_fwd(q, k, v, rows=None, row_block=1024):
    """Standard attention O = softmax(Q K^T / sqrt(d)) V, written out.

    Follows the definition: "Fast and memory-efficient exact attention 分析",
    section 数学表达形式, and "当注意力成为瓶颈…", section 平方级的诅咒
    (S = QK^T, then a softmax over each row of S, then O = PV; each row is
    normalised over all keys).

    For every query row i:
        s_ij = (q_i . k_j) / sqrt(d)
        m_i  = max_j s_ij                (the textbook stable softmax: the
                                          row max is subtracted before exp,
                                          which leaves the softmax unchanged)
        p_ij = exp(s_ij - m_i)
        l_i  = sum_j p_ij
        o_i  = (sum_j p_ij v_j) / l_i

    Rows are independent by definition, so they are evaluated in blocks of
    ``row_block`` query rows only to bound memory; ``rows`` (an index array)
    restricts the result to those query rows. Returns (o, m, l) with
    o: [..., r, d], m and l: [..., r] where r = number of rows evaluated.
    """
    q3, lead = _as_slices(q)
    k3, _ = _as_slices(k)
    v3, _ = _as_slices(v)
    G, n, d = q3.shape
    nk = k3.shape[1]
    idx = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    r = idx.shape[0]
    o = np.zeros((G, r, v3.shape[2]), dtype=np.float64)
    m = np.full((G, r), -np.inf, dtype=np.float64)
    l = np.zeros((G, r), dtype=np.float64)
    scale = softmax_scale(d)
    if nk == 0 or r == 0:
        return o.reshape(lead + o.shape[1:]), m.reshape(lead + (r,)), l.reshape(lead + (r,))
    for g in range(G):
        for b0 in range(0, r, row_block):
            sel = idx[b0:b0 + row_block]
            s = (q3[g, sel, :] @ k3[g].T) * scale
            mb = s.max(axis=1)
            p = np.exp(s - mb[:, None])
            lb = p.sum(axis=1)
            o[g, b0:b0 + len(sel)] = (p @ v3[g]) / lb[:, None]
            m[g, b0:b0 + len(sel)] = mb
            l[g, b0:b0 + len(sel)] = lb
    return o.reshape(lead + o.shape[1:]), m.reshape(lead + (r,)), l.reshape(lead + (r,))


def row_stats(q, k):
    """Per-row statistics of the softmax: m_i = max_j s_ij and
    l_i = sum_j exp(s_ij - m_i), with s_ij = q_i . k_j / sqrt(d).

    These are the running max and running sum of exponentiated scores that the
    method keeps per query ("Self-attention Does Not Need O(n^2) Memory",
    English digest, method bullets: a total weight accumulated with a tracked
    maximum), taken at the end of the key sweep. Returns (m, l), each [..., n].
    """
    q3, lead = _as_slices(q)
    k3, _ = _as_slices(k)
    G, n, d = q3.shape
    scale = softmax_scale(d)
    m = np.empty((G, n))
    l = np.empty((G, n))
    for g in range(G):
        s = (q3[g] @ k3[g].T) * scale
        m[g] = s.max(axis=1)
        l[g] = np.exp(s - m[g][:, None]).sum(axis=1)
    return m.reshape(lead + (n,)), l.reshape(lead + (n,))


def chunked_fwd(q, k, v, chunk=None):
    """The pages' method: keys and values in chunks, a running maximum, a
    running sum of exponentiated scores and a running weighted value sum per
    query, divided by the sum only once at the end.

    "Self-attention Does Not Need O(n^2) Memory": the abstract and the
    method sections (方法论, 方法详解; English digest method bullets) describe
    postponing the softmax normalisation to the end, keeping two accumulators
    (weighted value sum and total weight) with a tracked maximum for numerical
    stability, and splitting keys/values into chunks of about sqrt(n).
    "当注意力成为瓶颈…", section IO感知, gives the two-block merge
    (m = max of both block maxima; l and O combine the blocks re-based on m);
    applying it once per chunk, in order, gives the loop below.

    Starting from m = -inf, l = 0, acc = 0, for each key chunk c in order:
        s      = q k_c^T / sqrt(d)
        m_new  = max(m, max_j s_j)
        alpha  = exp(m - m_new)
        p      = exp(s - m_new)
        l      = alpha * l + sum_j p_j
        acc    = alpha * acc + p v_c
        m      = m_new
    and finally o = acc / l. ``chunk`` defaults to ceil(sqrt(n_keys)).
    Returns (o, m, l) like ``naive_fwd``.
    """
    q3, lead = _as_slices(q)
    k3, _ = _as_slices(k)
    v3, _ = _as_slices(v)
    G, n, d = q3.shape
    nk = k3.shape[1]
    if chunk is None:
        chunk = max(1, int(math.ceil(math.sqrt(max(nk, 1)))))
    scale = softmax_scale(d)
    o = np.zeros((G, n, v3.shape[2]))
    m_out = np.full((G, n), -np.inf)
    l_out = np.zeros((G, n))
    for g in range(G):
        m = np.full(n, -np.inf)
        l = np.zeros(n)
        acc = np.zeros((n, v3.shape[2]))
        for c0 in range(0, nk, chunk):
            s = (q3[g] @ k3[g, c0:c0 + chunk].T) * scale
            m_new = np.maximum(m, s.max(axis=1))
            alpha = np.exp(m - m_new)
            p = np.exp(s - m_new[:, None])
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v3[g, c0:c0 + chunk]
            m = m_new
        if nk > 0:
            o[g] = acc / l[:, None]
        m_out[g] = m
        l_out[g] = l
    return o.reshape(lead + o.shape[1:]), m_out.reshape(lead + (n,)), l_out.reshape(lead + (n,))


def single_query(qv, k, v):
    """One query, one key at a time, O(1) extra memory.

    "Self-attention Does Not Need O(n^2) Memory" (abstract; 方法详解; English
    digest method bullets): the score of each key is computed in turn and two
    running quantities are updated, the weighted sum of values v* and the sum
    of weights s*, both kept relative to the largest score m seen so far:
        s     = q . k_i / sqrt(d)
        m'    = max(m, s)
        v*    = v* exp(m - m') + v_i exp(s - m')
        s*    = s* exp(m - m') + exp(s - m')
        m     = m'
    The result v*/s* is formed once, after the last key. Pure Python over the
    keys (numpy only for the length-d vectors); for small inputs.
    qv: [d]; k, v: [n, d]. Returns (o [d], m, s*).
    """
    qv = np.asarray(qv, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    scale = softmax_scale(qv.shape[0])
    m = -math.inf
    vstar = np.zeros(v.shape[1])
    sstar = 0.0
    for i in range(k.shape[0]):
        s = float(qv @ k[i]) * scale
        m_new = max(m, s)
        decay = math.exp(m - m_new) if m != -math.inf else 0.0
        w = math.exp(s - m_new)
        vstar = vstar * decay + v[i] * w
        sstar = sstar * decay + w
        m = m_new
    return vstar / sstar, m, sstar


def naive_bwd(q, k, v, do, rows=None, cols=None, row_block=1024, o=None):
    """Gradients of the scalar L = sum(O * dO) with respect to Q, K and V.

    The pages state only that the method stays differentiable and that the
    backward pass recomputes chunk intermediates from a checkpoint instead of
    storing them ("Self-attention Does Not Need O(n^2) Memory", abstract;
    方法详解; English digest method bullets). They print no gradient formulas,
    so this is the textbook Jacobian of O = softmax(S) V, S = QK^T / sqrt(d):
        P      = softmax(S) (row-wise, as in ``naive_fwd``)
        dV     = P^T dO
        dP     = dO V^T
        D_i    = sum_j P_ij dP_ij
        dS     = P * (dP - D)           (elementwise; D broadcast over j)
        dQ     = dS K / sqrt(d)
        dK     = dS^T Q / sqrt(d)

    Query rows are visited in blocks of ``row_block`` (each row's softmax is
    complete within its block); dK and dV are sums over query rows and so are
    accumulated block by block. ``rows`` restricts dQ to those query rows and
    ``cols`` restricts dK, dV to those key rows (the full softmax is still
    formed for every query row that contributes; with an empty ``cols`` only
    the blocks holding requested rows are visited). Returns (dq, dk, dv).

    ``o``: a forward output to form the row term from, D_i = dO_i . o_i, in
    place of sum_j P_ij dP_ij. The two agree when ``o`` is the exact output,
    since sum_j P_ij (dO_i . v_j) = dO_i . sum_j P_ij v_j. With a rounded
    output (the bf16 forward's), this is the row term that a backward fed
    that output computes.
    """
    q3, lead = _as_slices(q)
    k3, _ = _as_slices(k)
    v3, _ = _as_slices(v)
    do3, _ = _as_slices(do)
    o3 = None if o is None else _as_slices(o)[0]
    G, n, d = q3.shape
    nk = k3.shape[1]
    ridx = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    cidx = np.arange(nk) if cols is None else np.asarray(cols, dtype=np.int64)
    scale = softmax_scale(d)
    dq = np.zeros((G, ridx.shape[0], d))
    dk = np.zeros((G, cidx.shape[0], d))
    dv = np.zeros((G, cidx.shape[0], v3.shape[2]))
    if nk == 0 or n == 0:
        return (dq.reshape(lead + dq.shape[1:]), dk.reshape(lead + dk.shape[1:]),
                dv.reshape(lead + dv.shape[1:]))
    # position of each requested query row in the dq output
    want_row = np.full(n, -1, dtype=np.int64)
    want_row[ridx] = np.arange(ridx.shape[0])
    # with no key rows requested, blocks holding no requested query row add nothing
    only_rows = cidx.shape[0] == 0
    for g in range(G):
        for b0 in range(0, n, row_block):
            b1 = min(n, b0 + row_block)
            if only_rows and not (want_row[b0:b1] >= 0).any():
                continue
            s = (q3[g, b0:b1] @ k3[g].T) * scale
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dp = do3[g, b0:b1] @ v3[g].T
            if o3 is None:
                D = (p * dp).sum(axis=1, keepdims=True)
            else:
                D = (do3[g, b0:b1] * o3[g, b0:b1]).sum(axis=1, keepdims=True)
            ds = p * (dp - D)
            wr = want_row[b0:b1]
            hit = wr >= 0
            if hit.any():
                dq[g, wr[hit]] = (ds[hit] @ k3[g]) * scale
            dk[g] += (ds[:, cidx].T @ q3[g, b0:b1]) * scale
            dv[g] += p[:, cidx].T @ do3[g, b0:b1]
    return (dq.reshape(lead + dq.shape[1:]), dk.reshape(lead + dk.shape[1:]),
            dv.reshape(lead + dv.shape[1:]))


def kv_head_of(h, H, H_kv):
    """Index of the key/value head that query head ``h`` reads.

    "当注意力成为瓶颈…", section 推理优化：减少KV Cache: grouped-query attention
    splits the H query heads into H_kv groups and every group shares one
    key/value head (multi-query attention is the case H_kv = 1). The page does
    not say which query heads form a group; the reading taken here is
    consecutive heads: group j holds query heads j*G .. j*G + G - 1, G = H/H_kv.
    """
    if H_kv <= 0 or H % H_kv != 0:
        raise ValueError("H must be a multiple of H_kv")
    return h // (H // H_kv)


def _kv_per_query_head(x, H):
    """[B, H_kv, n, d] -> [B, H, n, d]: query head h gets key/value head kv_head_of(h)."""
    x = np.asarray(x, dtype=np.float64)
    H_kv = x.shape[1]
    idx = np.array([kv_head_of(h, H, H_kv) for h in range(H)], dtype=np.int64)
    return x[:, idx]


def gqa_fwd(q, k, v, rows=None):
    """Attention where query head h reads key/value head kv_head_of(h).

    q: [B, H, n_q, d]; k, v: [B, H_kv, n_k, d]. Each query head is plain
    attention (``naive_fwd``) against the key/value head of its group. Returns
    (o, m, l) like ``naive_fwd`` with leading axes [B, H].
    """
    q = np.asarray(q, dtype=np.float64)
    H = q.shape[1]
    return naive_fwd(q, _kv_per_query_head(k, H), _kv_per_query_head(v, H), rows=rows)


def gqa_bwd(q, k, v, do, rows=None, cols=None):
    """Gradients of L = sum(O * dO) for ``gqa_fwd``.

    A key/value head is used by every query head of its group, so by the chain
    rule its gradient is the sum over that group of the per-query-head
    gradients of ``naive_bwd`` (same textbook softmax Jacobian). Returns
    (dq [B, H, ., d], dk [B, H_kv, ., d], dv [B, H_kv, ., d]).
    """
    q = np.asarray(q, dtype=np.float64)
    B, H = q.shape[:2]
    H_kv = np.asarray(k).shape[1]
    dq, dk_h, dv_h = naive_bwd(q, _kv_per_query_head(k, H), _kv_per_query_head(v, H), do,
                               rows=rows, cols=cols)
    dk = np.zeros((B, H_kv) + dk_h.shape[2:])
    dv = np.zeros((B, H_kv) + dv_h.shape[2:])
    for h in range(H):
        j = kv_head_of(h, H, H_kv)
        dk[:, j] += dk_h[:, h]
        dv[:, j] += dv_h[:, h]
    return dq, dk, dv


def block_summary(q, k, v):
    """Summary of one key/value block for every query row, as the two-block
    merge of "当注意力成为瓶颈…", section IO感知, uses it: the block's score
    maximum m_b = max_j s_j, its sum l_b = sum_j exp(s_j - m_b) and its
    unnormalised output u_b = sum_j exp(s_j - m_b) v_j, s_j = q . k_j / sqrt(d).
    "Self-attention Does Not Need O(n^2) Memory" (方法详解; English digest
    method bullets) processes such blocks independently and combines their
    summaries. q: [..., n, d]; k, v: [..., c, d] with c >= 1.
    Returns (m [..., n], l [..., n], u [..., n, d]).
    """
    q3, lead = _as_slices(q)
    k3, _ = _as_slices(k)
    v3, _ = _as_slices(v)
    if k3.shape[1] == 0:
        raise ValueError("a block holds at least one key")
    scale = softmax_scale(q3.shape[2])
    s = np.einsum("gid,gjd->gij", q3, k3) * scale
    m = s.max(axis=2)
    p = np.exp(s - m[:, :, None])
    l = p.sum(axis=2)
    u = np.einsum("gij,gjd->gid", p, v3)
    n = q3.shape[1]
    return m.reshape(lead + (n,)), l.reshape(lead + (n,)), u.reshape(lead + (n, v3.shape[2]))


def merge_summaries(parts):
    """Combine block summaries (m_b, l_b, u_b) into the exact result.

    The two-block merge of "当注意力成为瓶颈…", section IO感知 (m is the
    larger block maximum; l and O add the blocks' exponentials re-based on
    that m), written for any number of blocks at once:
        m = max_b m_b
        l = sum_b exp(m_b - m) l_b
        o = (sum_b exp(m_b - m) u_b) / l
    Returns (o, m, l).
    """
    if not parts:
        raise ValueError("nothing to merge")
    m = parts[0][0]
    for mb, _, _ in parts[1:]:
        m = np.maximum(m, mb)
    l = np.zeros_like(parts[0][1])
    u = np.zeros_like(parts[0][2])
    for mb, lb, ub in parts:
        w = np.exp(mb - m)
        l = l + w * lb
        u = u + w[..., None] * ub
    return u / l[..., None], m, l


def split_ranges(n_k, splits):
    """Key ranges [a, b) of ``splits`` near-equal consecutive blocks (each non-empty)."""
    if n_k <= 0 or splits <= 0:
        raise ValueError("need n_k >= 1 and splits >= 1")
    splits = min(splits, n_k)
    step = -(-n_k // splits)
    return [(a, min(n_k, a + step)) for a in range(0, n_k, step)]


def split_fwd(q, k, v, splits):
    """Split-key attention: summarise each consecutive key block on its own
    (``block_summary``) and merge the summaries once (``merge_summaries``).
    q: [..., n, d]; k, v: [..., n_k, d]. Returns (o, m, l) like ``naive_fwd``.
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    parts = [block_summary(q, k[..., a:b, :], v[..., a:b, :])
             for a, b in split_ranges(k.shape[-2], splits)]
    return merge_summaries(parts)
