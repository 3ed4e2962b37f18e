"""Plain, slow, obviously correct fp64 reference for exact attention.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may use this module.  It shares no code with the GPU path.

Sources (web pages on FlashAttention; the page is named, then its section):
  * "FlashAttention" concept note (llm-wiki-maxwellmou.pages.dev), section
    "是什么": the definition O = softmax(Q K^T / sqrt(d)) V, the per-block
    online-softmax update of (m, l, O), and the statement that causal masks,
    padding masks and multi-head / GQA handling sit inside the tile.
  * "FlashAttention" explainer (liu-gong-zi.com), section "核心问题": the
    naive three-step program S = Q K^T / sqrt(d); P = softmax(S); O = P V with
    S and P materialised.
  * Interview note "FlashAttention 为什么更快、更省显存？" (notes.arfxm.cn),
    section "先看普通 Attention 保存了什么": the size of one n x n score matrix.

Readings where the pages are silent (each also listed in the design notes):
  * LSE (not on the pages) is the natural log of the sum, over allowed keys,
    of exp(scaled score): LSE_i = m_i + ln(l_i).
  * Causal alignment when Nq != Nk is bottom-right: key j is visible to query
    i iff j <= i + (Nk - Nq).
  * Padding: keys j >= kv_seqlens[b] are excluded; every query row is still
    computed.  Lengths are clamped to [0, Nk].
  * A row with no allowed key has O = 0 and LSE = -inf.
  * GQA: query head hq reads KV head hq // (Hq // Hkv).
  * scale is the fp32 value handed to the kernel, upcast exactly to fp64;
    the default is 1/sqrt(d) rounded to fp32.
"""
import math

import numpy as np

try:  # torch is only used to accept torch tensors (e.g. bfloat16) as inputs
    import torch
except ImportError:  # pragma: no cover
    torch = None


def to_f64(x):
    """Exact upcast of an input array (numpy or torch, any float dtype) to fp64."""
    if torch is not None and isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def default_scale(d):
    """1/sqrt(d) as the fp32 number the kernels receive, upcast to fp64."""
    return float(np.float32(1.0 / math.sqrt(d)))


def _valid_length(kv_seqlens, b, nk):
    if kv_seqlens is None:
        return nk
    return int(min(max(int(kv_seqlens[b]), 0), nk))


def _allowed(nq, nk, length, causal):
    """Boolean [nq, nk] mask of (query i, key j) pairs that take part.

    Padding and causal masks of the concept note, section "是什么"; causal
    alignment is bottom-right (j <= i + nk - nq).
    """
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    allowed = np.broadcast_to(j < length, (nq, nk))
    if causal:
        allowed = allowed & (j <= i + (nk - nq))
    return allowed


def _head_map(hq, n_q_heads, n_kv_heads):
    """GQA: query heads are grouped contiguously onto KV heads."""
    return hq // (n_q_heads // n_kv_heads)


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, _, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k and v must be [B, Hkv, Nk, d] matching q")
    if Hq % k.shape[1] != 0:
        raise ValueError("Hq must be a multiple of Hkv")


def _one_head(qh, kh, vh, allowed, scale):
    """Definition of attention for one head, with S and P materialised.

    S = scale * Q K^T; disallowed entries -> -inf; P = softmax(S) row-wise;
    O = P V; LSE = ln sum_j exp(S_ij).  Returns (O, LSE, P).
    """
    S = scale * (qh @ kh.T)
    S = np.where(allowed, S, -np.inf)
    m = S.max(axis=1)
    empty = m == -np.inf
    m_safe = np.where(empty, 0.0, m)
    E = np.exp(S - m_safe[:, None])          # exp(-inf) = 0 on masked entries
    l = E.sum(axis=1)
    l_safe = np.where(empty, 1.0, l)
    P = E / l_safe[:, None]
    O = P @ vh
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    O[empty] = 0.0
    return O, lse, P


def attention_ref(q, k, v, causal=False, kv_seqlens=None, scale=None,
                  heads=None, rows=None):
    """Exact attention, fp64, per (batch, query head).

    q: [B, Hq, Nq, d]; k, v: [B, Hkv, Nk, d]; kv_seqlens: None or int[B].
    heads: optional list of (b, hq) pairs to compute (others left as NaN);
    rows: optional index array of query rows to compute (others NaN).
    Returns O [B, Hq, Nq, d] and LSE [B, Hq, Nq] as fp64 arrays.
    """
    q = to_f64(q); k = to_f64(k); v = to_f64(v)
    _check_shapes(q, k, v)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if scale is None:
        scale = default_scale(d)
    scale = float(np.float32(scale))
    if kv_seqlens is not None:
        kv_seqlens = to_f64(kv_seqlens).astype(np.int64)
    O = np.full((B, Hq, Nq, d), np.nan)
    LSE = np.full((B, Hq, Nq), np.nan)
    row_idx = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, hq in pairs:
        hk = _head_map(hq, Hq, Hkv)
        allowed = _allowed(Nq, Nk, _valid_length(kv_seqlens, b, Nk), causal)[row_idx]
        o, lse, _ = _one_head(q[b, hq, row_idx], k[b, hk], v[b, hk], allowed, scale)
        O[b, hq, row_idx] = o
        LSE[b, hq, row_idx] = lse
    return O, LSE


def attention_probs_ref(q, k, v, causal=False, kv_seqlens=None, scale=None):
    """The materialised probability matrix P [B, Hq, Nq, Nk] (fp64)."""
    q = to_f64(q); k = to_f64(k); v = to_f64(v)
    _check_shapes(q, k, v)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if scale is None:
        scale = default_scale(d)
    scale = float(np.float32(scale))
    P = np.zeros((B, Hq, Nq, Nk))
    for b in range(B):
        for hq in range(Hq):
            hk = _head_map(hq, Hq, Hkv)
            allowed = _allowed(Nq, Nk, _valid_length(kv_seqlens, b, Nk), causal)
            _, _, P[b, hq] = _one_head(q[b, hq], k[b, hk], v[b, hk], allowed, scale)
    return P


def attention_bwd_ref(q, k, v, do, causal=False, kv_seqlens=None, scale=None):
    """Gradients of exact attention, fp64: (dQ, dK, dV) for the loss sum(dO * O).

    The pages say only that the backward pass recomputes the intermediates
    instead of storing them (Exam deep-dive, section 技術版, "Recomputation";
    Interview note, section 节省显存，不等于所有内存都变少).  What it computes is
    the derivative of the forward definition above, written out with S and P
    materialised, per (batch, query head):
        dV = P^T dO
        dP = dO V^T
        dS = P * (dP - rowsum(dO * O))      (softmax Jacobian, row by row)
        dQ = scale * dS K
        dK = scale * dS^T Q
    Disallowed pairs have P = 0 and so dS = 0.  With GQA every query head adds
    its dK, dV into the KV head it reads.  A row with no allowed key has O = 0
    and contributes nothing.
    q, do: [B, Hq, Nq, d]; k, v: [B, Hkv, Nk, d].  Returns fp64 arrays shaped
    like q, k and v.
    """
    q = to_f64(q); k = to_f64(k); v = to_f64(v); do = to_f64(do)
    _check_shapes(q, k, v)
    if do.shape != q.shape:
        raise ValueError("do must be shaped like q")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if scale is None:
        scale = default_scale(d)
    scale = float(np.float32(scale))
    if kv_seqlens is not None:
        kv_seqlens = to_f64(kv_seqlens).astype(np.int64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        allowed = _allowed(Nq, Nk, _valid_length(kv_seqlens, b, Nk), causal)
        for hq in range(Hq):
            hk = _head_map(hq, Hq, Hkv)
            o, _, P = _one_head(q[b, hq], k[b, hk], v[b, hk], allowed, scale)
            g = do[b, hq]
            dv[b, hk] += P.T @ g
            dP = g @ v[b, hk].T
            Dr = (g * o).sum(axis=1)
            dS = P * (dP - Dr[:, None])
            dq[b, hq] = scale * (dS @ k[b, hk])
            dk[b, hk] += scale * (dS.T @ q[b, hq])
    return dq, dk, dv


def online_softmax_blocked(qh, kh, vh, block, scale, allowed=None):
    """The per-block online-softmax update of the concept note, section "是什么".

    One head: qh [Nq, d], kh, vh [Nk, d]; keys are visited in blocks of
    `block`.  Per row the state is (m, l, O) with O kept normalised, and on
    each block S_b = scale * Q K_b^T:
        m'  = max(m, rowmax S_b)
        l'  = e^(m - m') l + rowsum e^(S_b - m')
        O'  = (e^(m - m') l O + e^(S_b - m') V_b) / l'
    Masked scores are -inf; a row whose state is still empty (m' = -inf) keeps
    l = 0, O = 0.  Returns (O, LSE) with LSE = m + ln l.
    """
    qh = to_f64(qh); kh = to_f64(kh); vh = to_f64(vh)
    nq, nk = qh.shape[0], kh.shape[0]
    if allowed is None:
        allowed = np.ones((nq, nk), dtype=bool)
    m = np.full(nq, -np.inf)
    l = np.zeros(nq)
    O = np.zeros((nq, vh.shape[1]))
    for start in range(0, nk, block):
        stop = min(start + block, nk)
        Sb = scale * (qh @ kh[start:stop].T)
        Sb = np.where(allowed[:, start:stop], Sb, -np.inf)
        m_new = np.maximum(m, Sb.max(axis=1))
        live = m_new > -np.inf
        m_ref = np.where(live, m_new, 0.0)
        alpha = np.where(live, np.exp(m - m_ref), 0.0)   # e^(m - m'); 0 when m = -inf
        Eb = np.exp(Sb - m_ref[:, None])
        l_new = alpha * l + Eb.sum(axis=1)
        denom = np.where(l_new > 0, l_new, 1.0)
        O_new = ((alpha * l)[:, None] * O + Eb @ vh[start:stop]) / denom[:, None]
        O = np.where(live[:, None], O_new, O)
        l = np.where(live, l_new, l)
        m = m_new
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return O, lse


def merge_partials(o_parts, lse_parts):
    """Exact merge of partial attention results over disjoint key sets.

    o_parts [..., S, d] holds each part's normalised output, lse_parts [..., S]
    its log-sum-exp.  This is the concept note's online-softmax update with the
    blocks taken to be the parts:  M = max_s lse_s,
    LSE = M + ln sum_s e^(lse_s - M),  O = sum_s e^(lse_s - LSE) O_s.
    Parts with lse = -inf carry no weight; if all are -inf, O = 0, LSE = -inf.
    """
    o_parts = to_f64(o_parts); lse_parts = to_f64(lse_parts)
    M = lse_parts.max(axis=-1)
    empty = M == -np.inf
    M_safe = np.where(empty, 0.0, M)
    w = np.exp(lse_parts - M_safe[..., None])
    tot = w.sum(axis=-1)
    tot_safe = np.where(empty, 1.0, tot)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, M_safe + np.log(tot_safe))
    O = (w[..., None] * o_parts).sum(axis=-2) / tot_safe[..., None]
    O[empty] = 0.0
    return O, lse


def split_bounds(length, num_splits, tile):
    """Key ranges [begin, end) of the split-KV decode partition.

    Chunk C = ceil(length / num_splits) rounded up to a multiple of `tile`;
    split s covers [s C, min((s+1) C, length)), possibly empty.
    """
    length = max(int(length), 0)
    c = -(-length // num_splits) if length > 0 else 0
    c = -(-c // tile) * tile
    return [(min(s * c, length), min((s + 1) * c, length)) for s in range(num_splits)]


def decode_partials_ref(q, k, v, kv_seqlens, scale, num_splits, tile):
    """Per-split partial (O_s, lse_s) of single-token decode, fp64.

    q [B, Hq, 1, d]; k, v [B, Hkv, Nk, d].  Each split is plain attention over
    its key range (the definition restricted to those keys); an empty range
    gives O_s = 0, lse_s = -inf.  Returns O [B, Hq, S, d], LSE [B, Hq, S].
    """
    q = to_f64(q); k = to_f64(k); v = to_f64(v)
    _check_shapes(q, k, v)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if Nq != 1:
        raise ValueError("decode takes one query token per sequence")
    if kv_seqlens is not None:
        kv_seqlens = to_f64(kv_seqlens).astype(np.int64)
    scale = float(np.float32(scale))
    O = np.zeros((B, Hq, num_splits, d))
    LSE = np.full((B, Hq, num_splits), -np.inf)
    for b in range(B):
        L = _valid_length(kv_seqlens, b, Nk)
        for s, (a, e) in enumerate(split_bounds(L, num_splits, tile)):
            if e <= a:
                continue
            for hq in range(Hq):
                hk = _head_map(hq, Hq, Hkv)
                allowed = np.ones((1, e - a), dtype=bool)
                o, lse, _ = _one_head(q[b, hq], k[b, hk, a:e], v[b, hk, a:e], allowed, scale)
                O[b, hq, s] = o[0]
                LSE[b, hq, s] = lse[0]
    return O, LSE


def _seq_bounds(cu, b, total):
    """Rows [start, stop) of packed sequence b; offsets are clamped to [0, total]."""
    start = int(min(max(int(cu[b]), 0), total))
    stop = int(min(max(int(cu[b + 1]), start), total))
    return start, stop


def attention_varlen_ref(q, k, v, cu_seqlens_q, cu_seqlens_k, causal=False, scale=None):
    """Exact attention over packed variable-length sequences, fp64.

    The pages put padding masks inside the tile (Concept note, section "是什么")
    and contrast prompt processing with one-token decode against a KV cache
    (the same note's list of misconceptions); they give no packed layout.  The
    plainest reading, used here: the sequences of a batch are concatenated
    along the token axis of every head, q [Hq, total_q, d] and k, v
    [Hkv, total_k, d]; sequence b owns query rows cu_seqlens_q[b] ..
    cu_seqlens_q[b+1] - 1 and key rows cu_seqlens_k[b] .. cu_seqlens_k[b+1] - 1,
    and attends only to its own keys.  Each sequence is the definition above
    with Nq = Lq_b and Nk = Lk_b, so the causal mask is bottom-right aligned
    per sequence: local key j is visible to local query i iff j <= i + Lk_b - Lq_b
    (a chunk of new queries sees the whole cache before it).  A query row with
    no visible key has O = 0, LSE = -inf.  Returns O [Hq, total_q, d] and
    LSE [Hq, total_q]; rows outside every sequence stay NaN.
    """
    q = to_f64(q); k = to_f64(k); v = to_f64(v)
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3 or k.shape != v.shape or k.shape[2] != q.shape[2]:
        raise ValueError("q must be [Hq, total_q, d]; k, v [Hkv, total_k, d]")
    Hq, total_q, d = q.shape
    Hkv, total_k = k.shape[0], k.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    cu_q = np.asarray(to_f64(cu_seqlens_q), dtype=np.int64)
    cu_k = np.asarray(to_f64(cu_seqlens_k), dtype=np.int64)
    if cu_q.shape != cu_k.shape or cu_q.ndim != 1 or cu_q.size < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be int[B + 1]")
    if scale is None:
        scale = default_scale(d)
    scale = float(np.float32(scale))
    O = np.full((Hq, total_q, d), np.nan)
    LSE = np.full((Hq, total_q), np.nan)
    for b in range(cu_q.size - 1):
        qs, qe = _seq_bounds(cu_q, b, total_q)
        ks, ke = _seq_bounds(cu_k, b, total_k)
        if qe == qs:
            continue
        if ke == ks:  # no keys at all: every row is empty
            O[:, qs:qe] = 0.0
            LSE[:, qs:qe] = -np.inf
            continue
        allowed = _allowed(qe - qs, ke - ks, ke - ks, causal)
        for hq in range(Hq):
            hk = _head_map(hq, Hq, Hkv)
            o, lse, _ = _one_head(q[hq, qs:qe], k[hk, ks:ke], v[hk, ks:ke], allowed, scale)
            O[hq, qs:qe] = o
            LSE[hq, qs:qe] = lse
    return O, LSE


def paged_to_contiguous(pages, block_table, lengths, page_size):
    """Gather a paged KV cache into contiguous per-sequence rows.

    The pages place the KV cache under page management (PagedAttention) and
    leave the layout open (Concept note, section "是什么", table of related
    concepts).  The plainest reading, used here: pages is a pool
    [num_pages, Hkv, page_size, d]; block_table[b] lists sequence b's pages
    in key order, so key j of sequence b is row j % page_size of page
    block_table[b][j // page_size].  Returns [B, Hkv, max_pages * page_size, d]
    with the rows at or beyond lengths[b] set to NaN (they must never be read).
    """
    pages = to_f64(pages)
    table = np.asarray(to_f64(block_table), dtype=np.int64)
    lengths = np.asarray(to_f64(lengths), dtype=np.int64)
    B, max_pages = table.shape
    _, Hkv, P, d = pages.shape
    if P != page_size:
        raise ValueError("page_size does not match the pool")
    out = np.full((B, Hkv, max_pages * P, d), np.nan)
    for b in range(B):
        L = int(min(max(lengths[b], 0), max_pages * P))
        for j in range(L):
            out[b, :, j] = pages[table[b, j // P], :, j % P]
    return out


def score_matrix_bytes(n, bytes_per_element):
    """Bytes of one materialised n x n score (or probability) matrix."""
    return n * n * bytes_per_element
