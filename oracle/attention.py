"""Float64 attention forward and backward, written as the plain definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition followed ([FA4-news] "Por qué el enfoque estándar ya no funciona":
the two products S = Q·Kᵀ and O = P·V with a softmax between them; [FA3-wiki]
"El problema del mecanismo de atención": the naive form materialises the
intermediate matrix, which is exactly what this oracle does):

    S   = scale · Q · Kᵀ                        (N × N per head)
    S_ij = −∞ for j > i when causal             (reading: key j is visible to
                                                 query i iff j ≤ i)
    P   = softmax over each row of S
    O   = P · V
    LSE_i = ln Σ_j exp(S_ij)                    (natural log, scale included)

Backward (standard gradient of ⟨O, dO⟩; the pages name only dS and dQ, in
[FA4-gist] technical summary 2.C):

    dV = Pᵀ·dO,  dP = dO·Vᵀ,  D_i = Σ_j P_ij dP_ij,
    dS = P ∘ (dP − D),  dQ = scale·dS·K,  dK = scale·dSᵀ·Q.

Variable-length sequences packed along N (varlen; the pages name it only as a
variant the tiled design enables, [FA4-gist-pt] "Significado e Impacto"):
offsets cu_seqlens = [c_0, …, c_n] split the rows into segments
[c_s, c_{s+1}); reading: key j is visible to query i iff both lie in the same
segment (and, when causal, j ≤ i). Each segment is then an independent
attention problem; rows outside every segment see no key.

Block-sparse attention (the pages name it, like varlen, only as a variant
the tiled design enables): a 0/1 block mask M over blocks of `block` query
rows × `block` key rows (block = 128 for the kernels); reading: key j is
visible to query i iff M[i // block, j // block] ≠ 0 (and the causal and
segment conditions, when given, also hold).

A row with no visible key (impossible for square causal attention, possible
under a block mask) has O = 0, LSE = −∞ and contributes no gradient.

All inputs are float64 arrays of shape [B, H, N, d]; they are the exact values
of the bf16 inputs the GPU consumes.
"""
import numpy as np


def segment_ids(n, cu_seqlens):
    """Segment index of each of n rows for the offsets cu_seqlens (−1 for rows
    outside every segment)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    ids = np.full(n, -1, dtype=np.int64)
    for s in range(len(cu) - 1):
        ids[cu[s]:cu[s + 1]] = s
    return ids


def _scores(q, k, causal, scale, rows=None, seg=None, bmask=None, block=128):
    """S = scale·q·kᵀ for one head with the causal, segment and block masks.

    rows: the global row index of each query row (default 0..n_q−1); seg: the
    segment id of every key row (None: one segment holding all rows); bmask:
    the head's block mask [⌈N/block⌉, ⌈N/block⌉] (None: every block visible).
    """
    s = scale * (q @ k.T)
    n_q, n_k = s.shape
    r = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    cols = np.arange(n_k)[None, :]
    if causal:
        s = np.where(cols <= r[:, None], s, -np.inf)
    if seg is not None:
        sq = seg[r][:, None]
        s = np.where((seg[None, :] == sq) & (sq >= 0), s, -np.inf)
    if bmask is not None:
        vis = np.asarray(bmask)[r[:, None] // block, np.arange(n_k)[None, :] // block] != 0
        s = np.where(vis, s, -np.inf)
    return s


def _head_mask(block_mask, b, h, H):
    """The block mask of head (b, h): one [nb, nb] mask for all heads, or
    [B·H, nb, nb] with one per head."""
    if block_mask is None:
        return None
    m = np.asarray(block_mask)
    return m if m.ndim == 2 else m[b * H + h]


def softmax_rows(s):
    """Row softmax of a score matrix and its natural-log normaliser.

    Returns (P, LSE). Rows that are entirely −∞ give P = 0 and LSE = −∞.
    """
    m = np.max(s, axis=1, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe)
    l = np.sum(e, axis=1, keepdims=True)
    l_safe = np.where(empty, 1.0, l)
    p = np.where(empty, 0.0, e / l_safe)
    lse = np.where(empty[:, 0], -np.inf, m_safe[:, 0] + np.log(l_safe[:, 0]))
    return p, lse


def attention_forward(q, k, v, causal, scale, cu_seqlens=None, block_mask=None, block=128):
    """O = softmax(scale·Q·Kᵀ [causal] [segments] [block mask]) · V and LSE,
    per (b, h), in float64.

    q, k, v: [B, H, N, d] float64; cu_seqlens: optional segment offsets (the
    same for every (b, h)); block_mask: optional 0/1 block mask, [nb, nb] for
    all heads or [B·H, nb, nb], nb = ⌈N/block⌉. Returns (O [B,H,N,d], LSE [B,H,N]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    seg = None if cu_seqlens is None else segment_ids(N, cu_seqlens)
    o = np.empty((B, H, N, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = _scores(q[b, h], k[b, h], causal, scale, seg=seg,
                        bmask=_head_mask(block_mask, b, h, H), block=block)
            p, lse[b, h] = softmax_rows(s)
            o[b, h] = p @ v[b, h]
    return o, lse


def attention_forward_rows(q, k, v, causal, scale, b, h, rows, cu_seqlens=None, block_mask=None,
                           block=128):
    """Forward for selected query rows of one head (b, h); same definition.

    Used to check outputs at full problem sizes on sampled rows. Returns
    (O_rows [len(rows), d], LSE_rows [len(rows)]).
    """
    rows = np.asarray(rows, dtype=np.int64)
    qh = np.asarray(q[b, h], dtype=np.float64)[rows]
    kh = np.asarray(k[b, h], dtype=np.float64)
    vh = np.asarray(v[b, h], dtype=np.float64)
    seg = None if cu_seqlens is None else segment_ids(kh.shape[0], cu_seqlens)
    s = _scores(qh, kh, causal, scale, rows=rows, seg=seg,
                bmask=_head_mask(block_mask, b, h, np.asarray(q).shape[1]), block=block)
    p, lse = softmax_rows(s)
    return p @ vh, lse


def attention_backward(q, k, v, do, causal, scale, cu_seqlens=None, block_mask=None, block=128):
    """Gradients of ⟨O, dO⟩ with respect to Q, K, V, in float64.

    P is formed again from the definition (not from any saved statistic).
    Returns (dQ, dK, dV, D) with D = rowsum(P ∘ dP) of shape [B, H, N].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, N, d = q.shape
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    dvec = np.empty((B, H, N), dtype=np.float64)
    seg = None if cu_seqlens is None else segment_ids(N, cu_seqlens)
    for b in range(B):
        for h in range(H):
            s = _scores(q[b, h], k[b, h], causal, scale, seg=seg,
                        bmask=_head_mask(block_mask, b, h, H), block=block)
            p, _ = softmax_rows(s)
            dv[b, h] = p.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T
            dvec[b, h] = np.sum(p * dp, axis=1)
            ds = p * (dp - dvec[b, h][:, None])
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
    return dq, dk, dv, dvec
