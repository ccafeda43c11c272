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

A row with no visible key (impossible for square causal attention, kept for
completeness) has O = 0, LSE = −∞ and contributes no gradient.

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


def _scores(q, k, causal, scale, rows=None, seg=None):
    """S = scale·q·kᵀ for one head with the causal and segment masks applied.

    rows: the global row index of each query row (default 0..n_q−1); seg: the
    segment id of every key row (None: one segment holding all rows).
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
    return s


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


def attention_forward(q, k, v, causal, scale, cu_seqlens=None):
    """O = softmax(scale·Q·Kᵀ [causal] [segments]) · V and LSE, per (b, h), in float64.

    q, k, v: [B, H, N, d] float64; cu_seqlens: optional segment offsets (the
    same for every (b, h)). Returns (O [B,H,N,d], LSE [B,H,N]).
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
            s = _scores(q[b, h], k[b, h], causal, scale, seg=seg)
            p, lse[b, h] = softmax_rows(s)
            o[b, h] = p @ v[b, h]
    return o, lse


def attention_forward_rows(q, k, v, causal, scale, b, h, rows, cu_seqlens=None):
    """Forward for selected query rows of one head (b, h); same definition.

    Used to check outputs at full problem sizes on sampled rows. Returns
    (O_rows [len(rows), d], LSE_rows [len(rows)]).
    """
    rows = np.asarray(rows, dtype=np.int64)
    qh = np.asarray(q[b, h], dtype=np.float64)[rows]
    kh = np.asarray(k[b, h], dtype=np.float64)
    vh = np.asarray(v[b, h], dtype=np.float64)
    seg = None if cu_seqlens is None else segment_ids(kh.shape[0], cu_seqlens)
    s = _scores(qh, kh, causal, scale, rows=rows, seg=seg)
    p, lse = softmax_rows(s)
    return p @ vh, lse


def attention_backward(q, k, v, do, causal, scale, cu_seqlens=None):
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
            s = _scores(q[b, h], k[b, h], causal, scale, seg=seg)
            p, _ = softmax_rows(s)
            dv[b, h] = p.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T
            dvec[b, h] = np.sum(p * dp, axis=1)
            ds = p * (dp - dvec[b, h][:, None])
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
    return dq, dk, dv, dvec
