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

A row with no visible key (impossible for square causal attention, kept for
completeness) has O = 0, LSE = −∞ and contributes no gradient.

All inputs are float64 arrays of shape [B, H, N, d]; they are the exact values
of the bf16 inputs the GPU consumes.
"""
import numpy as np


def _scores(q, k, causal, scale):
    """S = scale·q·kᵀ for one head, with the causal mask applied."""
    s = scale * (q @ k.T)
    if causal:
        n_q, n_k = s.shape
        rows = np.arange(n_q)[:, None]
        cols = np.arange(n_k)[None, :]
        s = np.where(cols <= rows, s, -np.inf)
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


def attention_forward(q, k, v, causal, scale):
    """O = softmax(scale·Q·Kᵀ [causal]) · V and LSE, per (b, h), in float64.

    q, k, v: [B, H, N, d] float64. Returns (O [B,H,N,d], LSE [B,H,N]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    o = np.empty((B, H, N, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = _scores(q[b, h], k[b, h], causal, scale)
            p, lse[b, h] = softmax_rows(s)
            o[b, h] = p @ v[b, h]
    return o, lse


def attention_forward_rows(q, k, v, causal, scale, b, h, rows):
    """Forward for selected query rows of one head (b, h); same definition.

    Used to check outputs at full problem sizes on sampled rows. Returns
    (O_rows [len(rows), d], LSE_rows [len(rows)]).
    """
    rows = np.asarray(rows, dtype=np.int64)
    qh = np.asarray(q[b, h], dtype=np.float64)[rows]
    kh = np.asarray(k[b, h], dtype=np.float64)
    vh = np.asarray(v[b, h], dtype=np.float64)
    s = scale * (qh @ kh.T)
    if causal:
        cols = np.arange(kh.shape[0])[None, :]
        s = np.where(cols <= rows[:, None], s, -np.inf)
    p, lse = softmax_rows(s)
    return p @ vh, lse


def attention_backward(q, k, v, do, causal, scale):
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
    for b in range(B):
        for h in range(H):
            s = _scores(q[b, h], k[b, h], causal, scale)
            p, _ = softmax_rows(s)
            dv[b, h] = p.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T
            dvec[b, h] = np.sum(p * dp, axis=1)
            ds = p * (dp - dvec[b, h][:, None])
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
    return dq, dk, dv, dvec
