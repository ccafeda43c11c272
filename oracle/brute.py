"""Pure-Python triple-loop attention for tiny shapes — TEST INFRASTRUCTURE ONLY.

No numpy linear algebra, no vectorisation: every score, exponential, sum and
product is an explicit loop over scalars, so that it can be read against the
definition S = scale·Q·Kᵀ, P = row-softmax(S), O = P·V ([FA4-news] "Por qué el
enfoque estándar ya no funciona") term by term. It cross-checks
``oracle.attention`` on N ≤ 16. It uses no max-subtraction: with the small
inputs it is given, exp() cannot overflow, which keeps it a different
computation from the vectorised oracle.
"""
import math


def brute_forward(q, k, v, causal, scale, cu_seqlens=None, block_mask=None, block=128):
    """q, k, v: nested lists [N][d] (one head). Returns (O [N][d], LSE [N]).

    cu_seqlens: optional segment offsets; key j then counts for query i only
    if some segment [c_s, c_{s+1}) holds both. block_mask: optional nested
    list [nb][nb] of 0/1; key j counts for query i only if the entry of
    their blocks (block rows each) is 1. A query that sees no key gets
    O = 0 and LSE = −∞.
    """
    n = len(q)
    d = len(q[0])
    dv = len(v[0])
    o = [[0.0] * dv for _ in range(n)]
    lse = [0.0] * n
    for i in range(n):
        weights = []
        for j in range(n):
            if causal and j > i:
                weights.append(0.0)
                continue
            if block_mask is not None and block_mask[i // block][j // block] == 0:
                weights.append(0.0)
                continue
            if cu_seqlens is not None:
                same = False
                for s in range(len(cu_seqlens) - 1):
                    if cu_seqlens[s] <= i < cu_seqlens[s + 1] and cu_seqlens[s] <= j < cu_seqlens[s + 1]:
                        same = True
                if not same:
                    weights.append(0.0)
                    continue
            dot = 0.0
            for c in range(d):
                dot += q[i][c] * k[j][c]
            weights.append(math.exp(scale * dot))
        total = 0.0
        for w in weights:
            total += w
        if total == 0.0:
            lse[i] = -math.inf
            continue
        lse[i] = math.log(total)
        for c in range(dv):
            acc = 0.0
            for j in range(n):
                acc += weights[j] * v[j][c]
            o[i][c] = acc / total
    return o, lse


def brute_backward(q, k, v, do, causal, scale):
    """Gradients of sum_ic O_ic·dO_ic for one head, by explicit loops.

    Returns (dQ, dK, dV) as nested lists. Uses the chain rule through
    O_i = Σ_j P_ij V_j and P_ij = exp(S_ij)/Σ_t exp(S_it) without any of the
    D_i shortcut: dS_ij = Σ_t dP_it · ∂P_it/∂S_ij with
    ∂P_it/∂S_ij = P_it(δ_tj − P_ij).
    """
    n = len(q)
    d = len(q[0])
    dvd = len(v[0])
    p = [[0.0] * n for _ in range(n)]
    for i in range(n):
        w = []
        for j in range(n):
            if causal and j > i:
                w.append(0.0)
            else:
                dot = 0.0
                for c in range(d):
                    dot += q[i][c] * k[j][c]
                w.append(math.exp(scale * dot))
        tot = sum(w)
        for j in range(n):
            p[i][j] = w[j] / tot
    dv_ = [[0.0] * dvd for _ in range(n)]
    for j in range(n):
        for c in range(dvd):
            acc = 0.0
            for i in range(n):
                acc += p[i][j] * do[i][c]
            dv_[j][c] = acc
    dp = [[0.0] * n for _ in range(n)]
    for i in range(n):
        for j in range(n):
            acc = 0.0
            for c in range(dvd):
                acc += do[i][c] * v[j][c]
            dp[i][j] = acc
    ds = [[0.0] * n for _ in range(n)]
    for i in range(n):
        for j in range(n):
            acc = 0.0
            for t in range(n):
                jac = p[i][t] * ((1.0 if t == j else 0.0) - p[i][j])
                acc += dp[i][t] * jac
            ds[i][j] = acc
    dq = [[0.0] * d for _ in range(n)]
    dk = [[0.0] * d for _ in range(n)]
    for i in range(n):
        for c in range(d):
            acc = 0.0
            for j in range(n):
                acc += ds[i][j] * k[j][c]
            dq[i][c] = scale * acc
    for j in range(n):
        for c in range(d):
            acc = 0.0
            for i in range(n):
                acc += ds[i][j] * q[i][c]
            dk[j][c] = scale * acc
    return dq, dk, dv_
