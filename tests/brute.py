"""Scalar brute force of attention (and of the backward's magnitude sums) on
tiny inputs: nested Python lists and the ``math`` module only, no numpy or
torch arithmetic.

It is written independently of the oracle and in a different form: the row's
logsumexp is taken first, log(fsum(exp(s_j))), with no max subtraction, and each
weight is exp(s_j - lse).  Inputs must keep |s_j| small enough that exp does not
overflow.  Visibility is the causal predicate with bottom-right alignment
(key j visible to query i iff j <= i + Nk - N), as read from the ai6s.net page,
section "what ops-transformer adds", second item.
"""
import math


def attention(q, k, v, causal, scale):
    """q [B][N][Hq][d], k/v [B][Nk][Hkv][d] nested lists -> (o [B][N][Hq][d], lse [B][Hq][N])."""
    B, N, Hq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Nk, Hkv = len(k[0]), len(k[0][0])
    group = Hq // Hkv
    o = [[[[0.0] * d for _ in range(Hq)] for _ in range(N)] for _ in range(B)]
    lse = [[[0.0] * N for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for i in range(N):
                keys = [j for j in range(Nk) if (not causal) or j <= i + Nk - N]
                if not keys:
                    lse[b][h][i] = -math.inf
                    continue
                s = {j: scale * math.fsum(q[b][i][h][c] * k[b][j][g][c] for c in range(d))
                     for j in keys}
                z = math.log(math.fsum(math.exp(s[j]) for j in keys))
                lse[b][h][i] = z
                for c in range(d):
                    o[b][i][h][c] = math.fsum(math.exp(s[j] - z) * v[b][j][g][c] for j in keys)
    return o, lse


def bwd_magnitudes(q, k, v, do, causal, scale):
    """The absolute-value sums that bound the rounding in the backward, term
    by term, on nested lists (same layouts as ``attention``; do like q):
        mv[j][g][c] = sum over the group's heads h and rows i of P_hij |dO_hic|
        mq[i][h][c] = scale sum_j (|dS_hij| + a_hi P_hij) |K_jgc|
        mk[j][g][c] = scale sum over h, i of (|dS_hij| + a_hi P_hij) |Q_hic|
    with P the softmax of the visible scores, dP_hij = dO_hi . V_jg,
    dS_hij = P_hij (dP_hij - sum_l P_hil dP_hil) and a_hi = sum_c |dO_hic O_hic|,
    O = P V (the chain rule of the attention definition, each product taken in
    absolute value).  Returns (mq, mk, mv) as nested lists."""
    B, N, Hq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Nk, Hkv = len(k[0]), len(k[0][0])
    group = Hq // Hkv
    mq = [[[[0.0] * d for _ in range(Hq)] for _ in range(N)] for _ in range(B)]
    mk = [[[[0.0] * d for _ in range(Hkv)] for _ in range(Nk)] for _ in range(B)]
    mv = [[[[0.0] * d for _ in range(Hkv)] for _ in range(Nk)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for i in range(N):
                keys = [j for j in range(Nk) if (not causal) or j <= i + Nk - N]
                if not keys:
                    continue
                s = {j: scale * math.fsum(q[b][i][h][c] * k[b][j][g][c] for c in range(d)) for j in keys}
                z = math.log(math.fsum(math.exp(s[j]) for j in keys))
                p = {j: math.exp(s[j] - z) for j in keys}
                o = [math.fsum(p[j] * v[b][j][g][c] for j in keys) for c in range(d)]
                a = math.fsum(abs(do[b][i][h][c] * o[c]) for c in range(d))
                dp = {j: math.fsum(do[b][i][h][c] * v[b][j][g][c] for c in range(d)) for j in keys}
                dsum = math.fsum(p[j] * dp[j] for j in keys)
                w = {j: abs(p[j] * (dp[j] - dsum)) + a * p[j] for j in keys}
                for c in range(d):
                    mq[b][i][h][c] = scale * math.fsum(w[j] * abs(k[b][j][g][c]) for j in keys)
                for j in keys:
                    for c in range(d):
                        mv[b][j][g][c] += p[j] * abs(do[b][i][h][c])
                        mk[b][j][g][c] += scale * w[j] * abs(q[b][i][h][c])
    return mq, mk, mv
