"""Pure-Python scalar-loop restatement of the GQA definitions, for tiny inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).  It exists to pin the
NumPy oracle in ``gqa_oracle`` with an implementation of a different shape:
no NumPy arithmetic, correctly rounded sums (``math.fsum``), and the group of
each query head found by scanning the 1-based group ranges stated on
pinghaoyang.com.cn "GQA 完全拆解", section "GQA：插值在 MHA 与 MQA 之间的分组共享"
(group g holds query heads (g-1)*h/G+1 .. g*h/G, with G the number of groups
in that page's notation).

Inputs are nested Python lists (or anything indexable that yields floats).
"""
from __future__ import annotations

import math


def group_of_head(i1: int, num_heads: int, num_groups: int) -> int:
    """1-based group of the 1-based query head ``i1``, found by scanning the
    consecutive ranges ((g-1)*n/G, g*n/G]."""
    per = num_heads // num_groups
    for g1 in range(1, num_groups + 1):
        lo = (g1 - 1) * per + 1
        hi = g1 * per
        if lo <= i1 <= hi:
            return g1
    raise ValueError("head outside every group")


def _attend(qv, keys, values, scale):
    """softmax(scale * q . k_j) weighted sum of v_j, scalar loops."""
    n = len(keys)
    d = len(values[0])
    scores = [scale * math.fsum(qv[c] * keys[j][c] for c in range(len(qv)))
              for j in range(n)]
    top = max(scores)
    w = [math.exp(s - top) for s in scores]
    tot = math.fsum(w)
    return [math.fsum(w[j] * values[j][c] for j in range(n)) / tot for c in range(d)]


def decode_bruteforce(q, k_cache, v_cache, seq_lens, scale):
    """out[b][h][c] for one decode step; a sequence with L_b = 0 gives zeros."""
    B = len(q)
    H = len(q[0])
    d = len(q[0][0])
    K = len(k_cache[0])
    out = []
    for b in range(B):
        L = int(seq_lens[b])
        rows = []
        for i1 in range(1, H + 1):
            if L == 0:
                rows.append([0.0] * d)
                continue
            g0 = group_of_head(i1, H, K) - 1
            keys = [[float(x) for x in k_cache[b][g0][j]] for j in range(L)]
            vals = [[float(x) for x in v_cache[b][g0][j]] for j in range(L)]
            rows.append(_attend([float(x) for x in q[b][i1 - 1]], keys, vals, float(scale)))
        out.append(rows)
    return out


def prefill_bruteforce(q, k, v, scale):
    """out[b][h][i][c] of causal attention: query i sees keys 0..i."""
    B = len(q)
    H = len(q[0])
    S = len(q[0][0])
    K = len(k[0])
    out = []
    for b in range(B):
        heads = []
        for i1 in range(1, H + 1):
            g0 = group_of_head(i1, H, K) - 1
            rows = []
            for i in range(S):
                keys = [[float(x) for x in k[b][g0][j]] for j in range(i + 1)]
                vals = [[float(x) for x in v[b][g0][j]] for j in range(i + 1)]
                rows.append(_attend([float(x) for x in q[b][i1 - 1][i]], keys, vals, float(scale)))
            heads.append(rows)
        out.append(heads)
    return out


def meanpool_bruteforce(src, num_groups):
    """dst[o][g][i] = arithmetic mean of src[o][r][i] over the heads r of group g."""
    outer = len(src)
    H = len(src[0])
    inner = len(src[0][0])
    dst = []
    for o in range(outer):
        groups = []
        for g1 in range(1, num_groups + 1):
            members = [r1 for r1 in range(1, H + 1) if group_of_head(r1, H, num_groups) == g1]
            groups.append([math.fsum(float(src[o][r1 - 1][i]) for r1 in members) / len(members)
                           for i in range(inner)])
        dst.append(groups)
    return dst
