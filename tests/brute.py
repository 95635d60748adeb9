"""Pure-Python brute force for tiny MoE cases (test helper, no NumPy arithmetic).

Written independently of the oracle: plain loops over lists of Python floats,
used only to pin the oracle on inputs small enough to enumerate.
"""

import itertools
import math
import struct


def f32(v):
    """Round a Python float to the nearest IEEE float32 (ties to even).  A sum
    of two float32 values formed in double precision and rounded once this way
    is the correctly rounded float32 sum."""
    return struct.unpack("f", struct.pack("f", v))[0]


def matvec(W, x):
    """W is a list of rows; returns W x."""
    return [sum(w * xi for w, xi in zip(row, x)) for row in W]


def silu(z):
    # logistic written as a branch on the sign so exp never overflows
    if z >= 0:
        return z / (1.0 + math.exp(-z))
    ez = math.exp(z)
    return z * ez / (1.0 + ez)


def expert(x, Wg, Wu, Wd):
    u = matvec(Wg, x)
    v = matvec(Wu, x)
    a = [silu(ui) * vi for ui, vi in zip(u, v)]
    return matvec(Wd, a)


def best_subset(keys, k):
    """Enumerate every k-subset; keep the largest key sum, ties to the
    lexicographically smallest index tuple.  Returns a sorted tuple."""
    best, best_sum = None, None
    for sub in itertools.combinations(range(len(keys)), k):
        s = sum(keys[i] for i in sub)
        if best is None or s > best_sum:
            best, best_sum = sub, s
    return best


def topk_by_selection(keys, k):
    """Repeated selection of the maximum, lower index on ties: the slot order."""
    remaining = list(range(len(keys)))
    out = []
    for _ in range(k):
        m = remaining[0]
        for i in remaining[1:]:
            if keys[i] > keys[m]:
                m = i
        out.append(m)
        remaining.remove(m)
    return out


def route_and_drop(idx, E, cap):
    """idx: list of per-token expert lists.  Walk tokens in order; an expert
    accepts a token while it has taken fewer than ``cap`` (None = no limit).
    Returns per-token lists of booleans (kept) and per-expert routed counts."""
    taken = [0] * E
    count = [0] * E
    kept = []
    for sel in idx:
        row = []
        for e in sel:
            count[e] += 1
            ok = cap is None or taken[e] < cap
            if ok:
                taken[e] += 1
            row.append(ok)
        kept.append(row)
    return kept, count


def dense_layer(xs, Wr, Wg, Wu, Wd, k, cap=None, shared=(), logit_bias=None,
                select_bias=None):
    """Every expert on every token, weighted by a dense gate matrix that is zero
    for unselected or dropped experts.  ``select_bias`` shifts the selection
    keys only (added in float32 to the float32-rounded logit)."""
    E = len(Wr)
    out = []
    idx_all, gates_all = [], []
    for x in xs:
        l = matvec(Wr, x)
        if logit_bias is not None:
            l = [a + b for a, b in zip(l, logit_bias)]
        keys = l if select_bias is None else [f32(f32(a) + b) for a, b in zip(l, select_bias)]
        sel = topk_by_selection(keys, k)
        m = max(l[e] for e in sel)
        z = sum(math.exp(l[e] - m) for e in sel)
        idx_all.append(sel)
        gates_all.append([math.exp(l[e] - m) / z for e in sel])
    kept, _ = route_and_drop(idx_all, E, cap)
    for t, x in enumerate(xs):
        G = [0.0] * E
        for j, e in enumerate(idx_all[t]):
            if kept[t][j]:
                G[e] = gates_all[t][j]
        y = [0.0] * len(x)
        for e in range(E):
            ye = expert(x, Wg[e], Wu[e], Wd[e])
            y = [a + G[e] * b for a, b in zip(y, ye)]
        for (sg, su, sd) in shared:
            ys = expert(x, sg, su, sd)
            y = [a + b for a, b in zip(y, ys)]
        out.append(y)
    return out
