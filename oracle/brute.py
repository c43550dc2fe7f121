"""Pure-Python loop version of the path for tiny inputs (TEST INFRASTRUCTURE ONLY).

Written independently of oracle.py (no NumPy arithmetic, no shared helpers):
lists of floats, explicit loops, Python's own sort on (-score, position) keys.
Used to pin the NumPy oracle on n <= a few dozen compressed positions.
Definitions as in oracle.py's header ("DeepSeek-V4.1 Flash" section 1 Model
Introduction; "deepseek-ai/DeepSeek-V4.1-Flash" recipe, Overview, two-tier
sparse attention bullet).
"""
from __future__ import annotations

import math


def scores(qI, w, keys):
    """qI: 16 lists of 128 floats; w: 16 floats; keys: n lists of 128 floats."""
    out = []
    for k in keys:
        total = 0.0
        for h in range(len(qI)):
            d = 0.0
            for c in range(len(k)):
                d += qI[h][c] * k[c]
            if d > 0.0:
                total += w[h] * d
        out.append(total)
    return out


def select(I, k=512, cb=2048, blk=8):
    n = len(I)
    blocks = []
    for b in range((n + blk - 1) // blk):
        best = None
        for j in range(b * blk, min(n, b * blk + blk)):
            if best is None or I[j] > best:
                best = I[j]
        blocks.append((-best, b))
    blocks.sort()
    kept = sorted(b for _, b in blocks[:cb])
    cand = []
    for b in kept:
        for j in range(b * blk, min(n, b * blk + blk)):
            cand.append((-I[j], j))
    cand.sort()
    return kept, sorted(j for _, j in cand[:k])


def rescore(qI, w, keys, cand, n, k=512, blk=8):
    """Scores of the visible positions of candidate blocks `cand` only, then the first k by
    (-score, position), ascending. keys: n lists of floats."""
    pos = []
    for b in cand:
        if b < 0:
            continue
        for r in range(blk):
            if b * blk + r < n:
                pos.append(b * blk + r)
    s = scores(qI, w, [keys[p] for p in pos])
    ranked = sorted(zip([-v for v in s], pos))
    return sorted(p for _, p in ranked[:k])


def attend(q, X, scale):
    """q: H lists of D floats; X: m lists of D floats -> (o: H x D, lse: H)."""
    o, lse = [], []
    for qh in q:
        s = []
        for x in X:
            acc = 0.0
            for c in range(len(x)):
                acc += qh[c] * x[c]
            s.append(scale * acc)
        mu = max(s)
        e = [math.exp(v - mu) for v in s]
        Z = sum(e)
        row = [0.0] * len(X[0])
        for i, x in enumerate(X):
            p = e[i] / Z
            for c in range(len(x)):
                row[c] += p * x[c]
        o.append(row)
        lse.append(mu + math.log(Z))
    return o, lse


def compress_pair(x0, x1, z0, z1, b0, b1):
    """Per-channel two-slot softmax gate: lists of D floats -> D floats."""
    out = []
    for c in range(len(x0)):
        a0 = z0[c] + b0[c]
        a1 = z1[c] + b1[c]
        m = a0 if a0 > a1 else a1
        e0 = math.exp(a0 - m)
        e1 = math.exp(a1 - m)
        out.append((e0 * x0[c] + e1 * x1[c]) / (e0 + e1))
    return out
