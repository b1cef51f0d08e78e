"""Pure-Python brute force for tiny SFA shapes.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle.sfa``).  This is a second,
deliberately different formulation used to pin ``oracle.sfa``:

* visibility is written in (token, stream) coordinates, not as index arithmetic
  on the expanded position;
* the softmax is taken without the max shift, with ``math.exp`` on Python
  floats, accumulating in plain loops.

"Hidden Decoding at Scale" review, *Method*: within-stream layers read only
their own stream; mixing layers use the base model's full causal pattern over
the length-nL sequence (interleaved token-major, stream 0 first).
"""
from __future__ import annotations

import math


def sees(t, s, t2, s2, within):
    """Does query (token t, stream s) read key (token t2, stream s2)?"""
    if within:
        return s2 == s and t2 <= t
    return t2 < t or (t2 == t and s2 <= s)


def window_members(t, s, n, window):
    """The (token, stream) pairs inside a sliding window of ``window``
    positions ending at (t, s), found by walking back through the interleaved
    order one position at a time (stream s, s-1, ..., 0, then the previous
    token's stream n-1, ...).  Review, *Method*: mixing layers follow the base
    model's sliding-window pattern over the expanded sequence."""
    out = set()
    tt, ss = t, s
    for _ in range(window):
        if tt < 0:
            break
        out.add((tt, ss))
        ss -= 1
        if ss < 0:
            tt, ss = tt - 1, n - 1
    return out


def brute_attention(q, k, v, n, within, scale, window=None):
    """q[b][p][h][d], k/v[b][p][g][d] as nested Python float lists, p = t*n+s.
    ``window`` (mixing only): sliding window in positions.
    Returns out[b][p][h][d]."""
    B = len(q)
    N = len(q[0])
    Hq = len(q[0][0])
    Hkv = len(k[0][0])
    D = len(q[0][0][0])
    G = Hq // Hkv
    L = N // n
    out = []
    for b in range(B):
        ob = []
        for t in range(L):
            for s in range(n):
                p = t * n + s
                inside = None if window is None else window_members(t, s, n, window)
                oh = []
                for h in range(Hq):
                    g = h // G
                    wsum = 0.0
                    acc = [0.0] * D
                    for t2 in range(L):
                        for s2 in range(n):
                            if not sees(t, s, t2, s2, within):
                                continue
                            if inside is not None and (t2, s2) not in inside:
                                continue
                            p2 = t2 * n + s2
                            dot = 0.0
                            for d in range(D):
                                dot += q[b][p][h][d] * k[b][p2][g][d]
                            w = math.exp(scale * dot)
                            wsum += w
                            for d in range(D):
                                acc[d] += w * v[b][p2][g][d]
                    oh.append([a / wsum for a in acc])
                ob.append(oh)
        out.append(ob)
    return out


def brute_expand(ids, tables):
    """out[b][t*n+s] = tables[s][ids[b][t]] for nested lists; None rows for an
    id outside the table (the caller decides what that means)."""
    n = len(tables)
    out = []
    for row in ids:
        o = []
        for tok in row:
            for s in range(n):
                if 0 <= tok < len(tables[s]):
                    o.append(list(tables[s][tok]))
                else:
                    o.append(None)
        out.append(o)
    return out
