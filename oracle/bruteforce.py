"""Exhaustive router for tiny layers, in exact rational arithmetic.

TEST INFRASTRUCTURE ONLY.  It pins the C oracle's router (oracle.route) by a
different route to the same answer:

  * scores are the correctly rounded binary32 sigmoid, evaluated in 60-digit
    decimal arithmetic (not the oracle's binary64 sequence);
  * a group's score is the largest binary32 sum over all pairs of its biased
    scores (rounding is monotone, so this is the sum of its two largest),
    or its largest biased score when one score is summed;
  * the kept groups are the subset of the required size whose exact sum of
    group scores is largest, the lexicographically first among equals;
  * the experts are the subset of the eligible experts whose exact sum of
    biased scores is largest, the lexicographically first among equals, then
    listed by biased score (descending) and index;
  * weights: binary32 sum of the chosen unbiased scores in that order, then
    binary32 (s / D) * scale.

The method is the group-limited router of "Reflection Releases Beam ...",
section "Where Beam Saves and Where the Memory Bill Comes In", and of
"Reflection Beam", section "What Beam is"; the group-score rule is
DeepSeek-V3's (arXiv 2412.19437, section 2.1.2), which those sections invoke.
Cost is C(G, TG) * C(TG*E/G, K) subsets per token: keep layers tiny.
"""
from __future__ import annotations

import itertools
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

_PREC = 60


def exact_sigmoid(l: float) -> Fraction:
    """1 / (1 + e^-l) to about 60 significant digits, as a Fraction."""
    getcontext().prec = _PREC
    d = Decimal(1) / (Decimal(1) + (-Decimal(float(l))).exp())
    return Fraction(d)


def nearest_f32(q: Fraction):
    """Round a non-negative rational to binary32, nearest, ties to even.
    Returns (value, distance to the nearest rounding boundary / q)."""
    if q == 0:
        return np.float32(0.0), Fraction(1)
    c = np.float32(float(q))
    cands = {c, np.nextafter(c, np.float32(np.inf)),
             np.nextafter(c, np.float32(-np.inf))}
    cands = [v for v in cands if np.isfinite(v) and v >= 0]
    best = None
    for v in cands:
        d = abs(Fraction(float(v)) - q)
        if best is None or d < best[0] or (
                d == best[0] and (int(v.view(np.uint32)) & 1) == 0):
            best = (d, v)
    v = best[1]
    # distance to the midpoints on either side of v
    lo = np.nextafter(v, np.float32(-np.inf))
    hi = np.nextafter(v, np.float32(np.inf))
    mids = [(Fraction(float(v)) + Fraction(float(n))) / 2 for n in (lo, hi)
            if np.isfinite(n) and n >= 0]
    margin = min(abs(q - m) for m in mids) / q
    return v, margin


def sigmoid32_exact(l: float):
    """Correctly rounded binary32 sigmoid and its relative midpoint margin."""
    return nearest_f32(exact_sigmoid(l))


def route_token(shape, logits_row, bias=None, topn: int = None):
    E, G = shape.n_experts, shape.n_groups
    gs, TG, K = E // G, shape.topk_groups, shape.top_k
    topn = getattr(shape, "group_score_topn", 2) if topn is None else topn
    if topn not in (1, 2):
        raise ValueError("brute force covers one- or two-score group sums")
    f32 = np.float32
    s = [sigmoid32_exact(float(v))[0] for v in np.asarray(logits_row, f32)]
    b = [f32(0)] * E if bias is None else [f32(v) for v in np.asarray(bias, f32)]
    u = [f32(s[e] + b[e]) for e in range(E)]
    Gs = []
    for g in range(G):
        mem = range(g * gs, (g + 1) * gs)
        if topn == 1:
            Gs.append(max(u[e] for e in mem))
        else:
            Gs.append(max(f32(u[i] + u[j]) for i, j in itertools.combinations(mem, 2)))
    best, best_v = None, None
    for comb in itertools.combinations(range(G), TG):      # lexicographic order
        v = sum(Fraction(float(Gs[g])) for g in comb)
        if best is None or v > best_v:
            best, best_v = comb, v
    elig = [e for g in best for e in range(g * gs, (g + 1) * gs)]
    elig.sort()
    bestE, bestE_v = None, None
    for comb in itertools.combinations(elig, K):
        v = sum(Fraction(float(u[e])) for e in comb)
        if bestE is None or v > bestE_v:
            bestE, bestE_v = comb, v
    order = sorted(bestE, key=lambda e: (-Fraction(float(u[e])), e))
    D = s[order[0]]
    for e in order[1:]:
        D = f32(D + s[e])
    scale = f32(getattr(shape, "routed_scale", 2.5))
    w = [f32(f32(s[e] / D) * scale) for e in order]
    kept = sorted(best, key=lambda g: (-Fraction(float(Gs[g])), g))
    return (np.array(order, np.int32), np.array(w, np.float32),
            np.array(kept, np.int32))


def route(shape, logits, bias=None):
    out = [route_token(shape, row, bias) for row in np.asarray(logits, np.float32)]
    return (np.stack([o[0] for o in out]), np.stack([o[1] for o in out]),
            np.stack([o[2] for o in out]))
