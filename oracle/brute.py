"""Brute-force exact-rational reference for tiny rows (TEST INFRASTRUCTURE).

Written from the definitions, not from the C++ oracle, so that the two can
pin each other:

* the support is the set of entries whose *rank* is below k, where rank(i)
  counts entries with a larger value, or an equal value and a lower index
  (the FlashInfer "cake_sampling" page, Semantics: first k of
  lexsort(-prob, index); ties go to the lower vocabulary index).  This is an
  O(V^2) count, no sort;
* values are compared as exact rationals after sanitising (NaN, negative,
  -0.0 become +0; same page, NaN / Inf);
* masses are floor(min(x, 1) * 2^32) evaluated with ``fractions.Fraction``;
* the kept set is the shortest sorted prefix whose inclusive mass reaches
  (P / 2^24) of the top-k mass -- the nucleus of SonicSampler eq. (10),
  taken relative to the top-k mass as in the top-k-first composition;
* the token is the kept entry whose CDF interval [S_excl, S_incl) / M_p
  contains u / 2^64 (inverse CDF), again with exact rationals.

Usable for V up to a few dozen; intended for V <= 10.
"""

from __future__ import annotations

import math
import struct
from fractions import Fraction

TWO24 = 1 << 24
TWO32 = 1 << 32
TWO64 = 1 << 64


def _f32(x) -> float:
    """Round-trip through fp32 so the value is exactly the stored float."""
    return struct.unpack("<f", struct.pack("<f", float(x)))[0]


def _from_bits(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0]


def sanitized_value(x: float):
    """+0 for NaN and for anything carrying a sign bit; math.inf stays inf."""
    if math.isnan(x) or math.copysign(1.0, x) < 0:
        return Fraction(0)
    if math.isinf(x):
        return math.inf
    return Fraction(x)


def _greater(a, b) -> bool:
    if a is math.inf:
        return b is not math.inf
    if b is math.inf:
        return False
    return a > b


def fixed_p(p: float) -> int:
    p = _f32(p)
    if math.isnan(p) or p <= 0:
        return 1
    if p >= 1:
        return TWO24
    r = round(Fraction(p) * TWO24)  # Python rounds half to even
    return max(1, int(r))


def brute_support(row_bits, k: int):
    """The support in its order: the indices whose rank (the number of
    entries with a larger sanitised value, or an equal one at a lower index)
    is below k_eff, by ascending rank.  No sort is involved."""
    vals = [sanitized_value(_from_bits(int(v))) for v in row_bits]
    V = len(vals)
    k_eff = V if (k <= 0 or k >= V) else k
    rank = []
    for i in range(V):
        r = 0
        for j in range(V):
            if _greater(vals[j], vals[i]) or (vals[j] == vals[i] and j < i):
                r += 1
        rank.append(r)
    order = [None] * k_eff
    for i in range(V):
        if rank[i] < k_eff:
            order[rank[i]] = i
    return order


def brute_row(row_bits, k: int, p: float, u: int, min_p: float = 0.0):
    """Return (token, kept indices in sorted order, weights as Fractions).

    ``row_bits`` is a sequence of fp32 bit patterns (ints), so NaN payloads,
    -0.0 and denormals reach this function unchanged.  ``min_p`` (theta) is
    the min-p floor of SonicSampler eq. (11) on the fixed-point masses: an
    entry of the support stays only if q_i >= theta * max q (exact rational
    comparison), applied after top-k and top-p (the kept set is the
    intersection of the two sets); theta NaN or <= 0 is off, > 1 counts as 1.
    """
    xs = [_from_bits(int(v)) for v in row_bits]
    V = len(xs)
    vals = [sanitized_value(x) for x in xs]
    k_eff = V if (k <= 0 or k >= V) else k

    rank = []
    for i in range(V):
        r = 0
        for j in range(V):
            if _greater(vals[j], vals[i]) or (vals[j] == vals[i] and j < i):
                r += 1
        rank.append(r)
    support = sorted((i for i in range(V) if rank[i] < k_eff), key=lambda i: rank[i])

    infs = [i for i in support if vals[i] is math.inf]
    if infs:
        m = len(infs)
        # u / 2^64 falls in [t/m, (t+1)/m)
        t = next(t for t in range(m) if Fraction(u, TWO64) < Fraction(t + 1, m))
        return infs[t], infs, [Fraction(1, m)] * m

    def mass(v):
        return TWO32 if v >= 1 else math.floor(v * TWO32)

    q = [mass(vals[i]) for i in support]
    M_k = sum(q)
    if M_k == 0:
        return min(support), [], []

    target = Fraction(fixed_p(p), TWO24) * M_k
    n = next(n for n in range(1, len(support) + 1) if sum(q[:n]) >= target)
    theta = _f32(min_p)
    if not math.isnan(theta) and theta > 0:
        floor_mass = Fraction(min(theta, 1.0)) * max(q)
        keep = [j for j in range(n) if q[j] >= floor_mass]  # the intersection
        n = len(keep)
        assert keep == list(range(n)), "the min-p set is a prefix of the sorted support"
    kept = support[:n]
    M_p = sum(q[:n])
    x = Fraction(u, TWO64)
    acc = 0
    for j in range(n):
        lo, hi = Fraction(acc, M_p), Fraction(acc + q[j], M_p)
        acc += q[j]
        if lo <= x < hi:
            return kept[j], kept, [Fraction(qj, M_p) for qj in q[:n]]
    raise AssertionError("u outside [0, 1)")


def _mass(v):
    """floor(min(v, 1) * 2^32) of a sanitised value (Fraction or inf)."""
    if v is math.inf or v >= 1:
        return TWO32
    return math.floor(v * TWO32)


def brute_spec_request(target_bits, ks, ps, draft_bits, tokens, pi, u_draw, u_acc):
    """Speculative verification of one request with exact rationals
    (SonicSampler appendix C.4, eqs. (15)-(16)).

    target_bits[j] (fp32 bit patterns), ks[j], ps[j]: the request's target
    rows; draft_bits[l], tokens[l]: draft distribution and token of position
    l < L; pi[l] (l <= L): the target row of position l; u_draw[j] / u_acc[j]:
    the 64-bit uniforms of target row j (its own draw / the acceptance test).
    p_j = row j's final distribution (brute_row's kept weights; a zero-mass
    row is the point mass on its token); q_l(x) = floor(min(y, 1) 2^32) / 2^32.
    Position l's draft is accepted iff (u / 2^64) q_l(d) <= p(d); the first
    rejection draws from max(0, p - q_l) normalised, by interval containment
    of u_draw / 2^64 in vocabulary order (its own token if that is all zero);
    with every draft accepted, the bonus is row pi[L]'s own token.
    Returns (out tokens of length L + 1, accepted count)."""
    L = len(tokens)
    out = [-1] * (L + 1)
    for l in range(L + 1):
        j = pi[l]
        tok, kept, w = brute_row(target_bits[j], ks[j], ps[j], u_draw[j])
        p = dict(zip(kept, w)) if kept else {tok: Fraction(1)}
        if l == L:
            out[L] = tok
            return out, L
        ys = [sanitized_value(_from_bits(int(v))) for v in draft_bits[l]]
        q = [Fraction(_mass(y), TWO32) for y in ys]
        d = tokens[l]
        if Fraction(u_acc[j], TWO64) * q[d] <= p.get(d, Fraction(0)):
            out[l] = d
            continue
        r = [max(Fraction(0), p.get(x, Fraction(0)) - q[x]) for x in range(len(q))]
        R = sum(r)
        if R == 0:
            out[l] = tok
        else:
            u = Fraction(u_draw[j], TWO64)
            acc = Fraction(0)
            for x in range(len(r)):
                if acc / R <= u < (acc + r[x]) / R:
                    out[l] = x
                    break
                acc += r[x]
        return out, l
    raise AssertionError("unreachable")
