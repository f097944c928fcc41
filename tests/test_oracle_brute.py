"""Pin the C++ oracle against the exact-rational brute force on tiny rows.

The brute force (oracle/brute.py) defines the support by an O(V^2) rank
count, compares sanitised values as rationals, finds the kept prefix as the
shortest prefix reaching (P / 2^24) of the top-k mass and draws by interval
containment of u / 2^64.  The C++ oracle uses a stable sort, 64/128-bit
fixed point and floor/compare arithmetic.  Agreement on every case below --
ties, NaN payloads, -0.0, negatives, denormals, +inf, values >= 1, masses
below 2^-32, every k from -1 to V+1, p on exact boundaries, u at both ends
-- pins tokens, kept sets and renormalised weights.
"""

import struct

import numpy as np
import pytest

from oracle.brute import brute_row, brute_support

TWO64 = 1 << 64


def f2b(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


# fp32 bit patterns that exercise every sanitising and mass rule.
SPECIAL = [
    0x00000000,  # +0
    0x80000000,  # -0.0
    0x7FC00000,  # qNaN
    0xFFC00000,  # -qNaN
    0x7F800001,  # sNaN
    0xFF800000,  # -inf
    0x00000001,  # smallest denormal
    0x807FFFFF,  # negative denormal
    f2b(2.0**-33),  # positive, q = 0
    f2b(2.0**-32),  # q = 1
    f2b(3 * 2.0**-33),  # q = 1 (floor of 1.5)
    f2b(-0.25),
    f2b(1.0),
    f2b(1.5),  # > 1: q saturates at 2^32
]
PLAIN = [f2b(x) for x in (0.5, 0.25, 0.125, 0.0625, 0.3, 0.1, 0.1, 0.7, 1e-3, 1e-7)]


def _rows(rng, n, V, pool, with_inf=False):
    rows = []
    for _ in range(n):
        r = [int(pool[i]) for i in rng.integers(0, len(pool), size=V)]
        if with_inf:
            for i in rng.choice(V, int(rng.integers(1, V + 1)), replace=False):
                r[i] = 0x7F800000
        rows.append(r)
    return rows


U_GRID = [0, 1, 2**63, TWO64 - 1, 0x5555555555555555, 0xFEDCBA9876543210]
P_GRID = [0.0, -1.0, float("nan"), 1e-9, 0.25, 0.5, 0.5 + 2**-24, 0.75, 0.9, 0.999, 1.0, 2.0]


def _check(orc, bits, k, p, u):
    row = np.array(bits, dtype=np.uint32).view(np.float32)
    tok, ren, info = orc.sample_row(row, k, p, u)
    btok, bkept, bw = brute_row(bits, k, p, u)
    assert tok == btok, (bits, k, p, u)
    kept_mask = np.zeros(len(bits), bool)
    kept_mask[bkept] = True
    assert np.all(ren[~kept_mask] == 0.0), (bits, k, p, u)
    for i, w in zip(bkept, bw):
        exact = float(w)
        assert abs(float(ren[i]) - exact) <= 2.0**-23 * exact, (bits, k, p, u, i)
    return info


@pytest.mark.parametrize("V", [1, 2, 3, 5, 8])
def test_plain_and_special_rows(orc, V):
    rng = np.random.default_rng(100 + V)
    rows = _rows(rng, 12, V, PLAIN + SPECIAL) + _rows(rng, 6, V, PLAIN)
    for bits in rows:
        for k in range(-1, V + 2):
            for p in P_GRID[:: 1 if V <= 3 else 3]:
                for u in U_GRID[:: 1 if V <= 3 else 2]:
                    _check(orc, bits, k, p, u)


@pytest.mark.parametrize("V", [2, 4, 7])
def test_rows_with_infinities(orc, V):
    rng = np.random.default_rng(200 + V)
    for bits in _rows(rng, 10, V, PLAIN + SPECIAL, with_inf=True):
        for k in range(0, V + 1):
            for u in U_GRID:
                info = _check(orc, bits, k, 0.9, u)
                assert info["kind"] == 1


def test_heavy_ties(orc):
    # Many equal values: ties must go to the lower index in the support, in
    # the kept prefix and in the draw.
    rng = np.random.default_rng(7)
    pool = [f2b(0.125), f2b(0.125), f2b(0.25), 0]
    for bits in _rows(rng, 40, 8, pool):
        for k in (1, 2, 3, 5, 8):
            for p in (0.3, 0.5, 0.625, 0.9, 1.0):
                for u in U_GRID:
                    _check(orc, bits, k, p, u)


def test_exact_p_boundaries(orc):
    # Row masses 2^31, 2^30, 2^29, 2^29 (sum 2^32): p = 0.5, 0.75, 0.875 make
    # the inclusive prefix mass equal p * M_k exactly; one more 2^-24 step
    # must take the next entry.
    bits = [f2b(0.5), f2b(0.25), f2b(0.125), f2b(0.125)]
    expect = {0.5: 1, 0.5 + 2**-24: 2, 0.75: 2, 0.75 + 2**-24: 3, 0.875: 3, 0.875 + 2**-24: 4,
              1.0: 4}
    for p, n in expect.items():
        for u in U_GRID:
            info = _check(orc, bits, 0, p, u)
            assert info["kept"] == n, (p, info)


def test_p_rounds_half_to_even(orc):
    # p * 2^24 = 5033165.5 exactly (p in [0.25, 0.5) has half-integer steps).
    # Half-to-even gives P = 5033166; the top entry holds exactly 5033165/2^24
    # of the mass, so P = 5033166 must keep a second entry (truncation to
    # 5033165 would stop at one).
    top = 5033165
    rest = [2936012, 2936013, 2936013, 2936013]
    assert top + sum(rest) == 2**24
    bits = [f2b(v * 2.0**-24) for v in [top] + rest]
    p = 5033165.5 * 2.0**-24
    assert float(np.float32(p)) == p
    for u in U_GRID:
        info = _check(orc, bits, 0, p, u)
        assert info["P"] == 5033166 and info["kept"] == 2
    # one fp32 step lower: p * 2^24 = 5033165 exactly -> one entry
    info = _check(orc, bits, 0, 5033165 * 2.0**-24, 0)
    assert info["kept"] == 1


def test_random_tiny_rows(orc):
    rng = np.random.default_rng(31)
    for _ in range(300):
        V = int(rng.integers(1, 11))
        x = rng.random(V).astype(np.float32)
        x[rng.random(V) < 0.3] = x[0]  # inject ties
        bits = [int(b) for b in x.view(np.uint32)]
        k = int(rng.integers(-1, V + 2))
        p = float(rng.random())
        u = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        _check(orc, bits, k, p, u)


def _support(orc, row, k, cap):
    import numpy as np

    row = np.ascontiguousarray(row, dtype=np.float32)
    out = np.full(max(cap, 1), -7, np.int32)
    k_eff = int(orc.lib.oracle_support(row.ctypes.data, row.size, int(k), cap, out.ctypes.data))
    return k_eff, out[: min(k_eff, cap)].tolist()


def test_support_order_matches_rank_definition(orc):
    # The exported support order (the slab order: descending probability,
    # ascending index) against the O(V^2) rank definition, on rows of special
    # values with heavy ties, for every k.
    rng = np.random.default_rng(77)
    for trial in range(120):
        V = int(rng.integers(1, 9))
        bits = [int(SPECIAL[i]) for i in rng.integers(0, len(SPECIAL), size=V)]
        row = np.array(bits, np.uint32).view(np.float32)
        for k in range(-1, V + 2):
            want = brute_support(bits, k)
            k_eff, got = _support(orc, row, k, V)
            assert k_eff == len(want)
            assert got == want, (bits, k)


def test_support_order_matches_lexsort(orc):
    # Library cross-check on larger rows: numpy's lexsort by (-value, index)
    # of the sanitised values, truncated to k and to the capacity.
    rng = np.random.default_rng(78)
    for V, k, cap in ((1000, 50, 64), (5000, 700, 1024), (4096, 4096, 1024), (300, 0, 512)):
        x = np.round(rng.random(V) * 64).astype(np.float32) / 64  # many ties
        x[rng.choice(V, 5, replace=False)] = np.nan
        x[rng.choice(V, 5, replace=False)] = -1.0
        vals = np.where(np.isnan(x) | (np.signbit(x)), 0.0, x).astype(np.float64)
        order = np.lexsort((np.arange(V), -vals))
        k_eff = V if (k <= 0 or k >= V) else k
        got_k, got = _support(orc, x, k, cap)
        assert got_k == k_eff
        assert got == order[: min(k_eff, cap)].tolist()
