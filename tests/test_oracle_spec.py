"""Pins of the oracle's speculative verification (SonicSampler appendix C.4,
eqs. (15)-(16), draft-to-target mapping).

* Against the exact-rational brute force (oracle/brute.py) on tiny
  vocabularies: random target rows (special values included) with their own
  top-k / top-p, unnormalised draft rows, random draft tokens, random and
  identity maps, every draft count 0..3.
* The acceptance test at its exact boundary: the largest accepted u is
  floor(num 2^96 / (Q den)) (closed form with Python integers).
* The speculative-sampling property (Leviathan et al., the rule the page
  cites): with the draft token drawn from q, the first output token is
  distributed exactly as the target distribution p, whatever q is.  Checked
  by a chi-square test over 20,000 seeded requests.
* Out-of-range maps and draft tokens mark the request (-1).
"""

import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle.brute import brute_spec_request

TWO64 = 1 << 64


def f2b(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


SPECIAL = [0x7FC00000, 0x80000000, 0xFF800000, f2b(-0.3), 0x00000001, 0x7F800000]


def _row(rng, V, special):
    x = rng.random(V).astype(np.float32)
    x[rng.random(V) < 0.3] = 0.0
    bits = [f2b(float(v)) for v in x]
    if special:
        for i in rng.choice(V, int(rng.integers(1, V + 1)), replace=False):
            bits[i] = int(rng.choice(SPECIAL))
    return bits


def _case(rng, V, L, Lt, special, use_map):
    target = [_row(rng, V, special and rng.random() < 0.3) for _ in range(Lt)]
    ks = [int(rng.integers(0, V + 2)) for _ in range(Lt)]
    ps = [float(rng.choice([0.3, 0.7, 0.95, 1.0])) for _ in range(Lt)]
    draft = [_row(rng, V, special and rng.random() < 0.3) for _ in range(L)]
    tokens = [int(rng.integers(0, V)) for _ in range(L)]
    pi = [int(rng.integers(0, Lt)) for _ in range(L + 1)] if use_map else list(range(L + 1))
    return target, ks, ps, draft, tokens, pi


@pytest.mark.parametrize("special", [False, True])
@pytest.mark.parametrize("use_map", [False, True])
def test_spec_verify_against_brute_force(orc, special, use_map):
    rng = np.random.default_rng(10 + special + 2 * use_map)
    for trial in range(120):
        V = int(rng.integers(1, 7))
        L = int(rng.integers(0, 4))
        Lt = L + 1 + (int(rng.integers(0, 2)) if use_map else 0)
        N = 2
        cases = [_case(rng, V, L, Lt, special, use_map) for _ in range(N)]
        target = np.array([r for c in cases for r in c[0]], np.uint32).view(np.float32)
        ks = np.array([k for c in cases for k in c[1]], np.int32)
        ps = np.array([p for c in cases for p in c[2]], np.float32)
        draft = (np.array([r for c in cases for r in c[3]], np.uint32).view(np.float32)
                 if L else np.zeros((0, V), np.float32))
        toks = np.array([c[4] for c in cases], np.int32).reshape(N, L)
        pi = np.array([c[5] for c in cases], np.int32)
        seed, off = int(rng.integers(0, 2**63)), int(rng.integers(0, 2**40))
        out, acc = orc.spec_verify(target, Lt, ks, ps, draft, toks, pi if use_map else None,
                                   seed, off)
        for n, c in enumerate(cases):
            g0 = n * Lt
            u_draw = [orc.uniform_u64(seed, g0 + j, off) for j in range(Lt)]
            u_acc = [orc.uniform_u64_hi(seed, g0 + j, off) for j in range(Lt)]
            bout, bacc = brute_spec_request(c[0], c[1], c[2], c[3], c[4], c[5], u_draw, u_acc)
            assert out[n].tolist() == bout and acc[n] == bacc, (trial, n, c, out[n], bout)


def test_acceptance_boundary(orc):
    rng = np.random.default_rng(3)
    for _ in range(2000):
        num = int(rng.integers(0, 2**32 + 1))
        den = int(rng.integers(max(num, 1), 2**51))
        Q = int(rng.integers(1, 2**32 + 1))
        # largest accepted u: u Q den <= num 2^96
        umax = (num << 96) // (Q * den)
        for u in (umax - 1, umax, umax + 1, 0, TWO64 - 1):
            if 0 <= u < TWO64:
                want = u * Q * den <= num << 96
                assert orc.lib.oracle_accept_draft(u, Q, den, num) == int(want), (u, Q, den, num)
    # q = 0: every u accepts (u * 0 <= p); p = 0 < q: only u = 0 accepts.
    assert orc.lib.oracle_accept_draft(TWO64 - 1, 0, 5, 0) == 1
    assert orc.lib.oracle_accept_draft(1, 7, 5, 0) == 0
    assert orc.lib.oracle_accept_draft(0, 7, 5, 0) == 1


def test_first_output_is_distributed_as_the_target(orc):
    # Dyadic draft rows (masses sum to exactly 2^32), target rows with top-k
    # and top-p; the draft token is drawn from q by numpy.  The first output
    # token must follow the target's final distribution p exactly.
    from scipy.stats import chisquare

    V, L = 12, 3
    rng = np.random.default_rng(99)
    target = rng.random((L + 1, V)).astype(np.float32)
    ks = np.array([9, 12, 5, 7], np.int32)
    ps = np.array([0.9, 0.8, 1.0, 0.9], np.float32)
    qd = np.array([2.0**-1, 2.0**-2, 2.0**-3, 2.0**-4, 2.0**-5, 2.0**-6, 2.0**-7, 2.0**-8,
                   2.0**-9, 2.0**-10, 2.0**-11, 2.0**-11])
    assert qd.sum() == 1.0
    draft = np.stack([rng.permutation(qd) for _ in range(L)]).astype(np.float32)
    # p_0: the target row 0's final distribution (renorm of the oracle row).
    _, p0, _ = orc.sample_row(target[0], int(ks[0]), float(ps[0]), 0)
    p0 = p0.astype(np.float64)
    p0 /= p0.sum()
    N = 20000
    reqs = 500
    counts = np.zeros(V)
    big_t = np.tile(target, (reqs, 1))
    big_k = np.tile(ks, reqs)
    big_p = np.tile(ps, reqs)
    big_d = np.tile(draft, (reqs, 1))
    for rep in range(N // reqs):
        toks = np.stack([rng.choice(V, p=draft[l].astype(np.float64)) for l in range(L)
                         for _ in range(reqs)]).reshape(L, reqs).T.copy()
        out, acc = orc.spec_verify(big_t, L + 1, big_k, big_p, big_d, toks, None, 5, rep)
        counts += np.bincount(out[:, 0], minlength=V)
    live = p0 > 0
    assert counts[~live].sum() == 0
    stat, pval = chisquare(counts[live], p0[live] * N)
    assert pval > 1e-4, (stat, pval)


def test_out_of_range_map_and_tokens(orc):
    V, L = 5, 2
    target = np.full((3, V), 0.2, np.float32)
    draft = np.full((L, V), 0.2, np.float32)
    ks = np.zeros(3, np.int32)
    ps = np.ones(3, np.float32)
    out, acc = orc.spec_verify(target, 3, ks, ps, draft, [[0, 7]], None, 1, 1)
    assert acc[0] == -1 and out[0].tolist() == [-1, -1, -1]
    out, acc = orc.spec_verify(target, 3, ks, ps, draft, [[0, 1]], [[0, 1, 3]], 1, 1)
    assert acc[0] == -1 and out[0].tolist() == [-1, -1, -1]
    out, acc = orc.spec_verify(target, 3, ks, ps, draft, [[0, 1]], [[2, 2, 2]], 1, 1)
    assert acc[0] >= 0


def test_identical_distributions_accept_everything(orc):
    # p = q exactly (a dyadic row with top-k and top-p off): u q(d) <= p(d)
    # holds for every u, so every draft is accepted and the bonus follows.
    V, L = 8, 4
    row = np.array([2.0**-1, 2.0**-2, 2.0**-3, 2.0**-4, 2.0**-5, 2.0**-6, 2.0**-7, 2.0**-7],
                   np.float32)
    target = np.tile(row, (L + 1, 1))
    draft = np.tile(row, (L, 1))
    rng = np.random.default_rng(1)
    for off in range(50):
        toks = rng.integers(0, V, size=(1, L)).astype(np.int32)
        out, acc = orc.spec_verify(target, L + 1, np.zeros(L + 1, np.int32),
                                   np.ones(L + 1, np.float32), draft, toks, None, 3, off)
        assert acc[0] == L and out[0, :L].tolist() == toks[0].tolist() and out[0, L] >= 0
