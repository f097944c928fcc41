"""Closed forms, invariants, exact draw boundaries and a chi-square test that
pin the CPU oracle without reference to its own code.

Semantics: FlashInfer "cake_sampling" page (Semantics; stage 2 description);
nucleus definition: SonicSampler eq. (10).
"""

import math
import struct
from fractions import Fraction

import numpy as np
import pytest
from scipy import stats

import workloads

TWO24, TWO32, TWO64 = 1 << 24, 1 << 32, 1 << 64


def f2b(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def mass(x):
    """floor(min(x, 1) * 2^32) by exact rationals (x a finite fp32 >= 0)."""
    return TWO32 if x >= 1 else math.floor(Fraction(float(x)) * TWO32)


def fixed_p(p):
    p = float(np.float32(p))
    if not p > 0:
        return 1
    if p >= 1:
        return TWO24
    return max(1, round(Fraction(p) * TWO24))


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("n", [1, 2, 3, 10, 100, 1000])
@pytest.mark.parametrize("p", [0.001, 0.3, 0.5, 0.77, 0.95, 1.0])
def test_equal_values_keep_ceil_pn(orc, n, p):
    # n equal masses q: T = ceil(P n q / 2^24) and keeping j while j*q < T
    # keeps ceil(P n / 2^24) entries; ties are kept lowest index first.
    row = np.full(n, 1.0 / n, np.float32)
    P = fixed_p(p)
    want = -(-P * n // TWO24)
    for u in (0, TWO64 - 1, 2**63 + 12345):
        tok, ren, info = orc.sample_row(row, 0, p, u)
        assert info["kept"] == want
        assert np.count_nonzero(ren) == want and np.all(ren[:want] > 0)
        # uniform draw over the kept prefix: position floor(u * want / 2^64)
        assert tok == (u * want) >> 64


def test_p_one_keeps_every_positive_mass(orc):
    rng = np.random.default_rng(3)
    for _ in range(50):
        V = int(rng.integers(1, 400))
        x = rng.random(V).astype(np.float32) ** 8
        x[rng.random(V) < 0.2] = 0.0
        x[rng.random(V) < 0.1] = np.float32(2.0**-40)  # q = 0
        k = int(rng.integers(1, V + 1))
        _, ren, info = orc.sample_row(x, k, 1.0, int(rng.integers(0, 2**63)))
        order = np.argsort(-x, kind="stable")[:k]
        positive = [i for i in order if mass(x[i]) > 0]
        if info["kind"] == 2:
            assert not positive
        else:
            assert info["kept"] == len(positive)
            assert set(np.flatnonzero(ren)) == set(positive)


def test_k_one_is_first_argmax(orc):
    rng = np.random.default_rng(4)
    for _ in range(200):
        V = int(rng.integers(1, 300))
        x = rng.integers(0, 5, size=V).astype(np.float32) / 4
        if rng.random() < 0.3:
            x[rng.integers(0, V)] = np.nan
        san = np.where(np.isnan(x) | np.signbit(x), 0.0, x)
        tok, ren, _ = orc.sample_row(x, 1, float(rng.random()), int(rng.integers(0, 2**63)))
        assert tok == int(np.argmax(san))
        if san.max() > 0:
            assert ren[tok] == 1.0 and np.count_nonzero(ren) == 1


def test_inf_rows_uniform_over_first_infs(orc):
    rng = np.random.default_rng(5)
    for _ in range(100):
        V = int(rng.integers(2, 200))
        x = rng.random(V).astype(np.float32)
        inf_idx = np.sort(rng.choice(V, int(rng.integers(1, min(V, 6) + 1)), replace=False))
        x[inf_idx] = np.inf
        k = int(rng.integers(0, V + 1))
        k_eff = V if k <= 0 else k
        m = min(len(inf_idx), k_eff)
        u = int(rng.integers(0, 2**63)) * 2 + 1
        tok, ren, info = orc.sample_row(x, k, float(rng.random()), u)
        assert info["kind"] == 1 and info["m_inf"] == m
        assert tok == inf_idx[(u * m) >> 64]
        assert np.all(ren[inf_idx[:m]] == np.float32(1.0 / m))
        assert np.count_nonzero(ren) == m


def test_zero_mass_rows_return_smallest_support_index(orc):
    for V in (1, 5, 1000):
        for fill in (0.0, -1.0, np.nan, -0.0, 2.0**-40):
            x = np.full(V, fill, np.float32)
            for k in (0, 1, 3, V):
                tok, ren, info = orc.sample_row(x, k, 0.9, TWO64 - 1)
                assert info["kind"] == 2 and tok == 0 and not ren.any()
    # A row whose positive entries all have q = 0 and sit at high indices:
    # the support is those entries, the token is the smallest of them.
    # The largest of them (index 40) is not the smallest index.
    x = np.zeros(50, np.float32)
    x[[40, 17, 33]] = np.float32(2.0**-34), np.float32(2.0**-35), np.float32(2.0**-36)
    tok, _, info = orc.sample_row(x, 3, 0.5, 12345)
    assert info["kind"] == 2 and tok == 17


def test_sanitised_entries_behave_as_zero(orc):
    rng = np.random.default_rng(6)
    bad = np.array([0x7FC00000, 0xFFC00000, 0x80000000, 0xFF800000, f2b(-0.5), 0x807FFFFF],
                   np.uint32).view(np.float32)
    for _ in range(100):
        V = int(rng.integers(2, 100))
        x = rng.random(V).astype(np.float32)
        pos = rng.choice(V, int(rng.integers(1, V)), replace=False)
        y = x.copy()
        y[pos] = bad[rng.integers(0, bad.size, size=pos.size)]
        z = x.copy()
        z[pos] = 0.0
        k, p, u = int(rng.integers(0, V + 1)), float(rng.random()), int(rng.integers(0, 2**63))
        ty, ry, _ = orc.sample_row(y, k, p, u)
        tz, rz, _ = orc.sample_row(z, k, p, u)
        assert ty == tz and np.array_equal(ry, rz)
        assert np.all(np.isfinite(ry))


def test_masses_closed_form(orc):
    # M_k of a row of distinct powers of two and fp32 fractions equals the
    # exact floor(x * 2^32) sum.
    rng = np.random.default_rng(8)
    for _ in range(100):
        V = int(rng.integers(1, 50))
        x = (rng.random(V) * 2.0 ** rng.integers(-40, 1, size=V)).astype(np.float32)
        _, _, info = orc.sample_row(x, 0, 1.0, 0)
        want = sum(mass(v) for v in x)
        assert info["M_k"] == want if want else info["kind"] == 2


def test_permutation_equivariance_without_ties(orc):
    rng = np.random.default_rng(9)
    for _ in range(100):
        V = int(rng.integers(2, 300))
        x = rng.random(V).astype(np.float32) ** 3
        if len(np.unique(x)) != V:
            continue
        perm = rng.permutation(V)
        k, p, u = int(rng.integers(0, V + 1)), float(rng.random()), int(rng.integers(0, 2**63))
        t1, r1, _ = orc.sample_row(x, k, p, u)
        t2, r2, _ = orc.sample_row(x[perm], k, p, u)
        assert perm[t2] == t1 and np.array_equal(r2, r1[perm])


def test_draw_position_monotone_in_u(orc):
    rng = np.random.default_rng(10)
    x = rng.random(64).astype(np.float32) ** 4
    us = sorted(int(v) * 2 for v in rng.integers(0, 2**63, size=200))
    pos = [orc.sample_row(x, 40, 0.8, u)[2]["pos"] for u in us]
    assert pos == sorted(pos)


# --------------------------------------------------------------------------
# exact draw boundaries
# --------------------------------------------------------------------------
def test_exact_draw_boundaries(orc):
    # The draw maps u to the first kept j with S_incl(j) > floor(u M_p / 2^64).
    # So u_j = ceil(S_excl(j) 2^64 / M_p) is the smallest u drawing position
    # j, and u_j - 1 draws position j - 1.
    rng = np.random.default_rng(11)
    for _ in range(20):
        V = int(rng.integers(2, 60))
        x = (rng.random(V) ** 2).astype(np.float32)
        k = int(rng.integers(1, V + 1))
        _, _, info = orc.sample_row(x, k, 1.0, 0)
        order = np.argsort(-x, kind="stable")[:k]
        q = [mass(x[i]) for i in order][: info["kept"]]
        M_p = info["M_p"]
        assert M_p == sum(q)
        s_excl = 0
        for j, qj in enumerate(q):
            if qj == 0:
                break
            u_j = -(-s_excl * TWO64 // M_p)
            if u_j < TWO64:
                assert orc.sample_row(x, k, 1.0, u_j)[2]["pos"] == j
            if j > 0:
                assert orc.sample_row(x, k, 1.0, u_j - 1)[2]["pos"] == j - 1
            s_excl += qj


# --------------------------------------------------------------------------
# chi-square on seeded draws
# --------------------------------------------------------------------------
@pytest.mark.parametrize("k,p", [(12, 0.9), (0, 1.0), (5, 0.6)])
def test_chi_square_against_renormalised_distribution(orc, k, p):
    rng = np.random.default_rng(12)
    V, n = 20, 100_000
    x = (rng.random(V) ** 3).astype(np.float32)
    x /= x.sum()
    probs = np.broadcast_to(x, (n, V)).copy()
    tok, _, info = orc.sample(probs, np.full(n, k, np.int32), np.full(n, p, np.float32),
                              seed=2024, offset=0, want_info=True)
    kept, M_p = int(info[0, 5]), int(info[0, 6])
    order = np.argsort(-x, kind="stable")[:kept]
    q = np.array([mass(x[i]) for i in order], dtype=np.float64)
    assert int(q.sum()) == M_p
    expected = q / q.sum() * n
    observed = np.array([(tok == i).sum() for i in order], dtype=np.float64)
    assert observed.sum() == n  # nothing outside the kept set
    # merge bins with expected count < 5
    e_m, o_m, acc_e, acc_o = [], [], 0.0, 0.0
    for e, o in sorted(zip(expected, observed)):
        acc_e, acc_o = acc_e + e, acc_o + o
        if acc_e >= 5:
            e_m.append(acc_e)
            o_m.append(acc_o)
            acc_e = acc_o = 0.0
    if acc_e and e_m:
        e_m[-1] += acc_e
        o_m[-1] += acc_o
    if len(e_m) < 2:
        return
    _, pval = stats.chisquare(o_m, e_m)
    assert pval > 1e-4, pval


# --------------------------------------------------------------------------
# invariants on the synthetic workloads
# --------------------------------------------------------------------------
def _check_invariants(w, rows, orc):
    probs = w.probs[rows]
    tok, ren, info = orc.sample(probs, w.top_k[rows], w.top_p[rows], w.seed, w.offset,
                                want_renorm=True, want_info=True)
    assert np.all(np.isfinite(ren))
    for r, b in enumerate(rows):
        d = dict(zip(("k_eff", "P", "m", "M_k", "T", "kept", "M_p", "t", "pos", "kind"), info[r]))
        k_eff = d["k_eff"]
        assert 1 <= k_eff <= w.V and d["kept"] <= k_eff
        assert 1 <= d["P"] <= TWO24 and d["P"] == fixed_p(w.top_p[b])
        nz = np.flatnonzero(ren[r])
        assert tok[r] in nz or d["kind"] == 2
        if d["kind"] == 0:
            assert d["T"] == -(-d["P"] * d["M_k"] // TWO24)
            q_last = mass(probs[r, nz].min()) if nz.size else 0
            # the kept prefix reaches P/2^24 of M_k, and is the shortest one
            assert d["M_p"] * TWO24 >= d["P"] * d["M_k"]
            assert (d["M_p"] - q_last) * TWO24 < d["P"] * d["M_k"]
            assert nz.size == d["kept"]
            assert abs(float(ren[r].astype(np.float64).sum()) - 1.0) <= d["kept"] * 2.0**-23
        if d["kind"] == 2:
            assert not ren[r].any()


@pytest.mark.parametrize("cfg", [1, 2])
def test_invariants_small_configs(orc, cfg):
    w = workloads.make(cfg)
    _check_invariants(w, np.arange(w.B), orc)


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [3, 4])
def test_invariants_sampled_rows_large_configs(orc, cfg):
    w = workloads.make(cfg)
    rows = np.random.default_rng(cfg).choice(w.B, 24, replace=False)
    if cfg == 4:
        cls = w.meta["row_class"]
        rows = np.unique(np.concatenate([rows, np.flatnonzero(cls != "plain")[::3]]))
    _check_invariants(w, rows, orc)
