"""Pins of the oracle's logit rows (temperature, weights) and min-p.

* E(s), the fp32 exponential of the logit weights, against the exact
  exponential of the same fp32 argument (Python's decimal module, whose exp is
  correctly rounded): within one fp32 ulp of the exact value, exactly 1 at
  s = 0 and exactly 0 where the definition cuts off.
* The weights of a logit row against exp((x - max) / tau) computed in float64,
  with an error bound from the three fp32 roundings before E; the special
  rules (NaN and -inf weigh 0, the maximum weighs 1, +inf rows, all-masked
  rows, tau -> 0 and tau = +inf).
* Min-p against the exact-rational brute force (oracle/brute.py, written
  from SonicSampler eq. (11)) on tiny rows, with the floor theta * q_max
  landing exactly on and between masses, every k, and p values that make
  top-p or min-p the shorter cut.
* Eq. (12): on logit rows, the min-p set equals {x >= max + tau ln theta}
  except for entries within the weights' rounding of that threshold.
* The sampled distribution of logit rows against the exact softmax(x / tau)
  (float64), truncated by top-k and top-p, by a chi-square test over 10^5
  seeded draws.
"""

import decimal
import math
import struct

import numpy as np
import pytest

from oracle.brute import brute_row

decimal.getcontext().prec = 60
INF = float("inf")


def f32(x):
    return float(np.float32(x))


def ulp32(v):
    m, e = math.frexp(v)
    return 2.0 ** (e - 24)


def test_exp_weight_within_one_ulp(orc):
    rng = np.random.default_rng(0)
    s = np.concatenate([
        -rng.uniform(0, 86, 20000),
        -np.exp(rng.uniform(-25, math.log(86), 8000)),
        # arguments near the reduction boundaries (n ln 2 +- 0.5 ln 2) and
        # the largest |n| that still gives a weight
        np.array([-(n + h) * math.log(2) for n in range(0, 126) for h in (0.49, 0.5, 0.51)]),
    ]).astype(np.float32)
    worst = 0.0
    for v in s:
        e = orc.exp_weight(float(v))
        exact = decimal.Decimal(float(v)).exp()
        if exact < decimal.Decimal(2.0**-125):
            continue  # cut-off region, checked below
        err = float(abs(decimal.Decimal(e) - exact)) / ulp32(float(exact))
        worst = max(worst, err)
        assert err <= 1.0, (float(v), e, float(exact), err)
    assert worst > 0.3  # the test does reach rounding differences


def test_exp_weight_special_values(orc):
    assert orc.exp_weight(0.0) == 1.0
    assert orc.exp_weight(-0.0) == 1.0
    assert orc.exp_weight(-1e-30) == 1.0
    assert orc.exp_weight(-INF) == 0.0
    assert orc.exp_weight(float("nan")) == 0.0
    assert orc.exp_weight(-200.0) == 0.0
    # Nothing subnormal: the smallest nonzero weight is at least 2^-126.
    for v in np.linspace(-90, -85, 2001).astype(np.float32):
        e = orc.exp_weight(float(v))
        assert e == 0.0 or e >= 2.0**-126
    # Weights never exceed 1 for s <= 0 (every argument: the exhaustive scan
    # below).
    grid = -np.linspace(0, 87, 20001).astype(np.float32)
    w = np.array([orc.exp_weight(float(v)) for v in grid])
    assert np.all(w <= 1.0)


def test_logit_weights_against_float64_softmax(orc):
    rng = np.random.default_rng(1)
    for tau in (1.0, 0.7, 0.25, 1.7, 3.0):
        x = (3.0 * rng.standard_normal(4000)).astype(np.float32)
        x[rng.choice(4000, 5, replace=False)] += 12.0
        w = orc.logit_weights(x, tau)
        M = float(x.max())
        s = (x.astype(np.float64) - M) / float(np.float32(tau))
        ref = np.exp(s)
        # fl(x - M), fl(.*r) and r itself each add at most 2^-24 relative to
        # s, which moves exp(s) by |s| times that; E adds one ulp.
        tol = (3 * 2.0**-24) * np.abs(s) * ref + 2.0**-23 * ref
        live = ref >= 2.0**-120
        assert np.all(np.abs(w[live] - ref[live]) <= tol[live]), tau
        assert np.all(w[~live] <= 2.0**-119)
        assert w[np.argmax(x)] == 1.0


def test_logit_weight_rules(orc):
    x = np.array([1.0, np.nan, -np.inf, 3.0, 3.0, -2.0], np.float32)
    w = orc.logit_weights(x, 1.0)
    assert w[1] == 0 and w[2] == 0 and w[3] == 1 and w[4] == 1
    assert 0 < w[0] < 1 and 0 < w[5] < w[0]
    # tau -> 0 (tau <= 0 or NaN): weight 1 on every maximum, 0 elsewhere.
    for tau in (0.0, -1.0, float("nan"), 1e-45):
        assert orc.logit_weights(x, tau).tolist() == [0, 0, 0, 1, 1, 0], tau
    # tau = +inf: every finite entry weighs 1, masked entries 0.
    assert orc.logit_weights(x, INF).tolist() == [1, 0, 0, 1, 1, 1]
    # +inf logits: weight +inf on them, 0 elsewhere (the +inf-row rule).
    y = np.array([5.0, np.inf, 1.0, np.inf], np.float32)
    assert orc.logit_weights(y, 0.8).tolist() == [0, INF, 0, INF]
    # Every entry masked: all weights 0 (a zero-mass row).
    z = np.array([-np.inf, np.nan, -np.inf], np.float32)
    assert orc.logit_weights(z, 1.0).tolist() == [0, 0, 0]


def f2b(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def _minp_rows(rng):
    rows = []
    # masses on a grid so that theta * q_max lands exactly on some of them
    base = [0.5, 0.25, 0.125, 0.0625, 0.2, 0.1, 0.1, 0.05, 0.3]
    for _ in range(30):
        V = int(rng.integers(1, 9))
        rows.append([f2b(float(v)) for v in rng.choice(base, V)])
    for _ in range(10):
        V = int(rng.integers(2, 9))
        rows.append([f2b(float(v)) for v in rng.random(V).astype(np.float32)])
    return rows


@pytest.mark.parametrize("theta", [0.0, -0.5, float("nan"), 1e-9, 0.1, 0.2, 0.25, 0.4, 0.5,
                                   0.5 + 2**-24, 0.6, 0.999, 1.0, 3.0])
def test_min_p_against_brute_force(orc, theta):
    rng = np.random.default_rng(7)
    us = [0, 2**63, 2**64 - 1, 0x5555555555555555]
    for bits in _minp_rows(rng):
        V = len(bits)
        row = np.array(bits, np.uint32).view(np.float32)
        for k in range(0, V + 2):
            for p in (0.3, 0.8, 1.0):
                for u in us:
                    tok, ren, _ = orc.sample_row(row, k, p, u, min_p=theta)
                    btok, bkept, bw = brute_row(bits, k, p, u, min_p=theta)
                    assert tok == btok, (bits, k, p, theta, u)
                    mask = np.zeros(V, bool)
                    mask[bkept] = True
                    assert np.all(ren[~mask] == 0), (bits, k, p, theta)
                    for i, wv in zip(bkept, bw):
                        assert abs(float(ren[i]) - float(wv)) <= 2.0**-23 * float(wv)


def test_min_p_floor_exactly_on_a_mass(orc):
    # q = (2^31, 2^30, 2^30 - 2^6): theta = 0.5 puts the floor exactly on
    # 2^30, which stays; the next float below it goes.
    row = np.array([0.5, 0.25, np.nextafter(np.float32(0.25), np.float32(0))], np.float32)
    tok, ren, info = orc.sample_row(row, 0, 1.0, 2**64 - 1, min_p=0.5)
    assert info["kept"] == 2 and ren[2] == 0 and ren[1] > 0
    tok, ren, info = orc.sample_row(row, 0, 1.0, 2**64 - 1, min_p=np.float32(0.5 + 2**-24))
    assert info["kept"] == 1
    # An odd q_max: theta * q_max = 2^22 + 1/2 is not an integer, so the
    # floor is 2^22 + 1 (the ceiling): q = 2^22 + 1 stays, q = 2^22 goes.
    q0 = 2**23 + 1
    row = np.array([q0 * 2.0**-32, (2**22 + 1) * 2.0**-32, 2**22 * 2.0**-32], np.float32)
    assert [int(np.floor(np.float64(v) * 2**32)) for v in row] == [q0, 2**22 + 1, 2**22]
    tok, ren, info = orc.sample_row(row, 0, 1.0, 0, min_p=0.5)
    assert info["kept"] == 2 and ren[2] == 0


def test_min_p_equals_logit_threshold_eq12(orc):
    # With top-k and top-p off, the kept set of a logit row under min-p theta
    # is {x : x >= M + tau ln theta} (SonicSampler eq. (12)), up to entries
    # whose logit lies within the weights' rounding of that threshold.
    rng = np.random.default_rng(12)
    for trial in range(40):
        V = 3000
        tau = float(np.float32(rng.choice([0.5, 1.0, 1.3])))
        theta = float(np.float32(rng.choice([1e-4, 0.01, 0.05, 0.2, 0.7])))
        x = (2.0 * rng.standard_normal(V)).astype(np.float32)
        x[rng.choice(V, 3, replace=False)] += 6.0
        tok, ren, _ = orc.sample_logits(x[None, :], [V], [1.0], [tau], [theta], 3, trial,
                                        want_renorm=True)
        kept = ren[0] != 0
        M = float(x.max())
        thr = M + tau * math.log(theta)
        near = np.abs(x.astype(np.float64) - thr) <= 1e-5 * max(1.0, abs(thr))
        want = x.astype(np.float64) >= thr
        assert np.array_equal(kept[~near], want[~near]), trial


def test_logit_rows_sample_the_truncated_softmax(orc):
    # 10^5 draws (one per offset) from one logit row: the histogram matches
    # softmax(x / tau) restricted to the top-k / top-p set and renormalised,
    # all computed here in float64 from the textbook definitions.
    from scipy.stats import chisquare

    rng = np.random.default_rng(5)
    V, k, p, tau = 48, 30, 0.9, 0.8
    x = rng.standard_normal(V).astype(np.float32) * 2
    z = x.astype(np.float64) / np.float32(tau)
    prob = np.exp(z - z.max())
    prob /= prob.sum()
    order = np.argsort(-prob, kind="stable")[:k]
    cum = np.cumsum(prob[order]) / prob[order].sum()
    n = int(np.searchsorted(cum, p) + 1)
    keep = order[:n]
    want = prob[keep] / prob[keep].sum()
    N = 100000
    logits = np.repeat(x[None, :], 1000, axis=0)
    counts = np.zeros(V)
    for rep in range(N // 1000):
        tok, _, _ = orc.sample_logits(logits, np.full(1000, k), np.full(1000, p),
                                      np.full(1000, tau), None, 17, rep)
        counts += np.bincount(tok, minlength=V)
    assert counts[np.setdiff1d(np.arange(V), keep)].sum() == 0
    stat, pval = chisquare(counts[keep], want * N)
    assert pval > 1e-4, (stat, pval)


def test_exp_weight_is_monotone_within_one_ulp(orc, tmp_path):
    # Every fp32 argument in [-104, -0] (about 1.1e9 values, scanned by a
    # compiled helper on all host threads): E never exceeds 1, and E(s) is
    # never more than one unit in the last place below the largest E(s') at
    # any s' <= s.  The sampling kernels rely on this bound: a logit row's
    # entries whose weight reaches a threshold w0 are all among the logits x
    # >= the smallest logit whose weight reaches w0 less one ulp.
    import os
    import subprocess

    src = os.path.join(os.path.dirname(__file__), "native", "exp_weight_scan.cpp")
    exe = str(tmp_path / "exp_weight_scan")
    subprocess.run(["g++", "-O2", "-std=c++17", "-pthread", "-o", exe, src, "-ldl"], check=True)
    nt = max(1, len(os.sched_getaffinity(0)))
    out = subprocess.run([exe, orc.path, str(nt)], capture_output=True, text=True,
                         check=True).stdout.split()
    assert out[0] == "drop_ulp" and int(out[1]) <= 1, out
    assert out[2] == "max" and float.fromhex(out[3]) == 1.0, out
    assert out[4] == "above_one" and out[5] == "0", out
