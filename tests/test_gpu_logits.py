"""GPU parity of logit rows: topk_topp_sample_logits (temperature, min-p)
through the C ABI against the CPU oracle's logit rows.

Bar: token ids bit-exact, kept sets (nonzero pattern of renorm_out)
bit-exact, renorm_out within 1e-6 relative, on the five workloads fed as
logits, on every forced internal path, and on edge rows (masked, NaN and
+inf logits, temperatures 0 / NaN / tiny / huge / +inf, min-p floors on and
between masses, ragged vocabularies).
"""

import numpy as np
import pytest

import top_exact_sampling_amd as tes
import workloads
from tests.gpu_util import REL_TOL, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    tes.lib()
    return torch


@pytest.fixture(scope="module")
def samplers(torch_cuda):
    out = {
        "plain": tes.Sampler(0, 4096, 1 << 18, 0),
        "stats": tes.Sampler(0, 4096, 1 << 18, tes.TES_FLAG_STATS),
        "row_select": tes.Sampler(0, 4096, 1 << 18, tes.TES_FLAG_FORCE_ROW_SELECT),
        "tiny_buffer": tes.Sampler(0, 4096, 1 << 18, tes.TES_FLAG_TINY_BUFFER),
        "small_segments": tes.Sampler(0, 4096, 1 << 18, tes.TES_FLAG_SMALL_SEGMENTS),
        "no_wait": tes.Sampler(0, 4096, 1 << 18, tes.TES_FLAG_NO_WAIT),
        "row_topp": tes.Sampler(0, 4096, 1 << 18, tes.TES_FLAG_ROW_TOPP),
    }
    yield out
    for s in out.values():
        s.close()


_WL = {}


def wl(cfg):
    if cfg not in _WL:
        _WL[cfg] = workloads.make_logits(cfg)
    return _WL[cfg]


def run_logits(torch, sampler, x, ks, ps, tau, mp, seed, off, renorm=True, aligned=True):
    B, V = x.shape
    if aligned:
        xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    else:
        flat = torch.zeros(B * V + 1, dtype=torch.float32, device="cuda")
        flat[1:] = torch.from_numpy(np.ascontiguousarray(x).reshape(-1)).cuda()
        xd = flat[1:].view(B, V)
    kd = torch.from_numpy(np.ascontiguousarray(ks, np.int32)).cuda()
    pd = torch.from_numpy(np.ascontiguousarray(ps, np.float32)).cuda()
    td = None if tau is None else torch.from_numpy(np.ascontiguousarray(tau, np.float32)).cuda()
    md = None if mp is None else torch.from_numpy(np.ascontiguousarray(mp, np.float32)).cuda()
    tok = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    ren = torch.full((B, V), -1.0, dtype=torch.float32, device="cuda") if renorm else None
    sampler.sample_logits(xd, kd, pd, seed, off, temperature=td, min_p=md, out_tokens=tok,
                          renorm_out=ren)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), (ren.cpu().numpy() if renorm else None)


def assert_logit_parity(orc, x, ks, ps, tau, mp, seed, off, gtok, gren, label):
    otok, oren, info = orc.sample_logits(x, ks, ps, tau, mp, seed, off,
                                         want_renorm=gren is not None, want_info=True)
    bad = np.flatnonzero(gtok != otok)
    assert bad.size == 0, "%s: %d token mismatches; rows %s gpu %s oracle %s kind %s" % (
        label, bad.size, bad[:8], gtok[bad[:8]], otok[bad[:8]], info[bad[:8], 9])
    if gren is not None:
        assert np.all(np.isfinite(gren)), label + ": non-finite renorm_out"
        nzg, nzo = gren != 0, oren != 0
        rows = np.flatnonzero((nzg != nzo).any(axis=1))
        assert rows.size == 0, "%s: kept-set mismatch on rows %s (gpu %s oracle %s)" % (
            label, rows[:8], nzg[rows[:8]].sum(1), nzo[rows[:8]].sum(1))
        if nzo.any():
            rel = np.abs(gren[nzo].astype(np.float64) - oren[nzo]) / oren[nzo]
            assert rel.max() <= REL_TOL, "%s: renorm rel err %.3g" % (label, rel.max())


@pytest.mark.parametrize("renorm", [True, False])
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_logit_config_parity(samplers, orc, torch_cuda, cfg, renorm):
    w = wl(cfg)
    for which in ("plain", "stats"):
        log("[gpu] logits config %d %s renorm=%s sampler=%s" % (cfg, w.name, renorm, which))
        gtok, gren = run_logits(torch_cuda, samplers[which], w.probs, w.top_k, w.top_p,
                                w.temperature, w.min_p, w.seed, w.offset, renorm=renorm)
        assert_logit_parity(orc, w.probs, w.top_k, w.top_p, w.temperature, w.min_p, w.seed,
                            w.offset, gtok, gren, "%s/%s" % (w.name, which))
        if which == "stats":
            st = samplers["stats"].stats(w.B)
            log("[gpu]   paths %s kinds %s" % (np.bincount(st[:, 0], minlength=6).tolist(),
                                              np.bincount(st[:, 1], minlength=3).tolist()))


@pytest.mark.parametrize("variant", ["row_select", "tiny_buffer", "small_segments", "no_wait",
                                     "row_topp"])
@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_logit_forced_paths(samplers, orc, torch_cuda, variant, cfg):
    w = wl(cfg)
    rng = np.random.default_rng(cfg + 50)
    rows = np.sort(rng.choice(w.B, min(w.B, 40), replace=False))
    if cfg == 4:
        cls = w.meta["row_class"]
        rows = np.unique(np.concatenate([rows, np.flatnonzero(cls != "plain")]))
    x = np.ascontiguousarray(w.probs[rows])
    args = (w.top_k[rows], w.top_p[rows], w.temperature[rows], w.min_p[rows], w.seed, 3)
    log("[gpu] logits variant %s config %d rows %d" % (variant, cfg, rows.size))
    gtok, gren = run_logits(torch_cuda, samplers[variant], x, *args)
    assert_logit_parity(orc, x, *args, gtok, gren, "%s/%s" % (variant, w.name))


def _edge_logit_batch(V, rng):
    rows, ks, ps, taus, mps = [], [], [], [], []

    def add(x, k, p, tau, mp):
        rows.append(np.asarray(x, np.float32))
        ks.append(k)
        ps.append(p)
        taus.append(tau)
        mps.append(mp)

    base = (2.0 * rng.standard_normal(V)).astype(np.float32)
    base[rng.choice(V, min(V, 4), replace=False)] += 9.0
    for k in (1, 2, 50, 1024, 2000, V):
        for tau in (1.0, 0.0, float("nan"), 1e-30, 40.0, float("inf"), 0.3):
            add(base, k, 0.9, tau, 0.0)
        for mp in (1e-9, 0.01, 0.3, 0.999, 1.0, 3.0, float("nan"), -1.0):
            add(base, k, 1.0, 0.8, mp)
    masked = np.full(V, -np.inf, np.float32)
    for k in (1, 7, V):
        add(masked, k, 0.9, 1.0, 0.1)
    nanrow = base.copy()
    nanrow[rng.choice(V, min(V, 7), replace=False)] = np.nan
    nanrow[int(np.argmax(base))] = np.nan
    for k in (1, 30, V):
        add(nanrow, k, 0.9, 0.7, 0.05)
    allnan = np.full(V, np.nan, np.float32)
    add(allnan, 5, 0.9, 1.0, 0.0)
    infrow = base.copy()
    infrow[rng.choice(V, min(V, 3), replace=False)] = np.inf
    for k in (1, 2, 100, V):
        add(infrow, k, 0.5, 1.0, 0.2)
    ties = (np.rint(base * 2) / 2).astype(np.float32)
    for k in (3, 64, 1024, V):
        for mp in (0.0, 0.1, 0.5):
            add(ties, k, 0.95, 1.0, mp)
    flat = np.zeros(V, np.float32)
    for k in (1, 20, V):
        add(flat, k, 0.5, 1.0, 0.0)
        add(flat, k, 1.0, 1.0, 0.5)
    neg = (-50.0 - rng.random(V)).astype(np.float32)  # all negative, far from 0
    for k in (10, V):
        add(neg, k, 0.9, 0.01, 0.0)
        add(neg, k, 0.9, 2.0, 0.02)
    return (np.stack(rows), np.array(ks, np.int32), np.array(ps, np.float32),
            np.array(taus, np.float32), np.array(mps, np.float32))


@pytest.mark.parametrize("V", [151936, 262144, 20000, 1021, 4])
def test_logit_edge_rows(samplers, orc, torch_cuda, V):
    rng = np.random.default_rng(V + 101)
    x, ks, ps, taus, mps = _edge_logit_batch(V, rng)
    for which in ("plain", "row_select", "tiny_buffer", "small_segments", "row_topp"):
        log("[gpu] logit edge rows V=%d rows=%d sampler=%s" % (V, len(ks), which))
        gtok, gren = run_logits(torch_cuda, samplers[which], x, ks, ps, taus, mps, 11, 5)
        assert_logit_parity(orc, x, ks, ps, taus, mps, 11, 5, gtok, gren,
                            "logit edges V=%d %s" % (V, which))


def test_logit_null_temperature_and_min_p(samplers, orc, torch_cuda):
    w = wl(2)
    log("[gpu] logits without temperature and min-p arrays")
    gtok, gren = run_logits(torch_cuda, samplers["plain"], w.probs, w.top_k, w.top_p, None, None,
                            w.seed, 9)
    assert_logit_parity(orc, w.probs, w.top_k, w.top_p, None, None, w.seed, 9, gtok, gren,
                        "logits, no temperature / min-p")


def test_logit_unaligned_rows(samplers, orc, torch_cuda):
    w = wl(2)
    rows = np.arange(12)
    x = np.ascontiguousarray(w.probs[rows])
    args = (w.top_k[rows], w.top_p[rows], w.temperature[rows], w.min_p[rows], 4, 4)
    log("[gpu] logits on unaligned rows (scalar path)")
    gtok, gren = run_logits(torch_cuda, samplers["plain"], x, *args, aligned=False)
    assert_logit_parity(orc, x, *args, gtok, gren, "logits unaligned")


def test_logit_min_p_binds_on_every_path(samplers, orc, torch_cuda):
    # Rows where the min-p prefix is shorter than the top-p prefix, on the
    # binned finish (k <= 1024), the sorted finish (tiny buffer), the
    # whole-row passes (k = V, and 1024 < k < V) and split rows (small B).
    rng = np.random.default_rng(77)
    V = 151936
    B = 24
    x = (1.5 * rng.standard_normal((B, V))).astype(np.float32)
    for b in range(B):
        x[b, rng.choice(V, 40, replace=False)] += rng.uniform(3, 6, 40).astype(np.float32)
    ks = np.array(([1000, 300, V, 5000] * 6)[:B], np.int32)
    ps = np.full(B, 1.0, np.float32)
    taus = rng.uniform(0.7, 1.3, B).astype(np.float32)
    mps = rng.uniform(0.02, 0.4, B).astype(np.float32)
    for which in ("plain", "tiny_buffer", "stats", "row_topp"):
        log("[gpu] min-p binding rows sampler=%s" % which)
        gtok, gren = run_logits(torch_cuda, samplers[which], x, ks, ps, taus, mps, 21, 0)
        assert_logit_parity(orc, x, ks, ps, taus, mps, 21, 0, gtok, gren,
                            "min-p binds %s" % which)
        # the floor did cut: fewer kept than with top-p alone
        _, oren, _ = orc.sample_logits(x, ks, ps, taus, None, 21, 0, want_renorm=True)
        assert np.all((gren != 0).sum(1) <= (oren != 0).sum(1))
        assert np.any((gren != 0).sum(1) < (oren != 0).sum(1))
