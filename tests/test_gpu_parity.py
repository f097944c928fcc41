"""GPU parity: the HIP sampler (through the C ABI) against the CPU oracle.

Bar: token ids bit-exact, kept sets (nonzero pattern of renorm_out)
bit-exact, renorm_out within 1e-6 relative.  Every internal path (candidate
buffer, top-p-only hit, whole-row select, forced variants) must agree.
"""

import numpy as np
import pytest

import top_exact_sampling_amd as tes
import workloads
from tests import golden_cases
from tests.gpu_util import assert_parity, log, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    tes.lib()  # fail loudly when the HIP library is missing
    return torch


@pytest.fixture(scope="module")
def sampler(torch_cuda):
    s = tes.Sampler(0, max_batch=4096, max_vocab=1 << 18, flags=tes.TES_FLAG_STATS)
    yield s
    s.close()


@pytest.fixture(scope="module")
def plain_sampler(torch_cuda):
    # The shipping configuration: no flags (no statistics, no forced paths).
    s = tes.Sampler(0, max_batch=4096, max_vocab=1 << 18, flags=0)
    yield s
    s.close()


@pytest.fixture(scope="module")
def variant_samplers(torch_cuda):
    out = {
        "row_select": tes.Sampler(0, 4096, 1 << 18, tes.TES_FLAG_FORCE_ROW_SELECT),
        "tiny_buffer": tes.Sampler(0, 4096, 1 << 18, tes.TES_FLAG_TINY_BUFFER),
        "row_select_tiny": tes.Sampler(
            0, 4096, 1 << 18, tes.TES_FLAG_FORCE_ROW_SELECT | tes.TES_FLAG_TINY_BUFFER),
        "small_segments": tes.Sampler(0, 4096, 1 << 18, tes.TES_FLAG_SMALL_SEGMENTS),
        "small_tiny": tes.Sampler(
            0, 4096, 1 << 18, tes.TES_FLAG_SMALL_SEGMENTS | tes.TES_FLAG_TINY_BUFFER),
        "row_topp": tes.Sampler(0, 4096, 1 << 18, tes.TES_FLAG_ROW_TOPP | tes.TES_FLAG_STATS),
        "row_topp_tiny": tes.Sampler(
            0, 4096, 1 << 18, tes.TES_FLAG_ROW_TOPP | tes.TES_FLAG_TINY_BUFFER),
    }
    yield out
    for s in out.values():
        s.close()


_WL = {}


def wl(cfg):
    if cfg not in _WL:
        _WL[cfg] = workloads.make(cfg)
    return _WL[cfg]


@pytest.mark.parametrize("which", ["stats", "plain"])
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_config_parity_with_renorm(sampler, plain_sampler, orc, cfg, which):
    w = wl(cfg)
    s = sampler if which == "stats" else plain_sampler
    log("[gpu] config %d %s B=%d V=%d renorm (%s sampler)" % (cfg, w.name, w.B, w.V, which))
    gtok, gren = run_gpu(s, w.probs, w.top_k, w.top_p, w.seed, w.offset, renorm=True)
    assert_parity(orc, w.probs, w.top_k, w.top_p, w.seed, w.offset, gtok, gren, w.name)
    if which == "stats":
        st = sampler.stats(w.B)
        log("[gpu]   paths %s, kinds %s, gathered max %d" % (
            np.bincount(st[:, 0], minlength=5).tolist(),
            np.bincount(st[:, 1], minlength=3).tolist(), st[:, 4].max()))
        # Top-k and greedy rows record their kept entries (stats word 10), and
        # renorm_out's row is written from that list without a second read:
        # the list holds exactly the row's nonzero renorm entries.
        listed = np.isin(st[:, 0], [0, 4, 5])
        nz = np.count_nonzero(np.asarray(gren).reshape(w.B, w.V), axis=1)
        bad = np.flatnonzero(listed & (st[:, 10] != nz))
        assert bad.size == 0, "kept lists differ from renorm_out: rows %s" % bad[:8]
        log("[gpu]   %d rows written from kept lists" % int(listed.sum()))


@pytest.mark.parametrize("which", ["stats", "plain"])
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_config_parity_tokens_only(sampler, plain_sampler, orc, cfg, which):
    # The launch the benchmark times: renorm_out = NULL, on the sampler the
    # benchmark uses (no flags) and on the statistics sampler.
    w = wl(cfg)
    s = sampler if which == "stats" else plain_sampler
    log("[gpu] config %d %s tokens only (%s sampler)" % (cfg, w.name, which))
    gtok, _ = run_gpu(s, w.probs, w.top_k, w.top_p, w.seed, w.offset, renorm=False)
    assert_parity(orc, w.probs, w.top_k, w.top_p, w.seed, w.offset, gtok, None, w.name)
    # A second offset on the shipping sampler: draw-dependent paths differ.
    if which == "plain":
        gtok, _ = run_gpu(s, w.probs, w.top_k, w.top_p, w.seed, w.offset + 17, renorm=False)
        assert_parity(orc, w.probs, w.top_k, w.top_p, w.seed, w.offset + 17, gtok, None,
                      w.name + " offset+17")


@pytest.mark.parametrize("variant", ["row_select", "tiny_buffer", "row_select_tiny",
                                     "small_segments", "small_tiny", "row_topp",
                                     "row_topp_tiny"])
@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_forced_paths_agree(variant_samplers, orc, variant, cfg):
    w = wl(cfg)
    rows = np.arange(w.B)
    if cfg in (3, 4):
        rng = np.random.default_rng(cfg)
        rows = np.sort(rng.choice(w.B, 48, replace=False))
        if cfg == 4:
            cls = w.meta["row_class"]
            rows = np.unique(np.concatenate([rows, np.flatnonzero(cls != "plain")]))
    probs = np.ascontiguousarray(w.probs[rows])
    log("[gpu] variant %s config %d rows %d" % (variant, cfg, rows.size))
    gtok, gren = run_gpu(variant_samplers[variant], probs, w.top_k[rows], w.top_p[rows], w.seed,
                         w.offset, renorm=True)
    assert_parity(orc, probs, w.top_k[rows], w.top_p[rows], w.seed, w.offset, gtok, gren,
                  "%s/%s" % (variant, w.name))


def test_golden_worked_examples(sampler, orc):
    # The worked examples fix u directly while the GPU derives u from Philox,
    # so each example runs with several (seed, offset) and is compared with
    # the oracle's row function at that u, plus the fixed renorm values.
    for name, row, k, p, draws, ren_want in golden_cases.load():
        probs = row[None, :]
        for seed, off in ((0, 0), (1, 5), (77, 2**40)):
            u = orc.uniform_u64(seed, 0, off)
            gtok, gren = run_gpu(sampler, probs, [k], [p], seed, off, renorm=True)
            otok, _, _ = orc.sample_row(row, k, p, u)
            assert gtok[0] == otok, name
            np.testing.assert_allclose(gren[0], np.array(ren_want, np.float32), rtol=1e-6,
                                       atol=0, err_msg=name)


def _adversarial_batch(V, rng):
    rows, ks, ps, names = [], [], [], []

    def add(x, k, p, name):
        rows.append(np.asarray(x, np.float32))
        ks.append(k)
        ps.append(p)
        names.append(name)

    flat = np.full(V, 1.0 / V, np.float32)
    for k in (1, 50, 1024, 2000, V):
        for p in (0.5, 1.0):
            add(flat, k, p, "flat k%d p%g" % (k, p))
    asc = np.linspace(1.0, 2.0, V).astype(np.float64)
    asc = (asc / asc.sum()).astype(np.float32)
    for k in (1, 37, 1024, V):
        add(asc, k, 0.9, "ascending k%d" % k)
        add(asc[::-1], k, 0.9, "descending k%d" % k)
    few = np.zeros(V, np.float32)
    nf = min(V, 10)
    few[rng.choice(V, nf, replace=False)] = rng.random(nf).astype(np.float32)
    add(few, 100, 0.95, "k above positives")
    add(few, V, 1.0, "few positives full")
    den = np.full(V, np.float32(1e-40), np.float32)
    add(den, 20, 0.9, "all denormal")
    add(den, V, 0.9, "all denormal full")
    add(np.full(V, np.inf, np.float32), 50, 0.9, "all inf k50")
    add(np.full(V, np.inf, np.float32), V, 0.9, "all inf full")
    many_inf = rng.random(V).astype(np.float32)
    many_inf[rng.choice(V, min(V, 1500), replace=False)] = np.inf
    add(many_inf, V, 0.9, "1500 inf full")
    add(many_inf, 1024, 0.9, "1500 inf k1024")
    near = (1.0 + 1e-6 * rng.random(V)).astype(np.float64)
    add((near / near.sum()).astype(np.float32), V, 0.95, "near uniform full")
    fat = (rng.random(V) * 1e-6).astype(np.float32)
    fat[rng.choice(V, min(V, 3000), replace=False)] = np.float32(1e-4)
    fat[rng.choice(V, min(V, 200), replace=False)] = np.float32(1e-3)
    for k in (150, 1024, V):
        add(fat, k, 0.97, "fat bucket k%d" % k)
    for p in (1e-9, 0.0, float("nan"), 1.0, 5.0):
        add(asc, V, p, "p=%r" % p)
        add(asc, 64, p, "p=%r k64" % p)
    neg = rng.standard_normal(V).astype(np.float32)
    add(neg, 100, 0.9, "gaussian with negatives")
    add(neg, V, 0.9, "gaussian with negatives full")
    return np.stack(rows), np.array(ks, np.int32), np.array(ps, np.float32), names


@pytest.mark.parametrize("V", [151936, 262144, 5000, 1021, 4])
def test_adversarial_rows(sampler, variant_samplers, orc, V):
    rng = np.random.default_rng(V)
    probs, ks, ps, names = _adversarial_batch(V, rng)
    for label, s in (("default", sampler), ("row_select", variant_samplers["row_select"]),
                     ("tiny_buffer", variant_samplers["tiny_buffer"]),
                     ("small_segments", variant_samplers["small_segments"]),
                     ("small_tiny", variant_samplers["small_tiny"]),
                     ("row_topp", variant_samplers["row_topp"]),
                     ("row_topp_tiny", variant_samplers["row_topp_tiny"])):
        log("[gpu] adversarial V=%d rows=%d sampler=%s" % (V, len(names), label))
        gtok, gren = run_gpu(s, probs, ks, ps, 9, 3, renorm=True)
        assert_parity(orc, probs, ks, ps, 9, 3, gtok, gren, "adversarial V=%d %s" % (V, label))


def _above_one_batch(V, rng):
    """Rows with entries of exactly 1.0, finite entries above it, and NaN /
    negatives beside them; each as a top-p-only row, a k=1000 row and a
    greedy row."""
    rows, ks, ps = [], [], []

    def add(x, p):
        for k in (V, 1000, 1):
            rows.append(np.asarray(x, np.float32))
            ks.append(k)
            ps.append(p)

    base = (rng.random(V) * 1e-4).astype(np.float32)
    one_hot = np.zeros(V, np.float32)
    one_hot[rng.integers(V)] = 1.0
    add(one_hot, 0.9)
    x = base.copy()
    x[rng.choice(V, 2, replace=False)] = 1.0
    add(x, 0.5)
    x = base.copy()
    x[rng.choice(V, 3, replace=False)] = [1.5, 3e38, 1.0]
    add(x, 0.95)
    x = base.copy()
    i = rng.choice(V, 40, replace=False)
    x[i[:20]] = rng.uniform(1.0, 4.0, 20).astype(np.float32)
    x[i[20:30]] = np.nan
    x[i[30:]] = -rng.random(10).astype(np.float32)
    add(x, 1.0)
    x = np.full(V, np.float32(1e-40), np.float32)
    x[rng.integers(V)] = 1.0
    add(x, 0.9)
    return np.stack(rows), np.array(ks, np.int32), np.array(ps, np.float32)


def test_row_path_over_many_draws(sampler, orc, torch_cuda):
    # The one-workgroup top-p path predicts the boundary's and the draw's
    # bins from a prefix of the row; a row whose bins fall outside the
    # predicted window takes another (exact) pass.  Over twelve draws of the
    # speculative-verify batch some rows do: tokens must match the oracle
    # on every draw, and the extra-pass rows must occur.
    w = wl(5)
    x = torch_cuda.from_numpy(w.probs).cuda()
    k = torch_cuda.from_numpy(w.top_k).cuda()
    p = torch_cuda.from_numpy(w.top_p).cuda()
    extra = 0
    for off in range(12):
        log("[gpu] row path draw %d" % off)
        g = sampler.sample(x, k, p, w.seed, off)
        torch_cuda.cuda.synchronize()
        otok = orc.sample(w.probs, w.top_k, w.top_p, w.seed, off)[0]
        bad = np.flatnonzero(g.cpu().numpy() != otok)
        assert bad.size == 0, "draw %d: rows %s differ" % (off, bad[:8])
        st = sampler.stats(w.B)
        assert np.all(st[:, 0] == 6), "paths %s" % np.bincount(st[:, 0]).tolist()
        extra += int(((st[:, 3] > 1) | ((st[:, 7] >> 16) != 0)).sum())
    log("[gpu]   rows with an extra pass over 12 draws: %d" % extra)
    assert extra > 0, "no row took the extra pass: the test no longer reaches it"


@pytest.mark.parametrize("V", [151936, 20000])
def test_entries_at_and_above_one(sampler, variant_samplers, orc, V):
    # The mass histograms take floor(x * 2^32) from a saturating conversion:
    # every entry from 1.0 up weighs 2^32 - 1 in the top bin, whose count
    # (its sum over 2^32 - 1) becomes count * 2^32, and NaN or negative bits
    # weigh nothing.  The rows of _above_one_batch on the segment path, the
    # one-workgroup path and the top-k paths.
    probs, ks, ps = _above_one_batch(V, np.random.default_rng(V + 1))
    for label, s in (("default", sampler), ("small_segments", variant_samplers["small_segments"]),
                     ("row_topp", variant_samplers["row_topp"])):
        log("[gpu] entries at and above 1.0, V=%d sampler=%s" % (V, label))
        gtok, gren = run_gpu(s, probs, ks, ps, 21, 5, renorm=True)
        assert_parity(orc, probs, ks, ps, 21, 5, gtok, gren, "above one V=%d %s" % (V, label))


@pytest.mark.parametrize("V", [1, 2, 3, 7, 999, 1000, 1024, 1025, 4097, 8191, 8192, 8193, 40000])
def test_ragged_vocab_sizes(sampler, variant_samplers, orc, V):
    rng = np.random.default_rng(V + 17)
    B = 24
    x = 2.0 * rng.standard_normal((B, V))
    x[:, : min(V, 3)] += 9.0
    e = np.exp(x - x.max(1, keepdims=True))
    probs = (e / e.sum(1, keepdims=True)).astype(np.float32)
    ks = rng.integers(-2, V + 3, size=B).astype(np.int32)
    ks[:4] = [1, V, 0, 1024]
    ps = rng.uniform(0.3, 1.0, size=B).astype(np.float32)
    for label in ("default", "row_topp"):
        s = sampler if label == "default" else variant_samplers[label]
        log("[gpu] ragged V=%d sampler=%s" % (V, label))
        gtok, gren = run_gpu(s, probs, ks, ps, 3, 11, renorm=True)
        assert_parity(orc, probs, ks, ps, 3, 11, gtok, gren, "ragged V=%d %s" % (V, label))


def test_unaligned_rows_use_scalar_path(sampler, orc, torch_cuda):
    torch = torch_cuda
    w = wl(2)
    B, V = 16, w.V
    flat = torch.zeros(B * V + 1, dtype=torch.float32, device="cuda")
    flat[1:] = torch.from_numpy(w.probs[:B].reshape(-1)).cuda()
    probs_dev = flat[1:].view(B, V)  # 4-byte aligned, not 16-byte aligned
    assert probs_dev.data_ptr() % 16 != 0
    log("[gpu] unaligned rows")
    gtok, gren = run_gpu(sampler, w.probs[:B], w.top_k[:B], w.top_p[:B], 5, 6, renorm=True,
                         probs_dev=probs_dev)
    assert_parity(orc, w.probs[:B], w.top_k[:B], w.top_p[:B], 5, 6, gtok, gren, "unaligned")


def test_seeds_and_offsets(sampler, orc):
    w = wl(2)
    for seed, off in ((0, 1), (2**64 - 1, 2**64 - 1), (123456789, 2**33 + 5)):
        log("[gpu] seed %d offset %d" % (seed, off))
        gtok, _ = run_gpu(sampler, w.probs, w.top_k, w.top_p, seed, off, renorm=False)
        assert_parity(orc, w.probs, w.top_k, w.top_p, seed, off, gtok, None, "seed/offset")


def test_determinism_streams_and_graph_replay(plain_sampler, torch_cuda):
    # The sampler without statistics: a captured call records kernel nodes only.
    sampler = plain_sampler
    torch = torch_cuda
    w = wl(3)
    pd = torch.from_numpy(w.probs).cuda()
    kd = torch.from_numpy(w.top_k).cuda()
    qd = torch.from_numpy(w.top_p).cuda()
    ref = sampler.sample(pd, kd, qd, w.seed, w.offset).clone()
    torch.cuda.synchronize()
    log("[gpu] determinism: side stream")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        again = sampler.sample(pd, kd, qd, w.seed, w.offset)
    torch.cuda.synchronize()
    assert torch.equal(again, ref)
    log("[gpu] determinism: graph capture and replay")
    out = torch.empty_like(ref)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        sampler.sample(pd, kd, qd, w.seed, w.offset, out_tokens=out)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        sampler.sample(pd, kd, qd, w.seed, w.offset, out_tokens=out)
    for i in range(4):
        out.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "replay %d differs" % i
        _ = (pd[:2].sum() + 1).item()  # eager work between replays


def test_zero_batch_and_argument_errors(sampler, torch_cuda):
    torch = torch_cuda
    h = sampler.handle
    assert tes.topk_topp_sample(h, 0, 0, 10, 0, 0, 0, 0, 0, None, None) == tes.TES_OK
    p = torch.zeros(4, 8, device="cuda")
    k = torch.zeros(4, dtype=torch.int32, device="cuda")
    q = torch.zeros(4, device="cuda")
    t = torch.zeros(4, dtype=torch.int32, device="cuda")
    args = (p.data_ptr(), 4, 8, k.data_ptr(), q.data_ptr(), 0, 0, t.data_ptr(), None, None)
    assert tes.topk_topp_sample(None, *args) == tes.TES_ERR_INVALID_ARGUMENT
    bad = list(args)
    bad[0] = p.data_ptr() + 2
    assert tes.topk_topp_sample(h, *bad) == tes.TES_ERR_INVALID_ARGUMENT
    bad = list(args)
    bad[1] = 10**6
    assert tes.topk_topp_sample(h, *bad) == tes.TES_ERR_TOO_LARGE
    assert tes.topk_topp_sample(h, *args) == tes.TES_OK
    torch.cuda.synchronize()


def _split_batch(V, rng):
    """Rows whose decisive entries straddle the point where a row split
    between two workgroups is cut (half the row's 16-byte vectors)."""
    cut = ((V // 4 + 1) // 2) * 4
    rows, ks, ps, names = [], [], [], []

    def add(x, k, p, name):
        rows.append(np.asarray(x, np.float32))
        ks.append(k)
        ps.append(p)
        names.append(name)

    base = (rng.random(V) * 1e-7).astype(np.float32)
    tie = base.copy()
    tie[cut - 300: cut] = np.float32(1e-3)
    tie[cut: cut + 300] = np.float32(1e-3)
    tie[V - 200:] = np.float32(1e-3)
    for k in (1, 2, 299, 300, 301, 600, 700, 1024):
        add(tie, k, 1.0, "ties across the cut k%d" % k)
        add(tie, k, 0.3, "ties across the cut k%d p0.3" % k)
    two = base.copy()
    two[cut - 1] = np.float32(0.25)
    two[cut] = np.float32(0.25)
    add(two, 1, 1.0, "greedy tie at the cut")
    add(two, 2, 0.9, "k2 tie at the cut")
    second = base.copy()
    second[cut + 5: cut + 905] = (0.5 + rng.random(900)).astype(np.float32) * 1e-3
    for k in (1, 10, 512, 1024):
        add(second, k, 0.8, "mass in the second half k%d" % k)
    first = second[::-1].copy()
    for k in (1, 10, 512, 1024):
        add(first, k, 0.8, "mass in the first half k%d" % k)
    inf2 = base.copy()
    inf2[[3, cut + 7, V - 1]] = np.inf
    for k in (1, 2, 3, 50):
        add(inf2, k, 0.5, "inf in both halves k%d" % k)
    nan2 = base.copy()
    nan2[cut + 11] = np.nan
    nan2[cut - 11] = np.float32(0.1)
    add(nan2, 1, 1.0, "greedy with NaN in the second half")
    add(nan2, 64, 0.9, "k64 with NaN in the second half")
    zero = np.zeros(V, np.float32)
    zero[cut + 1] = -1.0
    add(zero, 1, 1.0, "greedy on a zero row")
    add(zero, 8, 1.0, "k8 on a zero row")
    return np.stack(rows), np.array(ks, np.int32), np.array(ps, np.float32), names


@pytest.mark.parametrize("V", [151936, 65540])
def test_split_rows(sampler, orc, V):
    # A small batch leaves room for every top-k and greedy row to be split
    # between several workgroups; the stats word [2] says how many ran the row.
    rng = np.random.default_rng(V + 5)
    probs, ks, ps, names = _split_batch(V, rng)
    log("[gpu] split rows V=%d rows=%d" % (V, len(names)))
    gtok, gren = run_gpu(sampler, probs, ks, ps, 21, 4, renorm=True)
    st = sampler.stats(len(names))
    log("[gpu]   parts per row %s" % np.unique(st[:, 2]).tolist())
    assert np.all(st[:, 2] >= 2), "rows not split: %s" % [
        names[i] for i in np.flatnonzero(st[:, 2] < 2)]
    assert_parity(orc, probs, ks, ps, 21, 4, gtok, gren, "split rows V=%d" % V)


@pytest.mark.parametrize("B,V", [(64, 32000), (16, 4096), (30, 151936), (200, 20000), (3, 1025)])
def test_split_part_counts(sampler, orc, B, V):
    # Batches whose rows are cut into 2..8 parts (as many as the resident
    # slots and a part size of at least one vector per thread allow).
    rng = np.random.default_rng(B * 7 + V)
    x = 2.0 * rng.standard_normal((B, V))
    for b in range(B):
        x[b, rng.choice(V, rng.integers(1, 9), replace=False)] += rng.uniform(8, 15)
    e = np.exp(x - x.max(1, keepdims=True))
    probs = (e / e.sum(1, keepdims=True)).astype(np.float32)
    ks = rng.integers(1, min(V, 1024) + 1, size=B).astype(np.int32)
    ks[: min(B, 3)] = 1
    ps = rng.uniform(0.5, 1.0, size=B).astype(np.float32)
    log("[gpu] split part counts B=%d V=%d" % (B, V))
    gtok, gren = run_gpu(sampler, probs, ks, ps, 8, 1, renorm=True)
    st = sampler.stats(B)
    log("[gpu]   parts per row %s, paths %s" % (np.unique(st[:, 2]).tolist(),
                                                 np.bincount(st[:, 0], minlength=6).tolist()))
    assert_parity(orc, probs, ks, ps, 8, 1, gtok, gren, "split parts B=%d V=%d" % (B, V))


def _restream_batch(V, rng):
    """Top-k rows whose sampled threshold cannot decide them: too few sampled
    entries with a mass, or a run of equal values at the threshold longer than
    the candidate buffer."""
    rows, ks, ps, names = [], [], [], []

    def add(x, k, p, name):
        rows.append(np.asarray(x, np.float32))
        ks.append(k)
        ps.append(p)
        names.append(name)

    n_pos = min(V // 2, 4500)
    tail = np.zeros(V, np.float32)
    tail[V - n_pos:] = (rng.random(n_pos) + 0.5).astype(np.float32) / n_pos
    for k in (2, 700, 1024):
        add(tail, k, 0.9, "positives only in the tail k%d" % k)
    few_tail = np.zeros(V, np.float32)
    few_tail[V - 300:] = np.float32(1.0 / 300)
    few_tail[V - 300: V - 150] = np.float32(0.5 / 300)
    for k in (299, 300, 301, 500, 1024):
        add(few_tail, k, 0.95, "300 tail positives k%d" % k)
    inf_tail = few_tail.copy()
    inf_tail[[V - 7, V - 3]] = np.inf
    add(inf_tail, 500, 0.9, "two inf among tail positives k500")
    tiny_tail = np.zeros(V, np.float32)
    tiny_tail[V - 50:] = np.float32(1e-12)  # positive keys without a mass
    tiny_tail[[5, 9]] = -1.0
    for k in (20, 50, 51, 200):
        add(tiny_tail, k, 0.9, "massless tail k%d" % k)
    for k in (2, 500, 1024):
        add(np.zeros(V, np.float32), k, 0.9, "zero row k%d" % k)
    negz = np.zeros(V, np.float32)
    negz[: min(V, 1000)] = -0.0
    negz[min(V, 1000): min(V, 1003)] = np.nan
    add(negz, 64, 0.9, "-0.0 and NaN prefix k64")
    tie = np.full(V, np.float32(1e-9), np.float32)
    nt = min(V // 2, 6000)
    tie[rng.choice(V, nt, replace=False)] = np.float32(1e-4)
    tie[rng.choice(V, 40, replace=False)] = np.float32(2e-3)
    for k in (41, 500, 1024):
        for p in (0.5, 1.0):
            add(tie, k, p, "6000-long tie at the threshold k%d p%g" % (k, p))
    q = np.floor(rng.random(V) ** 8 * 64) / 2**20  # few distinct values, many zeros
    q = (q / q.sum()).astype(np.float32)
    for k in (1, 10, 700, 1024):
        add(q, k, 0.8, "quantised k%d" % k)
    return np.stack(rows), np.array(ks, np.int32), np.array(ps, np.float32), names


@pytest.mark.parametrize("V", [151936, 128256, 20000])
def test_restream_rows(sampler, orc, V):
    rng = np.random.default_rng(V + 29)
    probs, ks, ps, names = _restream_batch(V, rng)
    log("[gpu] restream rows V=%d rows=%d" % (V, len(names)))
    gtok, gren = run_gpu(sampler, probs, ks, ps, 13, 2, renorm=True)
    st = sampler.stats(len(names))
    log("[gpu]   paths %s" % np.bincount(st[:, 0], minlength=6).tolist())
    assert_parity(orc, probs, ks, ps, 13, 2, gtok, gren, "restream rows V=%d" % V)
    assert (st[:, 0] == 5).sum() >= 8, "the compacting pass did not run"


@pytest.mark.parametrize("B", [20, 200])
def test_rows_with_fewer_positive_keys_than_k(sampler, orc, B):
    # A top-k row with fewer positive keys than k (mostly zeros, as a logit
    # row at temperature 0 has) is decided by its first stream, split (B=20:
    # eight parts per row) or not (B=200), without the compacting pass.
    rng = np.random.default_rng(B + 71)
    V = 20000
    probs = np.zeros((B, V), np.float32)
    ks = np.empty(B, np.int32)
    short = np.zeros(B, bool)
    for b in range(B):
        m = int(rng.integers(0, 900))
        idx = rng.choice(V, m, replace=False)
        kind = b % 5
        if kind == 0:
            probs[b, idx] = rng.random(m).astype(np.float32) + 0.01
        elif kind == 1:
            probs[b, idx] = np.float32(1.0 / max(m, 1))  # ties
        elif kind == 2:
            probs[b, idx] = np.float32(1e-12)  # positive keys without a mass
        elif kind == 3:
            probs[b, idx] = rng.random(m).astype(np.float32)
            probs[b, idx[:2]] = np.inf
        else:
            probs[b, idx] = rng.random(m).astype(np.float32)
            probs[b, rng.choice(V, 3)] = -1.0
        ks[b] = int(rng.integers(m + 1, 1025)) if m < 1024 else 1024
        short[b] = m < ks[b] and ks[b] >= 2
    ps = rng.uniform(0.3, 1.0, B).astype(np.float32)
    log("[gpu] rows with fewer positive keys than k, B=%d" % B)
    gtok, gren = run_gpu(sampler, probs, ks, ps, 17, 5, renorm=True)
    st = sampler.stats(B)
    log("[gpu]   paths %s" % np.bincount(st[:, 0], minlength=6).tolist())
    assert_parity(orc, probs, ks, ps, 17, 5, gtok, gren, "fewer positives B=%d" % B)
    assert np.all(st[short, 0] == 0), "rows took paths %s" % np.unique(st[short, 0])


def test_wide_topp_bins_stay_on_the_fast_path(sampler, orc):
    # High-entropy rows at the speculative-verify shape gather more boundary
    # and draw entries than one buffer holds; the finish takes them one fine
    # bin at a time instead of re-reading the row.
    w = wl(5)
    rows = np.arange(0, w.B, 8)
    probs = np.ascontiguousarray(w.probs[rows])
    log("[gpu] wide top-p bins rows=%d" % rows.size)
    gtok, gren = run_gpu(sampler, probs, w.top_k[rows], w.top_p[rows], w.seed, w.offset,
                         renorm=True)
    st = sampler.stats(rows.size)
    log("[gpu]   paths %s gathered max %d" % (np.bincount(st[:, 0], minlength=6).tolist(),
                                             st[:, 4].max()))
    assert_parity(orc, probs, w.top_k[rows], w.top_p[rows], w.seed, w.offset, gtok, gren,
                  "wide top-p bins")
    assert np.all(st[:, 0] == 1), "rows left the fast path: %s" % np.flatnonzero(st[:, 0] != 1)


def test_oversubscribed_topp_rows_take_the_row_path(sampler, variant_samplers, orc):
    # The speculative-verify shape holds more top-p-only segments than the
    # device keeps resident workgroups: its top-p-only rows are decided by
    # one workgroup each (path 6) without exchanges, and agree with the
    # oracle at two offsets; the same rows through the forced flag agree
    # with the segmented path's tokens.
    w = wl(5)
    topp = np.flatnonzero((w.top_k <= 0) | (w.top_k >= w.V))
    for off in (w.offset, w.offset + 5):
        log("[gpu] oversubscribed top-p rows offset %d" % off)
        gtok, gren = run_gpu(sampler, w.probs, w.top_k, w.top_p, w.seed, off, renorm=True)
        st = sampler.stats(w.B)
        log("[gpu]   paths %s gathered max %d passes max %d" % (
            np.bincount(st[:, 0], minlength=7).tolist(), st[topp, 4].max(), st[topp, 3].max()))
        assert_parity(orc, w.probs, w.top_k, w.top_p, w.seed, off, gtok, gren,
                      "oversubscribed offset %d" % off)
        assert np.all(st[topp, 2] == 1), "top-p-only rows were segmented"
        assert np.mean(st[topp, 0] == 6) >= 0.95, np.bincount(st[topp, 0], minlength=7)
    rows = topp[:48]
    probs = np.ascontiguousarray(w.probs[rows])
    log("[gpu] forced row path on %d top-p-only rows" % rows.size)
    gtok, gren = run_gpu(variant_samplers["row_topp"], probs, w.top_k[rows], w.top_p[rows],
                         w.seed, w.offset, renorm=True)
    st = variant_samplers["row_topp"].stats(rows.size)
    assert_parity(orc, probs, w.top_k[rows], w.top_p[rows], w.seed, w.offset, gtok, gren,
                  "forced row path")
    assert np.all(st[:, 2] == 1) and np.mean(st[:, 0] == 6) >= 0.95, st[:, 0]


def test_row_path_tie_runs(sampler, variant_samplers, orc):
    # Quantised rows (multiples of 2^-20, as in the ties-and-edges recipe)
    # as top-p-only rows on the one-workgroup path: every fine bin holds one
    # value, and the boundary's and the draw's bins hold thousands of equal
    # entries, more than a select buffer takes, so they are selected by rank
    # in index order.
    w = wl(4)
    cls = w.meta["row_class"]
    rows = np.flatnonzero(cls == "plain")[:24]
    probs = np.ascontiguousarray(w.probs[rows])
    ks = np.full(rows.size, w.V, np.int32)
    ps = np.random.default_rng(44).uniform(0.3, 0.99, rows.size).astype(np.float32)
    for off in (0, 1):
        for label in ("default", "row_topp"):
            s = sampler if label == "default" else variant_samplers[label]
            log("[gpu] tie runs on top-p-only rows offset %d sampler=%s" % (off, label))
            gtok, gren = run_gpu(s, probs, ks, ps, 5, off, renorm=True)
            assert_parity(orc, probs, ks, ps, 5, off, gtok, gren, "tie runs %s %d" % (label, off))


def test_batches_longer_than_one_launch(sampler, orc):
    # More rows than one launch takes (1024): the call enqueues several
    # launches, each with its own row offset for the Philox counter, mixing
    # every row class.
    B, V = 2500, 4096
    rng = np.random.default_rng(2500)
    x = 2.0 * rng.standard_normal((B, V))
    x[np.arange(B), rng.integers(0, V, size=B)] += 10.0
    e = np.exp(x - x.max(1, keepdims=True))
    probs = (e / e.sum(1, keepdims=True)).astype(np.float32)
    ks = rng.choice(np.array([1, 7, 300, 1024, 2000, 0, V], np.int32), size=B)
    ps = rng.uniform(0.3, 1.0, size=B).astype(np.float32)
    log("[gpu] multi-launch batch B=%d V=%d" % (B, V))
    gtok, gren = run_gpu(sampler, probs, ks, ps, 99, 7, renorm=True)
    assert_parity(orc, probs, ks, ps, 99, 7, gtok, gren, "multi-launch")


@pytest.mark.parametrize("trial", range(6))
def test_random_shapes(sampler, variant_samplers, orc, trial):
    # Random batch and vocabulary sizes, row recipes and parameters, including
    # out-of-range k and p.
    rng = np.random.default_rng(1000 + trial)
    B = int(rng.integers(1, 80))
    V = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(300, 20000)),
                        int(rng.integers(20000, 140000))]))
    scale = float(rng.choice([0.3, 2.0, 6.0]))
    x = scale * rng.standard_normal((B, V))
    e = np.exp(x - x.max(1, keepdims=True))
    probs = (e / e.sum(1, keepdims=True)).astype(np.float32)
    if rng.random() < 0.5:  # coarse values: many ties
        probs = (np.round(probs * 2**12) / 2**12).astype(np.float32)
    ks = rng.integers(-3, V + 5, size=B).astype(np.int32)
    ks[rng.random(B) < 0.3] = 1
    ps = rng.uniform(-0.2, 1.3, size=B).astype(np.float32)
    seed, off = (int(v) for v in rng.integers(0, 2**63, size=2))
    for label in ("default", "row_topp"):
        s = sampler if label == "default" else variant_samplers[label]
        log("[gpu] random shapes trial %d B=%d V=%d sampler=%s" % (trial, B, V, label))
        gtok, gren = run_gpu(s, probs, ks, ps, seed, off, renorm=True)
        assert_parity(orc, probs, ks, ps, seed, off, gtok, gren,
                      "random trial %d %s" % (trial, label))


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_slab_export(sampler, orc, cfg):
    # The sorted support of every row with k_eff <= 1024 (its order is the
    # cake_sampling slab order), the renormalised weights in that order, and
    # the same tokens and renorm_out as the plain call.
    from tests.gpu_util import assert_slab_parity, run_gpu_slab

    w = wl(cfg)
    log("[gpu] slab export config %d %s" % (cfg, w.name))
    out = run_gpu_slab(sampler, w.probs, w.top_k, w.top_p, w.seed, w.offset, 1024)
    assert_slab_parity(orc, w.probs, w.top_k, w.top_p, w.seed, w.offset, 1024, out, w.name)
    st = sampler.stats(w.B)
    assert np.array_equal(out[5], st[:, 0]), "route differs from the recorded paths"
    # With the slab export, top-k and greedy rows record their support's
    # positive entries (stats word 10), min(k_eff, positive entries) of them;
    # rows whose list holds the whole support are exported from it.
    listed = np.isin(st[:, 0], [0, 4, 5])
    k_eff = np.where((w.top_k <= 0) | (w.top_k >= w.V), w.V, w.top_k)
    expect = np.minimum(k_eff, np.count_nonzero(w.probs > 0, axis=1))
    bad = np.flatnonzero(listed & (st[:, 10] != expect))
    assert bad.size == 0, "support lists: rows %s lengths %s expected %s" % (
        bad[:8], st[bad[:8], 10], expect[bad[:8]])
    log("[gpu]   %d rows exported from their support lists" % int(
        (listed & (st[:, 10] == k_eff)).sum()))


@pytest.mark.parametrize("V", [151936, 20000, 1000])
def test_slab_export_edge_rows(sampler, variant_samplers, orc, V):
    # Restream rows (zeros completing the support), ties, +inf, NaN, split
    # rows and the forced whole-row and tiny-buffer paths, at capacities
    # below and above the support sizes.
    from tests.gpu_util import assert_slab_parity, run_gpu_slab

    rng = np.random.default_rng(V + 31)
    p1, k1, q1, _ = _restream_batch(V, rng)
    p2, k2, q2, _ = _adversarial_batch(V, rng)
    probs = np.concatenate([p1, p2])
    ks = np.concatenate([k1, k2])
    ps = np.concatenate([q1, q2])
    for label, s in (("default", sampler), ("row_select", variant_samplers["row_select"]),
                     ("tiny_buffer", variant_samplers["tiny_buffer"])):
        for cap in (1024, 100):
            log("[gpu] slab edge rows V=%d %s cap %d" % (V, label, cap))
            out = run_gpu_slab(s, probs, ks, ps, 5, 9, cap)
            assert_slab_parity(orc, probs, ks, ps, 5, 9, cap, out, "slab V=%d %s" % (V, label))


def test_slab_export_split_rows(sampler, orc):
    from tests.gpu_util import assert_slab_parity, run_gpu_slab

    rng = np.random.default_rng(404)
    probs, ks, ps, _ = _split_batch(151936, rng)
    log("[gpu] slab export split rows")
    out = run_gpu_slab(sampler, probs, ks, ps, 2, 3, 1024)
    assert np.all(sampler.stats(len(ks))[:, 2] >= 2)
    assert_slab_parity(orc, probs, ks, ps, 2, 3, 1024, out, "slab split rows")


def test_route_report(sampler, variant_samplers):
    V = 151936
    ks = np.array([1, 2, 1024, 1025, V - 1, V, 0, -5, V + 7], np.int32)
    want = [4, 0, 0, 3, 3, 1, 1, 1, 1]
    assert sampler.route(V, ks).tolist() == want
    assert variant_samplers["row_select"].route(V, ks).tolist() == [3] * len(ks)
    # Greedy rows stay greedy for a one-entry vocabulary too (k_eff = V = 1).
    assert sampler.route(1, np.array([1, 0, 5], np.int32)).tolist() == [4, 4, 4]


def test_read_probe_reads_and_leaves_the_sink(torch_cuda):
    # The reference read kernel runs over ordinary data without writing its
    # sink (the fold of these bytes is not the sentinel) and reports success.
    torch = torch_cuda
    x = torch.arange(1 << 20, dtype=torch.float32, device="cuda")
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    log("[gpu] read probe")
    rc = tes.sampler_read_probe(x.data_ptr(), x.numel() * 4, sink.data_ptr(), 0,
                                torch.cuda.current_stream().cuda_stream)
    assert rc == tes.TES_OK
    assert tes.sampler_read_probe(x.data_ptr(), 0, sink.data_ptr(), 0, None) == tes.TES_OK
    torch.cuda.synchronize()
    assert int(sink.item()) == 7


def test_wide_draw_ranges_stay_on_the_fast_path(sampler, orc):
    # Top-p-only rows whose few large entries sit many octaves above the
    # bulk: before the boundary is known, a draw can fall anywhere from the
    # large entries down to the bulk, a range of up to ~150 coarse bins that
    # are almost all empty.  Only the bins with mass are exchanged (or, in
    # the one-workgroup row path this batch takes, listed), so these rows
    # stay on a fast path.
    B, V = 256, 151936
    rng = np.random.default_rng(4242)
    probs = np.empty((B, V), np.float32)
    for b in range(B):
        x = rng.standard_normal(V)
        e = np.exp(x - x.max())
        nb = int(rng.integers(1, 4))
        big = rng.dirichlet(np.ones(nb)) * rng.uniform(0.3, 0.7)
        row = e / e.sum() * (1.0 - big.sum())
        row[rng.choice(V, nb, replace=False)] = big
        probs[b] = row.astype(np.float32)
    ks = np.full(B, V, np.int32)
    ps = rng.uniform(0.85, 0.99, size=B).astype(np.float32)
    for off in (0, 1, 2):
        log("[gpu] wide draw ranges offset %d" % off)
        gtok, gren = run_gpu(sampler, probs, ks, ps, 77, off, renorm=(off == 0))
        st = sampler.stats(B)
        log("[gpu]   paths %s" % np.bincount(st[:, 0], minlength=6).tolist())
        assert_parity(orc, probs, ks, ps, 77, off, gtok, gren, "wide draw ranges %d" % off)
        slow = ~np.isin(st[:, 0], (1, 6))
        assert not slow.any(), "rows left the fast path: %s (why %s)" % (
            np.flatnonzero(slow), st[slow, 7])


def test_exchange_timeout_fallback(orc, torch_cuda):
    # Top-p-only rows cut into several segments exchange their histograms
    # through bounded waits.  With TES_FLAG_NO_WAIT every wait reports a
    # timeout without polling, so each such row takes the timeout path (failure flag, the last segment decides the row by whole-row
    # passes, the row state is reset).  Tokens, kept sets and renorm_out must
    # still equal the oracle's, and a second identical call (which starts
    # from the reset row state) must agree too.
    s = tes.Sampler(0, max_batch=1024, max_vocab=1 << 18,
                    flags=tes.TES_FLAG_NO_WAIT | tes.TES_FLAG_STATS)
    try:
        w3, w5 = wl(3), wl(5)
        rng = np.random.default_rng(77)
        full3 = np.flatnonzero(w3.top_k >= w3.V)
        rows3 = np.sort(np.concatenate([full3, rng.choice(np.flatnonzero(w3.top_k < w3.V), 16,
                                                          replace=False)]))
        rows5 = np.sort(rng.choice(w5.B, 24, replace=False))
        adv, aks, aps, _ = _adversarial_batch(262144, np.random.default_rng(262144))
        cases = [
            ("hetero subset", np.ascontiguousarray(w3.probs[rows3]), w3.top_k[rows3],
             w3.top_p[rows3], w3.seed, w3.offset),
            ("speculative-verify subset", np.ascontiguousarray(w5.probs[rows5]), w5.top_k[rows5],
             w5.top_p[rows5], w5.seed, w5.offset),
            ("adversarial V=262144", adv, aks, aps, 9, 3),
        ]
        for label, probs, ks, ps, seed, off in cases:
            V = probs.shape[1]
            multi = np.asarray(ks) >= V  # top-p-only rows (several segments at these V)
            for call in (1, 2):
                log("[gpu] exchange timeout fallback: %s call %d rows %d" % (label, call,
                                                                             len(ks)))
                gtok, gren = run_gpu(s, probs, ks, ps, seed, off, renorm=True)
                assert_parity(orc, probs, ks, ps, seed, off, gtok, gren,
                              "timeout fallback %s call %d" % (label, call))
                st = s.stats(len(ks))
                assert np.all(st[multi, 2] >= 2), "top-p-only rows were not segmented"
                assert np.all(st[multi, 0] == 2), "paths %s" % st[multi, 0]
                assert np.all(st[multi, 7] & 5), "timeout bits %s" % st[multi, 7]
    finally:
        s.close()
