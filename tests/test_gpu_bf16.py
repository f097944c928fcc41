"""GPU parity for bfloat16 probability rows (topk_topp_sample_bf16).

A bf16 entry means its exact widening to fp32 (its 16 bits become the upper
half of the fp32 word), so the oracle runs on the widened rows and the bar is
the fp32 one: tokens and kept sets bit-exact, renorm_out within 1e-6
relative.  Rows are rounded to bf16 by torch on the CPU; whatever bits that
gives (NaN payloads included) are what both sides read.
"""

import numpy as np
import pytest

import top_exact_sampling_amd as tes
import workloads
from tests.gpu_util import assert_parity, log, to_dev
from tests.test_gpu_parity import (_above_one_batch, _adversarial_batch, _restream_batch,
                                   _split_batch)

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
def variants(torch_cuda):
    out = {
        "row_select": tes.Sampler(0, 1024, 1 << 18, tes.TES_FLAG_FORCE_ROW_SELECT),
        "tiny_buffer": tes.Sampler(0, 1024, 1 << 18, tes.TES_FLAG_TINY_BUFFER),
        "small_tiny": tes.Sampler(
            0, 1024, 1 << 18, tes.TES_FLAG_SMALL_SEGMENTS | tes.TES_FLAG_TINY_BUFFER),
        "row_topp": tes.Sampler(0, 1024, 1 << 18, tes.TES_FLAG_ROW_TOPP),
    }
    yield out
    for s in out.values():
        s.close()


def to_bf16_bits(probs):
    """fp32 rows -> (uint16 bf16 bit patterns, their fp32 widening)."""
    import torch

    bits = torch.from_numpy(np.ascontiguousarray(probs, np.float32)).to(torch.bfloat16)
    b16 = bits.view(torch.int16).numpy().view(np.uint16).copy()
    wide = (b16.astype(np.uint32) << 16).view(np.float32)
    return b16, wide


def run_bf16(sampler, b16, top_k, top_p, seed, offset, renorm=True):
    import torch

    B, V = b16.shape
    pd = to_dev(b16.view(np.int16), torch).view(torch.bfloat16)
    kd = to_dev(np.asarray(top_k, np.int32), torch)
    qd = to_dev(np.asarray(top_p, np.float32), torch)
    tok = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    ren = torch.full((B, V), -1.0, dtype=torch.float32, device="cuda") if renorm else None
    sampler.sample(pd, kd, qd, seed, offset, out_tokens=tok, renorm_out=ren)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), (ren.cpu().numpy() if renorm else None)


def check(sampler, orc, probs, ks, ps, seed, offset, label, renorm=True):
    b16, wide = to_bf16_bits(probs)
    log("[gpu] bf16 %s B=%d V=%d" % (label, b16.shape[0], b16.shape[1]))
    gtok, gren = run_bf16(sampler, b16, ks, ps, seed, offset, renorm)
    return assert_parity(orc, wide, ks, ps, seed, offset, gtok, gren, "bf16 " + label)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_config_parity(sampler, orc, cfg):
    w = workloads.make(cfg)
    check(sampler, orc, w.probs, w.top_k, w.top_p, w.seed, w.offset, w.name,
          renorm=cfg != 5)


@pytest.mark.parametrize("V", [151936, 5000, 1024])
def test_adversarial_rows(sampler, variants, orc, V):
    rng = np.random.default_rng(V + 3)
    probs, ks, ps, names = _adversarial_batch(V, rng)
    for label, s in (("default", sampler),) + tuple(variants.items()):
        check(s, orc, probs, ks, ps, 9, 3, "adversarial V=%d %s" % (V, label))


@pytest.mark.parametrize("V", [151936, 20000])
def test_entries_at_and_above_one(sampler, variants, orc, V):
    # bf16 entries of 1.0 and above (1.5, 3e38 round to bf16 values above
    # 1.0), NaN and negatives: the saturating mass conversion on 8-entry
    # vectors, on the segment path and the one-workgroup path.
    probs, ks, ps = _above_one_batch(V, np.random.default_rng(V + 2))
    for label, s in (("default", sampler), ("row_topp", variants["row_topp"])):
        check(s, orc, probs, ks, ps, 21, 5, "above one V=%d %s" % (V, label))


@pytest.mark.parametrize("V", [151936, 128256, 20000])
def test_restream_rows(sampler, orc, V):
    # The compacting restream appends an 8-entry vector in two halves.
    rng = np.random.default_rng(V + 29)
    probs, ks, ps, names = _restream_batch(V, rng)
    check(sampler, orc, probs, ks, ps, 13, 2, "restream V=%d" % V)
    st = sampler.stats(len(names))
    log("[gpu]   paths %s" % np.bincount(st[:, 0], minlength=6).tolist())
    assert (st[:, 0] == 5).sum() >= 4, "the compacting pass did not run"


def test_split_rows(sampler, orc):
    rng = np.random.default_rng(151941)
    probs, ks, ps, names = _split_batch(151936, rng)
    check(sampler, orc, probs, ks, ps, 21, 4, "split rows")
    st = sampler.stats(len(names))
    log("[gpu]   parts per row %s" % np.unique(st[:, 2]).tolist())


def test_exchange_timeout_fallback(orc, torch_cuda):
    # bf16 top-p-only segments publish their whole fine histograms with the
    # first exchange and have no second one.  With TES_FLAG_NO_WAIT every
    # wait reports a timeout without polling: each segment flags the row and
    # the last segment decides it by whole-row passes (path 2).  Tokens, kept
    # sets and renorm_out must equal the oracle's, also on a second identical
    # call (from the reset row state).
    s = tes.Sampler(0, 1024, 1 << 18, tes.TES_FLAG_NO_WAIT | tes.TES_FLAG_STATS)
    try:
        w3 = workloads.make(3)
        rng = np.random.default_rng(78)
        full3 = np.flatnonzero(w3.top_k >= w3.V)
        rows3 = np.sort(np.concatenate([full3, rng.choice(np.flatnonzero(w3.top_k < w3.V), 16,
                                                          replace=False)]))
        adv, aks, aps, _ = _adversarial_batch(262144, np.random.default_rng(262145))
        cases = [
            ("hetero subset", np.ascontiguousarray(w3.probs[rows3]), w3.top_k[rows3],
             w3.top_p[rows3], w3.seed, w3.offset),
            ("adversarial V=262144", adv, aks, aps, 9, 3),
        ]
        for label, probs, ks, ps, seed, off in cases:
            multi = np.asarray(ks) >= probs.shape[1]
            for call in (1, 2):
                check(s, orc, probs, ks, ps, seed, off,
                      "timeout fallback %s call %d" % (label, call))
                st = s.stats(len(ks))
                assert np.all(st[multi, 2] >= 2), "top-p-only rows were not segmented"
                assert np.all(st[multi, 7] & 1), "timeout bits %s" % st[multi, 7]
                assert not np.any(st[multi, 7] & 4), "bf16 rows have no second exchange"
                assert np.all(st[multi, 0] == 2), "paths %s" % st[multi, 0]
    finally:
        s.close()


@pytest.mark.parametrize("trial", range(4))
def test_random_shapes(sampler, orc, trial):
    rng = np.random.default_rng(2000 + trial)
    B = int(rng.integers(1, 80))
    V = 8 * int(rng.choice([int(rng.integers(1, 40)), int(rng.integers(40, 2500)),
                            int(rng.integers(2500, 18000))]))
    x = float(rng.choice([0.3, 2.0, 6.0])) * rng.standard_normal((B, V))
    e = np.exp(x - x.max(1, keepdims=True))
    probs = (e / e.sum(1, keepdims=True)).astype(np.float32)
    ks = rng.integers(-3, V + 5, size=B).astype(np.int32)
    ks[rng.random(B) < 0.3] = 1
    ps = rng.uniform(-0.2, 1.3, size=B).astype(np.float32)
    seed, off = (int(v) for v in rng.integers(0, 2**63, size=2))
    check(sampler, orc, probs, ks, ps, seed, off, "random trial %d" % trial)


def test_multi_launch_batch(sampler, orc):
    B, V = 1500, 4096
    rng = np.random.default_rng(1500)
    x = 2.0 * rng.standard_normal((B, V))
    x[np.arange(B), rng.integers(0, V, size=B)] += 10.0
    e = np.exp(x - x.max(1, keepdims=True))
    probs = (e / e.sum(1, keepdims=True)).astype(np.float32)
    ks = rng.choice(np.array([1, 7, 300, 1024, 2000, 0, V], np.int32), size=B)
    ps = rng.uniform(0.3, 1.0, size=B).astype(np.float32)
    check(sampler, orc, probs, ks, ps, 99, 7, "multi-launch")


def test_matches_the_fp32_entry_on_widened_rows(sampler, torch_cuda):
    torch = torch_cuda
    w = workloads.make(2)
    b16, wide = to_bf16_bits(w.probs)
    kd, qd = to_dev(w.top_k, torch), to_dev(w.top_p, torch)
    a = sampler.sample(to_dev(b16.view(np.int16), torch).view(torch.bfloat16), kd, qd, 5, 1)
    b = sampler.sample(to_dev(wide, torch), kd, qd, 5, 1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_bf16_argument_errors(sampler, torch_cuda):
    torch = torch_cuda
    B, V = 4, 1000
    k = torch.ones(B, dtype=torch.int32, device="cuda")
    p = torch.ones(B, dtype=torch.float32, device="cuda")
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    flat = torch.zeros(B * V + 8, dtype=torch.bfloat16, device="cuda")
    ok = flat[:B * V].view(B, V)
    assert tes.topk_topp_sample_bf16(sampler.handle, ok.data_ptr(), B, V - 4, k.data_ptr(),
                                     p.data_ptr(), 0, 0, out.data_ptr(), None,
                                     None) == tes.TES_ERR_INVALID_ARGUMENT  # V % 8 != 0
    assert tes.topk_topp_sample_bf16(sampler.handle, flat.data_ptr() + 2, B, V, k.data_ptr(),
                                     p.data_ptr(), 0, 0, out.data_ptr(), None,
                                     None) == tes.TES_ERR_INVALID_ARGUMENT  # misaligned
    assert tes.topk_topp_sample_bf16(sampler.handle, ok.data_ptr(), 0, V, 0, 0, 0, 0, 0, None,
                                     None) == tes.TES_OK  # empty batch
