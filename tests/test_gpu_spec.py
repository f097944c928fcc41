"""GPU parity of speculative verification (spec_verify_sample) through the C
ABI against the CPU oracle's spec_verify: output tokens and accepted counts
bit-exact, on the speculative-verify shape (64 requests x (7 drafts + 1
bonus row), V=262,144), on mixed top-k / top-p target rows, with random
draft-to-target maps, every forced internal path, batches over several
launches, the scalar row path and invalid maps and tokens."""

import numpy as np
import pytest

import top_exact_sampling_amd as tes
import workloads
from tests.gpu_util import log

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
        _WL[cfg] = workloads.make_spec(cfg)
    return _WL[cfg]


def run_spec(torch, sampler, target, Lt, ks, ps, draft, toks, tmap, seed, off, aligned=True):
    def dev(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a, dt)).cuda()

    if aligned:
        td = dev(target, np.float32)
    else:
        flat = torch.zeros(target.size + 1, dtype=torch.float32, device="cuda")
        flat[1:] = torch.from_numpy(np.ascontiguousarray(target).reshape(-1)).cuda()
        td = flat[1:].view(target.shape)
    out, acc = sampler.spec_verify(td, Lt, dev(ks, np.int32), dev(ps, np.float32),
                                   dev(draft, np.float32), dev(toks, np.int32), seed, off,
                                   target_map=None if tmap is None else dev(tmap, np.int32))
    torch.cuda.synchronize()
    return out.cpu().numpy(), acc.cpu().numpy()


def assert_spec_parity(orc, target, Lt, ks, ps, draft, toks, tmap, seed, off, gout, gacc, label):
    oout, oacc = orc.spec_verify(target, Lt, ks, ps, draft, toks, tmap, seed, off)
    bad = np.flatnonzero((gout != oout).any(axis=1) | (gacc != oacc))
    assert bad.size == 0, "%s: %d requests differ; first %s gpu %s/%s oracle %s/%s" % (
        label, bad.size, bad[:4], gout[bad[:2]].tolist(), gacc[bad[:2]].tolist(),
        oout[bad[:2]].tolist(), oacc[bad[:2]].tolist())
    return oacc


@pytest.mark.parametrize("cfg", [2, 5])
def test_spec_verify_parity(samplers, orc, torch_cuda, cfg):
    w = wl(cfg)
    for off in (0, 1, 2):
        log("[gpu] spec verify %s offset %d" % (w.name, off))
        gout, gacc = run_spec(torch_cuda, samplers["plain"], w.target, w.Lt, w.top_k, w.top_p,
                              w.draft, w.draft_tokens, None, w.seed, off)
        oacc = assert_spec_parity(orc, w.target, w.Lt, w.top_k, w.top_p, w.draft, w.draft_tokens,
                                  None, w.seed, off, gout, gacc, w.name)
        log("[gpu]   accepted lengths %s" % np.bincount(oacc, minlength=w.Lt).tolist())


@pytest.mark.parametrize("variant", ["row_select", "tiny_buffer", "small_segments", "no_wait",
                                     "row_topp"])
def test_spec_verify_forced_paths(samplers, orc, torch_cuda, variant):
    w = wl(2)
    log("[gpu] spec verify %s on %s" % (variant, w.name))
    gout, gacc = run_spec(torch_cuda, samplers[variant], w.target, w.Lt, w.top_k, w.top_p,
                          w.draft, w.draft_tokens, None, w.seed, 4)
    assert_spec_parity(orc, w.target, w.Lt, w.top_k, w.top_p, w.draft, w.draft_tokens, None,
                       w.seed, 4, gout, gacc, "%s/%s" % (variant, w.name))


def _random_batch(rng, N, L, Lt, V, special):
    x = 2.0 * rng.standard_normal((N * Lt, V))
    x[np.arange(N * Lt), rng.integers(0, V, N * Lt)] += 8.0
    e = np.exp(x - x.max(1, keepdims=True))
    target = (e / e.sum(1, keepdims=True)).astype(np.float32)
    ks = rng.choice(np.array([1, 5, 50, 1024, 2000, 0], np.int32), size=N * Lt)
    ps = rng.uniform(0.5, 1.0, N * Lt).astype(np.float32)
    src = target[rng.integers(0, N * Lt, N * L)] if L else np.zeros((0, V), np.float32)
    noise = rng.standard_normal(src.shape) * 0.7
    d = np.exp(np.log(np.maximum(src.astype(np.float64), 1e-30)) + noise)
    draft = (d / d.sum(1, keepdims=True)).astype(np.float32) if L else src
    toks = np.stack([[rng.choice(V, p=draft[n * L + l].astype(np.float64) /
                                 draft[n * L + l].astype(np.float64).sum())
                      for l in range(L)] for n in range(N)]).astype(np.int32).reshape(N, L)
    if special:
        # +inf, NaN, zero and negative target rows and draft entries; p = q rows.
        target[0] = 0.0
        target[1, :3] = np.inf
        target[2, rng.choice(V, 5)] = np.nan
        target[3] = -target[3]
        if L:
            draft[0, rng.choice(V, 7)] = np.nan
            draft[1] = 0.0
            draft[min(2, N * L - 1)] = target[min(2, N * L - 1)]
    tmap = rng.integers(0, Lt, size=(N, L + 1)).astype(np.int32)
    return target, ks, ps, draft, toks, tmap


@pytest.mark.parametrize("L", [0, 1, 3, 7, 63])
def test_spec_verify_random_maps(samplers, orc, torch_cuda, L):
    rng = np.random.default_rng(L + 300)
    N, V = 24 if L < 63 else 4, 20000
    Lt = L + 3
    target, ks, ps, draft, toks, tmap = _random_batch(rng, N, L, Lt, V, special=True)
    for use_map in (True, False):
        m = tmap if use_map else None
        log("[gpu] spec verify random batch L=%d map=%s" % (L, use_map))
        gout, gacc = run_spec(torch_cuda, samplers["plain"], target, Lt, ks, ps, draft, toks, m,
                              77, L)
        assert_spec_parity(orc, target, Lt, ks, ps, draft, toks, m, 77, L, gout, gacc,
                           "random L=%d map=%s" % (L, use_map))


def test_spec_verify_several_launches_and_scalar_rows(samplers, orc, torch_cuda):
    # 300 requests x 8 target rows = 2400 rows: three launches of whole
    # requests; then the same on unaligned rows (one-float loads).
    rng = np.random.default_rng(5)
    N, L, V = 300, 5, 4096
    Lt = 8
    target, ks, ps, draft, toks, tmap = _random_batch(rng, N, L, Lt, V, special=False)
    for aligned in (True, False):
        log("[gpu] spec verify N=%d rows=%d aligned=%s" % (N, N * Lt, aligned))
        gout, gacc = run_spec(torch_cuda, samplers["plain"], target, Lt, ks, ps, draft, toks, tmap,
                              3, 9, aligned=aligned)
        assert_spec_parity(orc, target, Lt, ks, ps, draft, toks, tmap, 3, 9, gout, gacc,
                           "several launches aligned=%s" % aligned)


def test_spec_verify_invalid_maps_and_tokens(samplers, orc, torch_cuda):
    rng = np.random.default_rng(8)
    N, L, V, Lt = 6, 3, 1000, 4
    target, ks, ps, draft, toks, tmap = _random_batch(rng, N, L, Lt, V, special=False)
    toks[1, 2] = V
    toks[2, 0] = -3
    tmap[3, 3] = Lt
    tmap[4, 0] = -1
    log("[gpu] spec verify invalid maps and tokens")
    gout, gacc = run_spec(torch_cuda, samplers["plain"], target, Lt, ks, ps, draft, toks, tmap,
                          1, 1)
    oacc = assert_spec_parity(orc, target, Lt, ks, ps, draft, toks, tmap, 1, 1, gout, gacc,
                              "invalid")
    assert oacc[1:5].tolist() == [-1, -1, -1, -1]
    assert np.all(gout[1:5] == -1)


def test_spec_verify_argument_errors(samplers, torch_cuda):
    torch = torch_cuda
    h = samplers["plain"].handle
    t = torch.zeros(8, 16, device="cuda")
    k = torch.zeros(8, dtype=torch.int32, device="cuda")
    q = torch.ones(8, device="cuda")
    d = torch.zeros(6, 16, device="cuda")
    dt = torch.zeros(2, 3, dtype=torch.int32, device="cuda")
    o = torch.zeros(2, 4, dtype=torch.int32, device="cuda")
    a = torch.zeros(2, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    args = [h, t.data_ptr(), 2, 4, 16, k.data_ptr(), q.data_ptr(), d.data_ptr(), 3, dt.data_ptr(),
            None, 1, 1, o.data_ptr(), a.data_ptr(), st]
    assert tes.spec_verify_sample(*args) == tes.TES_OK
    bad = list(args)
    bad[8] = 64  # L above 63
    assert tes.spec_verify_sample(*bad) == tes.TES_ERR_INVALID_ARGUMENT
    bad = list(args)
    bad[3] = 3  # Lt < L + 1 without a map
    assert tes.spec_verify_sample(*bad) == tes.TES_ERR_INVALID_ARGUMENT
    bad = list(args)
    bad[13] = None
    assert tes.spec_verify_sample(*bad) == tes.TES_ERR_INVALID_ARGUMENT
    bad = list(args)
    bad[2] = 10**6
    assert tes.spec_verify_sample(*bad) == tes.TES_ERR_TOO_LARGE
    torch.cuda.synchronize()
