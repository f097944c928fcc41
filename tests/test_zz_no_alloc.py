"""The allocation-free entry point (topk_topp_sample_noalloc) against the
handle-based topk_topp_sample: same inputs, same outputs.

Called through the C ABI on the current device.  Two calls in a row (the
second with a smaller input), then a batch of more rows than one launch of
the entry point takes, then a vocabulary above its limit (rejected on the
host)."""

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


def _run_both(torch, sampler, probs, top_k, top_p, seed, offset):
    B, V = probs.shape
    pd = torch.from_numpy(np.ascontiguousarray(probs)).cuda()
    kd = torch.from_numpy(np.ascontiguousarray(top_k, np.int32)).cuda()
    qd = torch.from_numpy(np.ascontiguousarray(top_p, np.float32)).cuda()
    st = torch.cuda.current_stream()
    outs = []
    for which in ("handle", "noalloc"):
        tok = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        ren = torch.full((B, V), -1.0, dtype=torch.float32, device="cuda")
        if which == "handle":
            rc = tes.topk_topp_sample(sampler.handle, pd.data_ptr(), B, V, kd.data_ptr(),
                                      qd.data_ptr(), seed, offset, tok.data_ptr(), ren.data_ptr(),
                                      st.cuda_stream)
        else:
            rc = tes.topk_topp_sample_noalloc(pd.data_ptr(), B, V, kd.data_ptr(), qd.data_ptr(),
                                              seed, offset, tok.data_ptr(), ren.data_ptr(),
                                              st.cuda_stream)
        assert rc == tes.TES_OK, (which, rc)
        torch.cuda.synchronize()
        outs.append((tok.cpu().numpy(), ren.cpu().numpy()))
    return outs


def _assert_same(outs, label):
    (ht, hr), (nt, nr) = outs
    bad = np.flatnonzero(ht != nt)
    assert bad.size == 0, "%s: tokens differ on rows %s" % (label, bad[:8])
    assert np.array_equal(hr != 0, nr != 0), label + ": kept sets differ"
    nz = hr != 0
    if nz.any():
        rel = np.abs(nr[nz].astype(np.float64) - hr[nz]) / np.abs(hr[nz])
        assert rel.max() <= REL_TOL, "%s: renorm rel err %.3g" % (label, rel.max())


def test_noalloc_matches_the_handle_entry_point(torch_cuda):
    torch = torch_cuda
    sampler = tes.Sampler(0, max_batch=1024, max_vocab=1 << 18)
    try:
        w3 = workloads.make(3)
        log("[gpu] noalloc call 1: %s B=%d V=%d" % (w3.name, w3.B, w3.V))
        _assert_same(_run_both(torch, sampler, w3.probs, w3.top_k, w3.top_p, w3.seed, 5),
                     "noalloc hetero")
        w2 = workloads.make(2)
        log("[gpu] noalloc call 2 (smaller): %s B=%d V=%d" % (w2.name, w2.B, w2.V))
        _assert_same(_run_both(torch, sampler, w2.probs, w2.top_k, w2.top_p, w2.seed, 6),
                     "noalloc small")
        w5 = workloads.make(5)
        rows = np.arange(0, 320)
        probs = np.ascontiguousarray(w5.probs[rows])
        log("[gpu] noalloc call 3 (two launches): B=%d V=%d" % probs.shape)
        _assert_same(_run_both(torch, sampler, probs, w5.top_k[rows], w5.top_p[rows], w5.seed,
                               7), "noalloc two launches")
        log("[gpu] noalloc call 4 (smaller again): B=4 V=1000")
        w1 = workloads.make(1)
        _assert_same(_run_both(torch, sampler, w1.probs, w1.top_k, w1.top_p, w1.seed, 8),
                     "noalloc tiny")
    finally:
        sampler.close()


def test_noalloc_rejects_sizes_beyond_its_limit(torch_cuda):
    torch = torch_cuda
    st = torch.cuda.current_stream().cuda_stream
    assert tes.topk_topp_sample_noalloc(0, 0, 10, 0, 0, 0, 0, 0, None, st) == tes.TES_OK
    assert tes.topk_topp_sample_noalloc(0, 4, (1 << 18) + 4, 0, 0, 0, 0, 0, None, st) == \
        tes.TES_ERR_TOO_LARGE
    assert tes.topk_topp_sample_noalloc(0, -1, 10, 0, 0, 0, 0, 0, None, st) == \
        tes.TES_ERR_INVALID_ARGUMENT
    assert tes.topk_topp_sample_noalloc(0, 4, 10, 0, 0, 0, 0, 0, None, st) == \
        tes.TES_ERR_INVALID_ARGUMENT
