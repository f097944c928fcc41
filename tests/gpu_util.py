"""Shared helpers for the GPU parity tests: run the HIP sampler through the C
ABI and compare with the CPU oracle."""

from __future__ import annotations

import sys

import numpy as np

REL_TOL = 1e-6  # renorm_out tolerance, relative


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_gpu(sampler, probs, top_k, top_p, seed, offset, renorm=True, probs_dev=None):
    """Run the HIP sampler; returns (tokens, renorm or None) as numpy."""
    import torch

    B, V = probs.shape
    pd = probs_dev if probs_dev is not None else to_dev(probs, torch)
    kd = to_dev(np.asarray(top_k, np.int32), torch)
    qd = to_dev(np.asarray(top_p, np.float32), torch)
    tok = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    ren = torch.full((B, V), -1.0, dtype=torch.float32, device="cuda") if renorm else None
    sampler.sample(pd, kd, qd, seed, offset, out_tokens=tok, renorm_out=ren)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), (ren.cpu().numpy() if renorm else None)


def assert_parity(orc, probs, top_k, top_p, seed, offset, gtok, gren, label):
    want_ren = gren is not None
    otok, oren, info = orc.sample(probs, top_k, top_p, seed, offset, want_renorm=want_ren,
                                  want_info=True)
    bad = np.flatnonzero(gtok != otok)
    assert bad.size == 0, (
        "%s: %d token mismatches; rows %s gpu %s oracle %s kind %s k %s" %
        (label, bad.size, bad[:8], gtok[bad[:8]], otok[bad[:8]], info[bad[:8], 9],
         np.asarray(top_k)[bad[:8]]))
    if want_ren:
        assert np.all(np.isfinite(gren)), label + ": non-finite renorm_out"
        nzg, nzo = gren != 0, oren != 0
        rows = np.flatnonzero((nzg != nzo).any(axis=1))
        assert rows.size == 0, "%s: kept-set mismatch on rows %s (gpu %s oracle %s)" % (
            label, rows[:8], nzg[rows[:8]].sum(1), nzo[rows[:8]].sum(1))
        if nzo.any():
            rel = np.abs(gren[nzo].astype(np.float64) - oren[nzo]) / oren[nzo]
            assert rel.max() <= REL_TOL, "%s: renorm rel err %.3g" % (label, rel.max())
    return otok, info


def run_gpu_slab(sampler, probs, top_k, top_p, seed, offset, cap):
    """Run the sampler with the slab export; returns numpy (tokens, renorm,
    slab_index, slab_renorm, slab_len, route)."""
    import torch

    B, V = probs.shape
    pd = to_dev(probs, torch)
    kd = to_dev(np.asarray(top_k, np.int32), torch)
    qd = to_dev(np.asarray(top_p, np.float32), torch)
    ren = torch.full((B, V), -1.0, dtype=torch.float32, device="cuda")
    tok, si, sr, sl, rt = sampler.sample_slab(pd, kd, qd, seed, offset, cap, renorm_out=ren)
    torch.cuda.synchronize()
    return (tok.cpu().numpy(), ren.cpu().numpy(), si.cpu().numpy(), sr.cpu().numpy(),
            sl.cpu().numpy(), rt.cpu().numpy().view(np.uint32))


def assert_slab_parity(orc, probs, top_k, top_p, seed, offset, cap, out, label):
    """Tokens and renorm_out as assert_parity; the slab against the oracle's
    support order (bit-exact indices and lengths) and its renormalised weights
    (1e-6 relative, zeros exact)."""
    import oracle

    gtok, gren, si, sr, sl, rt = out
    otok, _ = assert_parity(orc, probs, top_k, top_p, seed, offset, gtok, gren, label)
    _, oren, _ = orc.sample(probs, top_k, top_p, seed, offset, want_renorm=True)
    oi, ow, ol = oracle.slab(orc, probs, top_k, cap, oren)
    bad = np.flatnonzero(sl != ol)
    assert bad.size == 0, "%s: slab length mismatch rows %s (gpu %s oracle %s)" % (
        label, bad[:8], sl[bad[:8]], ol[bad[:8]])
    bad = np.flatnonzero((si != oi).any(axis=1))
    assert bad.size == 0, "%s: slab order mismatch on rows %s" % (label, bad[:8])
    assert np.array_equal(sr == 0, ow == 0), label + ": slab zero pattern"
    nz = ow != 0
    if nz.any():
        rel = np.abs(sr[nz].astype(np.float64) - ow[nz]) / ow[nz]
        assert rel.max() <= REL_TOL, "%s: slab weight rel err %.3g" % (label, rel.max())
    assert np.all(np.isin(rt, [0, 1, 2, 3, 4, 5])), label + ": route codes"
    return otok
