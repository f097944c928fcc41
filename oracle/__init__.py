"""CPU oracle for exact top-k -> top-p sampling (TEST INFRASTRUCTURE ONLY).

Only the tests, the package smoke check and the CPU-baseline leg of the
benchmark may import this package.  The HIP sampler never calls it and shares
no code with it.

``oracle/tes_oracle.cpp`` is the definition (plain C++, stable sort, 128-bit
integers, its own Philox4x32-10); this module builds it with the host
compiler and exposes it through ctypes.  ``oracle/brute.py`` is an
independent exact-rational brute force for tiny rows, used to pin it.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tes_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle_tes.so")
_lib = None

INFO_FIELDS = ("k_eff", "P", "m_inf", "M_k", "T", "kept", "M_p", "t", "pos", "kind")


def build(force: bool = True, out: str | None = None, src: str | None = None) -> str:
    """Compile the oracle into a shared library with g++ and return its path."""
    out = out or _LIB
    src = src or _SRC
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    # -ffp-contract=off: every fp32 operation of the logit weights is the one
    # written (no multiply-add fusion the source does not ask for).
    cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-shared", "-fPIC", "-pthread",
           "-o", tmp, src]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class Oracle:
    """ctypes view of one built oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        lib.oracle_philox4x32_10.argtypes = [u32p, u32p, u32p]
        lib.oracle_philox4x32_10.restype = None
        lib.oracle_uniform_u64.argtypes = [ctypes.c_uint64] * 3
        lib.oracle_uniform_u64.restype = ctypes.c_uint64
        lib.oracle_sample_row.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_uint64,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_sample_row.restype = ctypes.c_int
        lib.oracle_topk_topp_sample.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int]
        lib.oracle_topk_topp_sample.restype = ctypes.c_int
        lib.oracle_support.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_support.restype = ctypes.c_int64
        lib.oracle_exp_weight.argtypes = [ctypes.c_float]
        lib.oracle_exp_weight.restype = ctypes.c_float
        lib.oracle_logit_weights.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                                             ctypes.c_void_p]
        lib.oracle_logit_weights.restype = ctypes.c_int
        lib.oracle_sample_row_minp.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_float,
            ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_sample_row_minp.restype = ctypes.c_int
        lib.oracle_topk_topp_sample_logits.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_topk_topp_sample_logits.restype = ctypes.c_int
        lib.oracle_uniform_u64_hi.argtypes = [ctypes.c_uint64] * 3
        lib.oracle_uniform_u64_hi.restype = ctypes.c_uint64
        lib.oracle_spec_verify.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_spec_verify.restype = ctypes.c_int
        lib.oracle_accept_draft.argtypes = [ctypes.c_uint64] * 4
        lib.oracle_accept_draft.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    # -- Philox -------------------------------------------------------------
    def philox(self, ctr, key):
        c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
        k = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
        o = (ctypes.c_uint32 * 4)()
        self.lib.oracle_philox4x32_10(c, k, o)
        return [int(x) for x in o]

    def uniform_u64(self, seed: int, row: int, offset: int) -> int:
        return int(self.lib.oracle_uniform_u64(seed, row, offset))

    def uniform_u64_hi(self, seed: int, row: int, offset: int) -> int:
        """Philox words 2 and 3 of the row's block (the acceptance uniform)."""
        return int(self.lib.oracle_uniform_u64_hi(seed, row, offset))

    # -- speculative verification --------------------------------------------
    def spec_verify(self, target, Lt: int, top_k, top_p, draft, draft_tokens, target_map,
                    seed: int, offset: int, n_threads: int | None = None):
        """target [N*Lt][V], draft [N*L][V] (or [N][L][V]), draft_tokens [N][L],
        target_map [N][L+1] or None; returns (out_tokens [N][L+1], accept_len [N])."""
        target = np.ascontiguousarray(target, dtype=np.float32).reshape(-1, np.shape(target)[-1])
        V = target.shape[1]
        N = target.shape[0] // Lt
        toks = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(N, -1)
        L = toks.shape[1]
        dr = np.ascontiguousarray(draft, dtype=np.float32).reshape(-1, V) if L else None
        tk = np.ascontiguousarray(top_k, dtype=np.int32)
        tp = np.ascontiguousarray(top_p, dtype=np.float32)
        tm = None if target_map is None else np.ascontiguousarray(target_map, np.int32)
        out = np.zeros((N, L + 1), np.int32)
        acc = np.zeros(N, np.int32)
        if n_threads is None:
            n_threads = len(os.sched_getaffinity(0))
        rc = self.lib.oracle_spec_verify(
            target.ctypes.data, N, Lt, V, tk.ctypes.data, tp.ctypes.data,
            dr.ctypes.data if dr is not None else None, L, toks.ctypes.data,
            tm.ctypes.data if tm is not None else None, int(seed) & (2**64 - 1),
            int(offset) & (2**64 - 1), out.ctypes.data, acc.ctypes.data, int(n_threads))
        if rc:
            raise RuntimeError("oracle_spec_verify failed: %d" % rc)
        return out, acc

    # -- logit rows ---------------------------------------------------------
    def exp_weight(self, s: float) -> float:
        """E(s) of the logit-row weights (fp32 in, fp32 out)."""
        return float(np.float32(self.lib.oracle_exp_weight(float(np.float32(s)))))

    def logit_weights(self, row, tau: float):
        """The fp32 weights of one logit row at temperature tau."""
        row = np.ascontiguousarray(row, dtype=np.float32)
        w = np.zeros(row.size, np.float32)
        rc = self.lib.oracle_logit_weights(row.ctypes.data, row.size, float(np.float32(tau)),
                                           w.ctypes.data)
        if rc:
            raise RuntimeError("oracle_logit_weights failed: %d" % rc)
        return w

    def sample_logits(self, logits, top_k, top_p, temperature, min_p, seed: int, offset: int,
                      want_renorm: bool = False, want_info: bool = False,
                      n_threads: int | None = None):
        """Batched logit rows (temperature / min_p may be None: 1 and off)."""
        logits = np.ascontiguousarray(logits, dtype=np.float32)
        B, V = logits.shape
        top_k = np.ascontiguousarray(top_k, dtype=np.int32)
        top_p = np.ascontiguousarray(top_p, dtype=np.float32)
        tau = None if temperature is None else np.ascontiguousarray(temperature, np.float32)
        mp = None if min_p is None else np.ascontiguousarray(min_p, np.float32)
        tok = np.zeros(B, np.int32)
        ren = np.zeros((B, V), np.float32) if want_renorm else None
        info = np.zeros((B, 10), np.int64) if want_info else None
        if n_threads is None:
            n_threads = len(os.sched_getaffinity(0))
        rc = self.lib.oracle_topk_topp_sample_logits(
            logits.ctypes.data, B, V, top_k.ctypes.data, top_p.ctypes.data,
            tau.ctypes.data if tau is not None else None,
            mp.ctypes.data if mp is not None else None,
            int(seed) & (2**64 - 1), int(offset) & (2**64 - 1), tok.ctypes.data,
            ren.ctypes.data if ren is not None else None,
            info.ctypes.data if info is not None else None, int(n_threads))
        if rc:
            raise RuntimeError("oracle_topk_topp_sample_logits failed: %d" % rc)
        return tok, ren, info

    # -- sampling -------------------------------------------------------------
    def sample_row(self, row, top_k: int, top_p: float, u: int, want_renorm: bool = True,
                   min_p: float = 0.0):
        row = np.ascontiguousarray(row, dtype=np.float32)
        V = row.size
        tok = np.zeros(1, np.int32)
        ren = np.zeros(V, np.float32) if want_renorm else None
        info = np.zeros(10, np.int64)
        rc = self.lib.oracle_sample_row_minp(
            row.ctypes.data, V, int(top_k), float(top_p), float(min_p), int(u) & (2**64 - 1),
            tok.ctypes.data, ren.ctypes.data if ren is not None else None, info.ctypes.data)
        if rc:
            raise RuntimeError("oracle_sample_row failed: %d" % rc)
        return int(tok[0]), ren, dict(zip(INFO_FIELDS, (int(x) for x in info)))

    def sample(self, probs, top_k, top_p, seed: int, offset: int, want_renorm: bool = False,
               want_info: bool = False, n_threads: int | None = None):
        probs = np.ascontiguousarray(probs, dtype=np.float32)
        B, V = probs.shape
        top_k = np.ascontiguousarray(top_k, dtype=np.int32)
        top_p = np.ascontiguousarray(top_p, dtype=np.float32)
        assert top_k.shape == (B,) and top_p.shape == (B,)
        tok = np.zeros(B, np.int32)
        ren = np.zeros((B, V), np.float32) if want_renorm else None
        info = np.zeros((B, 10), np.int64) if want_info else None
        if n_threads is None:
            n_threads = len(os.sched_getaffinity(0))
        rc = self.lib.oracle_topk_topp_sample(
            probs.ctypes.data, B, V, top_k.ctypes.data, top_p.ctypes.data,
            int(seed) & (2**64 - 1), int(offset) & (2**64 - 1), tok.ctypes.data,
            ren.ctypes.data if ren is not None else None,
            info.ctypes.data if info is not None else None, int(n_threads))
        if rc:
            raise RuntimeError("oracle_topk_topp_sample failed: %d" % rc)
        return tok, ren, info


def slab(orc: Oracle, probs, top_k, cap: int, renorm):
    """Per row: the support's indices in sorted order (descending
    probability, ascending index) and their renormalised weights taken from
    ``renorm`` (the oracle's dense renorm_out), for rows whose support holds
    at most ``cap`` entries; other rows get length -1.  Returns
    (index[B][cap] filled with -1, weight[B][cap] filled with 0, length[B])."""
    probs = np.ascontiguousarray(probs, dtype=np.float32)
    B, V = probs.shape
    idx = np.full((B, cap), -1, np.int32)
    wgt = np.zeros((B, cap), np.float32)
    length = np.full(B, -1, np.int32)
    buf = np.zeros(max(cap, 1), np.int32)
    for b in range(B):
        k_eff = int(orc.lib.oracle_support(probs[b].ctypes.data, V, int(top_k[b]), cap,
                                           buf.ctypes.data))
        if k_eff < 0:
            raise RuntimeError("oracle_support failed")
        if k_eff <= cap:
            idx[b, :k_eff] = buf[:k_eff]
            wgt[b, :k_eff] = renorm[b, buf[:k_eff]]
            length[b] = k_eff
    return idx, wgt, length


def load(path: str | None = None) -> Oracle:
    """Load the built oracle (building it first if it is missing or stale)."""
    global _lib
    if path is not None:
        return Oracle(path)
    if _lib is None:
        build(force=False)
        _lib = Oracle(_LIB)
    return _lib
