"""Seeded synthetic workloads for exact top-k -> top-p sampling.

This module only builds inputs: fp32 probability rows and the per-row
``top_k`` / ``top_p`` parameters.  It holds none of the sampling method's
arithmetic, so the CPU oracle and the GPU path can both consume it without
sharing any logic.

Every config follows one recipe, all in float64 until the final cast:

1. ``rng = numpy.random.default_rng(seed)`` (PCG64);
2. logits ``x = scale * rng.standard_normal((B, V))``;
3. per row, a few tokens get a boost (the low-entropy "informative" outliers
   that the Qrita page describes on top of quasi-Gaussian noise, section 3.1);
4. ``probs = exp(x - max) / sum`` per row, then cast to fp32 round-to-nearest.

The generator call order below is frozen: changing it changes every input.
The vocabulary sizes are those of real tokenizers named on the pages
(151,936 and 128,256 in the Qrita evaluation setup, 262,144 = 2**18 in the
SonicSampler top-k sweep); the data is synthetic because no model logits
are available.
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "SpecWorkload", "CONFIGS", "make", "make_logits", "make_spec",
           "softmax64", "sha256_of"]


@dataclass
class Workload:
    name: str
    probs: np.ndarray  # float32 [B, V], C-contiguous (logits for logit workloads)
    top_k: np.ndarray  # int32 [B]
    top_p: np.ndarray  # float32 [B]
    seed: int
    offset: int
    meta: dict = field(default_factory=dict)
    temperature: np.ndarray | None = None  # float32 [B], logit workloads only
    min_p: np.ndarray | None = None        # float32 [B], logit workloads only

    @property
    def B(self) -> int:
        return int(self.probs.shape[0])

    @property
    def V(self) -> int:
        return int(self.probs.shape[1])


def softmax64(x: np.ndarray) -> np.ndarray:
    """Row softmax in float64: exp(x - rowmax) / rowsum."""
    m = x.max(axis=1, keepdims=True)
    e = np.exp(x - m)
    e /= e.sum(axis=1, keepdims=True)
    return e


def _boost_rows(rng, x, n_lo, n_hi, b_lo, b_hi):
    """Per row: n ~ U{n_lo..n_hi} distinct tokens get a boost ~ U[b_lo, b_hi]."""
    B, V = x.shape
    for b in range(B):
        n = int(rng.integers(n_lo, n_hi + 1))
        idx = rng.choice(V, n, replace=False)
        x[b, idx] += rng.uniform(b_lo, b_hi, size=n)


def _rows_out(x, logits):
    """fp32 logits (logit workloads) or fp32 probabilities of float64 logits."""
    return x.astype(np.float32) if logits else softmax64(x).astype(np.float32)


def _cfg1(logits=False):
    # Tiny reference: B=4, V=1000, 3 random tokens boosted by +10, k=50, p=0.9.
    B, V, seed = 4, 1000, 0
    rng = np.random.default_rng(seed)
    x = 2.0 * rng.standard_normal((B, V))
    for b in range(B):
        idx = rng.choice(V, 3, replace=False)
        x[b, idx] += 10.0
    probs = _rows_out(x, logits)
    top_k = np.full(B, 50, np.int32)
    top_p = np.full(B, 0.9, np.float32)
    return Workload("tiny_b4_v1000", probs, top_k, top_p, seed, 0)


def _cfg2(logits=False):
    # B=64, V=32,000, low-entropy rows; k ~ U{1..1024}, p ~ U[0.5, 1.0].
    B, V, seed = 64, 32000, 1
    rng = np.random.default_rng(seed)
    x = 2.0 * rng.standard_normal((B, V))
    _boost_rows(rng, x, 1, 8, 8.0, 15.0)
    probs = _rows_out(x, logits)
    top_k = rng.integers(1, 1025, size=B).astype(np.int32)
    top_p = rng.uniform(0.5, 1.0, size=B).astype(np.float32)
    return Workload("b64_v32000", probs, top_k, top_p, seed, 0)


def _cfg3(logits=False):
    # Heterogeneous batch B=256, V=151,936: 25% greedy (k=1), 25% top-p only
    # (k=V, p ~ U[0.8, 0.99]), 50% k ~ U{20..1024} with p ~ U[0.7, 1.0].
    B, V, seed = 256, 151936, 2
    rng = np.random.default_rng(seed)
    x = 2.0 * rng.standard_normal((B, V))
    _boost_rows(rng, x, 1, 8, 8.0, 15.0)
    probs = _rows_out(x, logits)
    perm = rng.permutation(B)
    greedy, full, slab = perm[:64], perm[64:128], perm[128:]
    top_k = np.empty(B, np.int32)
    top_p = np.empty(B, np.float32)
    top_k[greedy] = 1
    top_p[greedy] = 1.0
    top_k[full] = V
    top_p[full] = rng.uniform(0.8, 0.99, size=full.size).astype(np.float32)
    top_k[slab] = rng.integers(20, 1025, size=slab.size)
    top_p[slab] = rng.uniform(0.7, 1.0, size=slab.size).astype(np.float32)
    cls = np.empty(B, dtype="<U6")
    cls[greedy], cls[full], cls[slab] = "greedy", "full", "slab"
    return Workload("hetero_b256_v151936", probs, top_k, top_p, seed, 0, {"row_class": cls})


_NAN_PATTERNS = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0x7FFFFFFF], dtype=np.uint32)


def _cfg4(logits=False):
    # Ties and edge rows: B=1024, V=128,256, probs quantised to multiples of
    # 2**-20 then renormalised; 1% all-zero rows, 1% rows with NaN / negative /
    # -0.0 entries, 1% rows with 2-5 +inf entries.  As logits: the logits
    # quantised to multiples of 1/4 (ties); all -inf rows for the zero rows.
    B, V, seed = 1024, 128256, 3
    rng = np.random.default_rng(seed)
    x = 2.0 * rng.standard_normal((B, V))
    _boost_rows(rng, x, 1, 8, 8.0, 15.0)
    if logits:
        probs = (np.rint(x * 4.0) / 4.0).astype(np.float32)
        del x
    else:
        p64 = softmax64(x)
        del x
        p64 = np.rint(p64 * 2.0**20) * 2.0**-20
        p64 /= p64.sum(axis=1, keepdims=True)
        probs = p64.astype(np.float32)
        del p64
    perm = rng.permutation(B)
    zero_rows, nan_rows, inf_rows = perm[:10], perm[10:20], perm[20:30]
    probs[zero_rows] = -np.inf if logits else 0.0
    bits = probs.view(np.uint32)
    for b in nan_rows:
        am = int(np.argmax(probs[b]))
        idx = rng.choice(V, 12, replace=False)
        bits[b, am] = _NAN_PATTERNS[0]
        bits[b, idx[:4]] = _NAN_PATTERNS
        probs[b, idx[4:8]] = -probs[b, idx[4:8]]
        bits[b, idx[8:12]] = 0x80000000  # -0.0
    for b in inf_rows:
        n = int(rng.integers(2, 6))
        idx = rng.choice(V, n, replace=False)
        probs[b, idx] = np.inf
    top_k = rng.integers(1, 1025, size=B).astype(np.int32)
    top_p = rng.uniform(0.5, 1.0, size=B).astype(np.float32)
    cls = np.full(B, "plain", dtype="<U5")
    cls[zero_rows], cls[nan_rows], cls[inf_rows] = "zero", "nan", "inf"
    return Workload("ties_edges_b1024_v128256", probs, top_k, top_p, seed, 0, {"row_class": cls})


def _cfg5(logits=False):
    # Speculative-verify shape, top-p only: 64 requests x 8 draft positions =
    # 512 rows, V=262,144, high-entropy logits 0.5*N(0,1), k=V, p=0.95.
    B, V, seed = 512, 262144, 4
    rng = np.random.default_rng(seed)
    probs = np.empty((B, V), np.float32)
    step = 64
    for r0 in range(0, B, step):
        x = 0.5 * rng.standard_normal((step, V))
        probs[r0:r0 + step] = _rows_out(x, logits)
    top_k = np.full(B, V, np.int32)
    top_p = np.full(B, 0.95, np.float32)
    return Workload("specverify_b512_v262144", probs, top_k, top_p, seed, 0)


CONFIGS = {1: _cfg1, 2: _cfg2, 3: _cfg3, 4: _cfg4, 5: _cfg5}


def make(cfg: int) -> Workload:
    """Build config ``cfg`` (1..5)."""
    return CONFIGS[cfg]()


def make_logits(cfg: int) -> Workload:
    """Config ``cfg`` as fp32 logit rows: the same generator calls, stopped
    before the softmax, with the same top_k / top_p, plus a per-row
    temperature and min-p floor from a second generator seeded seed + 7919:
    temperature ~ U[0.5, 1.5], with 5% of rows at 0 (the greedy limit) and
    5% at exactly 1; min_p 0 on half the rows, else ~ U[0.005, 0.3]."""
    w = CONFIGS[cfg](logits=True)
    rng = np.random.default_rng(w.seed + 7919)
    B = w.B
    tau = rng.uniform(0.5, 1.5, size=B).astype(np.float32)
    pick = rng.random(B)
    tau[pick < 0.05] = 0.0
    tau[(pick >= 0.05) & (pick < 0.10)] = 1.0
    mp = rng.uniform(0.005, 0.3, size=B).astype(np.float32)
    mp[rng.random(B) < 0.5] = 0.0
    w.name = w.name + "_logits"
    w.temperature = tau
    w.min_p = mp
    return w


@dataclass
class SpecWorkload:
    name: str
    target: np.ndarray        # float32 [N * Lt][V] target probabilities
    top_k: np.ndarray         # int32 [N * Lt]
    top_p: np.ndarray         # float32 [N * Lt]
    draft: np.ndarray         # float32 [N * L][V] draft probabilities
    draft_tokens: np.ndarray  # int32 [N][L]
    Lt: int
    seed: int
    offset: int


def make_spec(cfg: int = 5, L: int = 7, sigma: float = 0.5) -> SpecWorkload:
    """Speculative-verification inputs on config ``cfg``'s rows: each request
    owns L + 1 consecutive target rows (its draft positions and the bonus
    position).  The draft distribution of position l is a perturbed copy of
    its target row, softmax(log p + sigma * N(0, 1)) in float64, cast to fp32,
    and the draft token is drawn from it; both from a generator seeded
    seed + 104729.  (Config 5, 512 rows, is 64 requests of 7 drafts.)"""
    w = CONFIGS[cfg]()
    Lt = L + 1
    N = w.B // Lt
    rng = np.random.default_rng(w.seed + 104729)
    V = w.V
    draft = np.empty((N * L, V), np.float32)
    toks = np.empty((N, L), np.int32)
    for n in range(N):
        lp = np.log(np.maximum(w.probs[n * Lt:n * Lt + L].astype(np.float64), 1e-300))
        q = softmax64(lp + sigma * rng.standard_normal((L, V)))
        draft[n * L:(n + 1) * L] = q.astype(np.float32)
        for l in range(L):
            toks[n, l] = rng.choice(V, p=q[l] / q[l].sum())
    rows = N * Lt
    return SpecWorkload("spec_%s_L%d" % (w.name, L), np.ascontiguousarray(w.probs[:rows]),
                        w.top_k[:rows].copy(), w.top_p[:rows].copy(), draft, toks, Lt, w.seed,
                        w.offset)


def sha256_of(w: Workload) -> str:
    h = hashlib.sha256()
    for a in (w.probs, w.top_k, w.top_p, w.temperature, w.min_p):
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    h.update(f"{w.seed}:{w.offset}".encode())
    return h.hexdigest()
