"""Python binding of the MI355X exact top-k -> top-p sampler (C ABI in
``include/tes_sampler.h``).

The functions below carry the C names and only marshal arguments: every step
of the sampling path runs in the HIP kernels of ``libtes_sampler.so``.  The
library must have been built (``top_exact_sampling_amd.build.build()``); if
it is missing, loading fails with an error instead of falling back to
anything else.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtes_sampler.so")

TES_OK = 0
TES_ERR_INVALID_ARGUMENT = -1
TES_ERR_NO_DEVICE = -2
TES_ERR_UNSUPPORTED_DEVICE = -3
TES_ERR_OUT_OF_MEMORY = -4
TES_ERR_LAUNCH = -5
TES_ERR_TOO_LARGE = -6

TES_FLAG_NONE = 0
TES_FLAG_FORCE_ROW_SELECT = 1
TES_FLAG_TINY_BUFFER = 2
TES_FLAG_STATS = 4
TES_FLAG_SMALL_SEGMENTS = 8
TES_FLAG_NO_WAIT = 16
TES_FLAG_ROW_TOPP = 32

STAT_WORDS = 16  # uint32 per row returned by sampler_get_stats

EXPORTED = ("sampler_create", "topk_topp_sample", "sampler_destroy", "sampler_status_string",
            "sampler_get_stats", "sampler_read_probe", "topk_topp_sample_slab", "sampler_route",
            "topk_topp_sample_bf16", "topk_topp_sample_noalloc", "topk_topp_sample_logits",
            "spec_verify_sample")

_lib = None


class TesError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s failed: %s (%d)" % (what, sampler_status_string(status), status))
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libtes_sampler.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libtes_sampler.so is not built; run "
                              "top_exact_sampling_amd.build.build() first")
        L = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        L.sampler_create.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_uint]
        L.sampler_create.restype = ctypes.c_int
        L.topk_topp_sample.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, vp, vp,
                                       ctypes.c_uint64, ctypes.c_uint64, vp, vp, vp]
        L.topk_topp_sample.restype = ctypes.c_int
        L.topk_topp_sample_bf16.argtypes = L.topk_topp_sample.argtypes
        L.topk_topp_sample_bf16.restype = ctypes.c_int
        L.topk_topp_sample_noalloc.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, vp,
                                               ctypes.c_uint64, ctypes.c_uint64, vp, vp, vp]
        L.topk_topp_sample_noalloc.restype = ctypes.c_int
        L.topk_topp_sample_logits.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp,
                                              ctypes.c_uint64, ctypes.c_uint64, vp, vp, vp]
        L.topk_topp_sample_logits.restype = ctypes.c_int
        L.spec_verify_sample.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp,
                                         vp, ctypes.c_int, vp, vp, ctypes.c_uint64,
                                         ctypes.c_uint64, vp, vp, vp]
        L.spec_verify_sample.restype = ctypes.c_int
        L.sampler_destroy.argtypes = [vp]
        L.sampler_destroy.restype = ctypes.c_int
        L.sampler_status_string.argtypes = [ctypes.c_int]
        L.sampler_status_string.restype = ctypes.c_char_p
        L.sampler_get_stats.argtypes = [vp, vp, ctypes.c_int]
        L.sampler_get_stats.restype = ctypes.c_int
        L.sampler_read_probe.argtypes = [vp, ctypes.c_uint64, vp, ctypes.c_int, vp]
        L.sampler_read_probe.restype = ctypes.c_int
        L.topk_topp_sample_slab.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, vp, vp,
                                            ctypes.c_uint64, ctypes.c_uint64, vp, vp, vp, vp,
                                            ctypes.c_int, vp, vp, vp]
        L.topk_topp_sample_slab.restype = ctypes.c_int
        L.sampler_route.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, vp]
        L.sampler_route.restype = ctypes.c_int
        _lib = L
    return _lib


# -- C names ----------------------------------------------------------------
def sampler_status_string(status: int) -> str:
    return lib().sampler_status_string(int(status)).decode()


def sampler_create(device: int, max_batch: int, max_vocab: int, flags: int = 0) -> int:
    h = ctypes.c_void_p()
    rc = lib().sampler_create(ctypes.byref(h), int(device), int(max_batch), int(max_vocab),
                              int(flags))
    if rc != TES_OK:
        raise TesError(rc, "sampler_create")
    return h.value


def topk_topp_sample(handle, probs_ptr: int, B: int, V: int, top_k_ptr: int, top_p_ptr: int,
                     seed: int, offset: int, out_tokens_ptr: int, renorm_ptr, stream) -> int:
    """Raw call with device pointers (ints); returns the status code."""
    return lib().topk_topp_sample(handle, probs_ptr, int(B), int(V), top_k_ptr, top_p_ptr,
                                  int(seed) & (2**64 - 1), int(offset) & (2**64 - 1),
                                  out_tokens_ptr, renorm_ptr, stream)


def topk_topp_sample_bf16(handle, probs_ptr: int, B: int, V: int, top_k_ptr: int,
                          top_p_ptr: int, seed: int, offset: int, out_tokens_ptr: int, renorm_ptr,
                          stream) -> int:
    """Raw call over bf16 rows with device pointers (ints); returns the status."""
    return lib().topk_topp_sample_bf16(handle, probs_ptr, int(B), int(V), top_k_ptr, top_p_ptr,
                                       int(seed) & (2**64 - 1), int(offset) & (2**64 - 1),
                                       out_tokens_ptr, renorm_ptr, stream)


def topk_topp_sample_noalloc(probs_ptr: int, B: int, V: int, top_k_ptr: int, top_p_ptr: int,
                             seed: int, offset: int, out_tokens_ptr: int, renorm_ptr,
                             stream) -> int:
    """Raw call of the allocation-free entry point (no handle; the current
    device), with device pointers (ints); returns the status code."""
    return lib().topk_topp_sample_noalloc(probs_ptr, int(B), int(V), top_k_ptr, top_p_ptr,
                                          int(seed) & (2**64 - 1), int(offset) & (2**64 - 1),
                                          out_tokens_ptr, renorm_ptr, stream)


def topk_topp_sample_logits(handle, logits_ptr: int, B: int, V: int, top_k_ptr: int,
                            top_p_ptr: int, temperature_ptr, min_p_ptr, seed: int, offset: int,
                            out_tokens_ptr: int, renorm_ptr, stream) -> int:
    """Raw call over fp32 logit rows with device pointers (ints; temperature,
    min_p and renorm may be None); returns the status code."""
    return lib().topk_topp_sample_logits(handle, logits_ptr, int(B), int(V), top_k_ptr, top_p_ptr,
                                         temperature_ptr, min_p_ptr, int(seed) & (2**64 - 1),
                                         int(offset) & (2**64 - 1), out_tokens_ptr, renorm_ptr,
                                         stream)


def spec_verify_sample(handle, target_ptr: int, N: int, Lt: int, V: int, top_k_ptr: int,
                       top_p_ptr: int, draft_ptr, L: int, draft_tokens_ptr, target_map_ptr,
                       seed: int, offset: int, out_tokens_ptr: int, accept_len_ptr: int,
                       stream) -> int:
    """Raw speculative-verification call with device pointers (ints; the
    target map may be None); returns the status code."""
    return lib().spec_verify_sample(handle, target_ptr, int(N), int(Lt), int(V), top_k_ptr,
                                    top_p_ptr, draft_ptr, int(L), draft_tokens_ptr,
                                    target_map_ptr, int(seed) & (2**64 - 1),
                                    int(offset) & (2**64 - 1), out_tokens_ptr, accept_len_ptr,
                                    stream)


def sampler_destroy(handle) -> int:
    return lib().sampler_destroy(handle)


def sampler_get_stats(handle, B: int):
    import numpy as np

    out = np.zeros((B, STAT_WORDS), np.uint32)
    rc = lib().sampler_get_stats(handle, out.ctypes.data, int(B))
    if rc != TES_OK:
        raise TesError(rc, "sampler_get_stats")
    return out


def topk_topp_sample_slab(handle, probs_ptr: int, B: int, V: int, top_k_ptr: int, top_p_ptr: int,
                          seed: int, offset: int, out_tokens_ptr: int, renorm_ptr, slab_index_ptr: int,
                          slab_renorm_ptr: int, slab_cap: int, slab_len_ptr: int, route_ptr,
                          stream) -> int:
    """Raw call with device pointers (ints); returns the status code."""
    return lib().topk_topp_sample_slab(handle, probs_ptr, int(B), int(V), top_k_ptr, top_p_ptr,
                                       int(seed) & (2**64 - 1), int(offset) & (2**64 - 1),
                                       out_tokens_ptr, renorm_ptr, slab_index_ptr,
                                       slab_renorm_ptr, int(slab_cap), slab_len_ptr, route_ptr,
                                       stream)


def sampler_route(handle, V: int, top_k_host):
    """Per-row path codes from host top_k, without launching anything."""
    import numpy as np

    k = np.ascontiguousarray(top_k_host, dtype=np.int32)
    out = np.zeros(k.size, np.uint32)
    rc = lib().sampler_route(handle, int(k.size), int(V), k.ctypes.data, out.ctypes.data)
    if rc != TES_OK:
        raise TesError(rc, "sampler_route")
    return out


def sampler_read_probe(data_ptr: int, nbytes: int, sink_ptr: int, device: int, stream) -> int:
    """Plain read of nbytes of device memory (reference timing); status code."""
    return lib().sampler_read_probe(data_ptr, int(nbytes), sink_ptr, int(device), stream)


# -- torch convenience (marshalling only) -----------------------------------
class Sampler:
    """Owns one sampler handle; ``sample`` passes torch tensors through."""

    def __init__(self, device: int = 0, max_batch: int = 1024, max_vocab: int = 262144,
                 flags: int = 0):
        self.device = device
        self.handle = sampler_create(device, max_batch, max_vocab, flags)

    def close(self):
        if self.handle:
            sampler_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def sample(self, probs, top_k, top_p, seed: int, offset: int, out_tokens=None,
               renorm_out=None, stream=None):
        import torch

        B, V = probs.shape
        # fp32 rows, or bf16 rows (topk_topp_sample_bf16).
        bf16 = probs.dtype == torch.bfloat16
        pdt = torch.bfloat16 if bf16 else torch.float32
        for t, dt in ((probs, pdt), (top_k, torch.int32), (top_p, torch.float32)):
            if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
                raise ValueError("expected contiguous %s on the GPU" % dt)
        if out_tokens is None:
            out_tokens = torch.empty(B, dtype=torch.int32, device=probs.device)
        if stream is None:
            stream = torch.cuda.current_stream(probs.device)
        fn = topk_topp_sample_bf16 if bf16 else topk_topp_sample
        rc = fn(self.handle, probs.data_ptr(), B, V, top_k.data_ptr(), top_p.data_ptr(), seed,
                offset, out_tokens.data_ptr(),
                renorm_out.data_ptr() if renorm_out is not None else None, stream.cuda_stream)
        if rc != TES_OK:
            raise TesError(rc, fn.__name__)
        return out_tokens

    def sample_logits(self, logits, top_k, top_p, seed: int, offset: int, temperature=None,
                      min_p=None, out_tokens=None, renorm_out=None, stream=None):
        """Sample fp32 logit rows (topk_topp_sample_logits); temperature and
        min_p are per-row fp32 tensors or None."""
        import torch

        B, V = logits.shape
        checks = [(logits, torch.float32), (top_k, torch.int32), (top_p, torch.float32)]
        for t in (temperature, min_p):
            if t is not None:
                checks.append((t, torch.float32))
        for t, dt in checks:
            if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
                raise ValueError("expected contiguous %s on the GPU" % dt)
        if out_tokens is None:
            out_tokens = torch.empty(B, dtype=torch.int32, device=logits.device)
        if stream is None:
            stream = torch.cuda.current_stream(logits.device)
        rc = topk_topp_sample_logits(
            self.handle, logits.data_ptr(), B, V, top_k.data_ptr(), top_p.data_ptr(),
            temperature.data_ptr() if temperature is not None else None,
            min_p.data_ptr() if min_p is not None else None, seed, offset, out_tokens.data_ptr(),
            renorm_out.data_ptr() if renorm_out is not None else None, stream.cuda_stream)
        if rc != TES_OK:
            raise TesError(rc, "topk_topp_sample_logits")
        return out_tokens

    def spec_verify(self, target, Lt: int, top_k, top_p, draft, draft_tokens, seed: int,
                    offset: int, target_map=None, stream=None):
        """Speculative verification (spec_verify_sample): target [N*Lt][V] fp32,
        draft [N*L][V] fp32, draft_tokens [N][L] int32, target_map [N][L+1]
        int32 or None.  Returns (out_tokens [N][L+1], accept_len [N])."""
        import torch

        V = target.shape[-1]
        N = target.shape[0] // Lt
        L = draft_tokens.shape[1]
        checks = [(target, torch.float32), (top_k, torch.int32), (top_p, torch.float32),
                  (draft, torch.float32), (draft_tokens, torch.int32)]
        if target_map is not None:
            checks.append((target_map, torch.int32))
        for t, dt in checks:
            if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
                raise ValueError("expected contiguous %s on the GPU" % dt)
        dev = target.device
        out = torch.empty((N, L + 1), dtype=torch.int32, device=dev)
        acc = torch.empty(N, dtype=torch.int32, device=dev)
        if stream is None:
            stream = torch.cuda.current_stream(dev)
        rc = spec_verify_sample(self.handle, target.data_ptr(), N, Lt, V, top_k.data_ptr(),
                                top_p.data_ptr(), draft.data_ptr() if L else None, L,
                                draft_tokens.data_ptr() if L else None,
                                target_map.data_ptr() if target_map is not None else None,
                                seed, offset, out.data_ptr(), acc.data_ptr(), stream.cuda_stream)
        if rc != TES_OK:
            raise TesError(rc, "spec_verify_sample")
        return out, acc

    def sample_slab(self, probs, top_k, top_p, seed: int, offset: int, slab_cap: int,
                    out_tokens=None, renorm_out=None, stream=None, want_route: bool = True):
        """Sample and export each row's sorted support (see topk_topp_sample_slab);
        returns (tokens, slab_index, slab_renorm, slab_len, route or None)."""
        import torch

        B, V = probs.shape
        for t, dt in ((probs, torch.float32), (top_k, torch.int32), (top_p, torch.float32)):
            if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
                raise ValueError("expected contiguous %s on the GPU" % dt)
        dev = probs.device
        if out_tokens is None:
            out_tokens = torch.empty(B, dtype=torch.int32, device=dev)
        si = torch.empty((B, slab_cap), dtype=torch.int32, device=dev)
        sr = torch.empty((B, slab_cap), dtype=torch.float32, device=dev)
        sl = torch.empty(B, dtype=torch.int32, device=dev)
        rt = torch.empty(B, dtype=torch.int32, device=dev) if want_route else None
        if stream is None:
            stream = torch.cuda.current_stream(dev)
        rc = topk_topp_sample_slab(self.handle, probs.data_ptr(), B, V, top_k.data_ptr(),
                                   top_p.data_ptr(), seed, offset, out_tokens.data_ptr(),
                                   renorm_out.data_ptr() if renorm_out is not None else None,
                                   si.data_ptr(), sr.data_ptr(), slab_cap, sl.data_ptr(),
                                   rt.data_ptr() if rt is not None else None, stream.cuda_stream)
        if rc != TES_OK:
            raise TesError(rc, "topk_topp_sample_slab")
        return out_tokens, si, sr, sl, rt

    def route(self, V: int, top_k_host):
        return sampler_route(self.handle, V, top_k_host)

    def stats(self, B: int):
        return sampler_get_stats(self.handle, B)
