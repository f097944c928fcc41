"""C-ABI checks that need no GPU: the library loads, exports every symbol
declared in include/tes_sampler.h, and rejects bad arguments on the host."""

import os
import re
import subprocess

import pytest

import top_exact_sampling_amd as tes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tes_sampler.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("sampler_create", "topk_topp_sample", "sampler_destroy"):
        assert n in names
    assert set(names) == set(tes.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", tes.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    for n in declared_functions():
        assert n in exported, n
    lib = tes.lib()
    for n in declared_functions():
        assert hasattr(lib, n)


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert tes.sampler_status_string(code) != "unknown status"
    assert tes.sampler_status_string(12345) == "unknown status"


def test_host_side_argument_validation():
    # None of these reach the device.
    assert tes.topk_topp_sample(None, 0, 1, 10, 0, 0, 0, 0, 0, None, None) == \
        tes.TES_ERR_INVALID_ARGUMENT
    assert tes.topk_topp_sample_bf16(None, 0, 1, 16, 0, 0, 0, 0, 0, None, None) == \
        tes.TES_ERR_INVALID_ARGUMENT
    with pytest.raises(tes.TesError) as e:
        tes.sampler_create(0, 0, 10)
    assert e.value.status == tes.TES_ERR_INVALID_ARGUMENT
    with pytest.raises(tes.TesError) as e:
        tes.sampler_create(0, 4, 2**31 - 1)
    assert e.value.status == tes.TES_ERR_INVALID_ARGUMENT
    with pytest.raises(tes.TesError) as e:
        tes.sampler_create(0, 4, 100, flags=1 << 20)
    assert e.value.status == tes.TES_ERR_INVALID_ARGUMENT
    assert tes.sampler_destroy(None) == tes.TES_OK
    # Slab export: no handle, or a capacity out of range.
    assert tes.topk_topp_sample_slab(None, 0, 1, 10, 0, 0, 0, 0, 0, None, 16, 16, 8, 16, None,
                                     None) == tes.TES_ERR_INVALID_ARGUMENT
    assert tes.lib().sampler_route(None, 1, 10, None, None) == tes.TES_ERR_INVALID_ARGUMENT
    # Reference read: null, misaligned or ragged buffers.
    assert tes.sampler_read_probe(0, 16, 64, 0, None) == tes.TES_ERR_INVALID_ARGUMENT
    assert tes.sampler_read_probe(8, 16, 64, 0, None) == tes.TES_ERR_INVALID_ARGUMENT
    assert tes.sampler_read_probe(16, 20, 64, 0, None) == tes.TES_ERR_INVALID_ARGUMENT
    assert tes.sampler_read_probe(16, 16, 0, 0, None) == tes.TES_ERR_INVALID_ARGUMENT
    assert tes.sampler_read_probe(16, 16, 64, -1, None) == tes.TES_ERR_INVALID_ARGUMENT


def test_create_without_gpu_reports_no_device():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(tes.TesError) as e:
        tes.sampler_create(0, 4, 1000)
    assert e.value.status == tes.TES_ERR_NO_DEVICE
