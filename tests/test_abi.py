"""The C-ABI library loads and exports every symbol include/msa.h declares;
host-side validation that returns before any HIP call (no GPU needed)."""

import ctypes
import os
import re

import numpy as np
import pytest

import long_context_memory_chunk_amd as msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "msa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(msa.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(msa.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_synth_library_exports():
    lib = ctypes.CDLL(os.path.join(ROOT, "msa_synth", "libmsasynth.so"))
    assert hasattr(lib, "msa_synth_fill_counter_bf16") and hasattr(lib, "msa_synth_stream_key")


def test_abi_version_and_status_strings():
    assert msa.msa_abi_version() == 2
    assert msa.msa_status_string(0) == "MSA_OK"
    assert msa.msa_status_string(4) == "MSA_ERR_WORKSPACE"
    assert msa.msa_status_string(99) == "MSA_STATUS_UNKNOWN"


def test_synth_stream_key_matches_numpy():
    import msa_synth
    from msa_synth import device
    for seed, stream in [(0, 0), (7, 3), (2**40 + 5, 123456789)]:
        assert device.stream_key(seed, stream) == msa_synth.splitmix64_key(seed, stream)


def test_chunk_offsets_host_helper():
    tok = np.array([0, 5, 7, 14, 78, 143], dtype=np.int64)
    assert msa.msa_chunk_offsets(tok, 2).tolist() == [0, 3, 4, 8, 40, 73]
    assert msa.msa_chunk_offsets(tok, 64).tolist() == [0, 1, 2, 3, 4, 6]
    off, longest = msa.msa_chunk_offsets(tok, 64, with_max_len=True)
    assert off.tolist() == [0, 1, 2, 3, 4, 6] and longest == 65      # lengths 5, 2, 7, 64, 65


def test_chunk_offsets_rejects_empty_document_and_bad_chunk():
    with pytest.raises(msa.MsaError) as e:
        msa.msa_chunk_offsets(np.array([0, 3, 3, 5], dtype=np.int64), 2)
    assert e.value.status == msa.MSA_ERR_INVALID_ARG and "no token" in str(e.value)
    with pytest.raises(msa.MsaError) as e:
        msa.msa_chunk_offsets(np.array([0, 3], dtype=np.int64), 0)
    assert e.value.status == msa.MSA_ERR_INVALID_ARG


def test_ctx_create_rejects_unsupported_head_dim_before_touching_hip():
    for d in (32, 96, 256):
        with pytest.raises(msa.MsaError) as e:
            msa.msa_ctx_create(0, d, 1e6, 1024)
        assert e.value.status == msa.MSA_ERR_UNSUPPORTED
    with pytest.raises(msa.MsaError) as e:
        msa.msa_ctx_create(0, 128, 0.5, 1024)
    assert e.value.status == msa.MSA_ERR_INVALID_ARG
    with pytest.raises(msa.MsaError) as e:
        msa.msa_ctx_create(0, 128, 1e6, 0)
    assert e.value.status == msa.MSA_ERR_INVALID_ARG


def test_hip_runtime_failure_maps_to_msa_err_hip():
    """With no GPU visible the HIP runtime itself fails (hipGetDeviceCount):
    the call returns MSA_ERR_HIP with the failing call and HIP's error named,
    and no exception crosses the ABI.  On a machine with a GPU the same
    context is created; the test needs the GPU-less case."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: the HIP runtime does not fail here")
    with pytest.raises(msa.MsaError) as e:
        msa.msa_ctx_create(0, 128, 1e6, 1024)
    assert e.value.status == msa.MSA_ERR_HIP
    assert "hipGetDeviceCount" in str(e.value)


def test_calls_without_context_fail_cleanly():
    L = msa.lib()
    assert L.msa_encode_pool(None, 1, *([None] * 5), 1, 1, 1, 1, 1, 1, None, None, None) == 1
    assert L.msa_route(None, 1, None, 1, 1, 1, None, 1, 1, None, 1, 1, None, None, None, None,
                       None, 0, None) == 1
    assert "ctx is NULL" in msa.msa_last_error()
    assert L.msa_sparse_attn(None, 1, None, 1, 1, 1, None, None, 0, 0, None, None, 1, 1, 0, 1.0,
                             None, None, 0, None) == 1


def test_gather_rejects_null_and_bad_sizes_before_hip():
    L = msa.lib()
    off = np.array([0, 2, 4], dtype=np.int64)
    ids = np.array([[0]], dtype=np.int32)
    mo = np.zeros(2, dtype=np.int64)
    assert L.msa_gather(None, 64, 4, off.ctypes.data, 2, ids.ctypes.data, 1, 1, 1, 8,
                        mo.ctypes.data, None, None, None) == 1
    assert L.msa_gather(1, 64, 4, off.ctypes.data, 2, ids.ctypes.data, 1, 3, 1, 8,
                        mo.ctypes.data, None, None, None) == 1    # top_k > n_docs
    assert L.msa_gather(1, 0, 4, off.ctypes.data, 2, ids.ctypes.data, 1, 1, 1, 8,
                        mo.ctypes.data, None, None, None) == 1    # row_bytes 0


def test_gather_rejects_pageable_host_store():
    L = msa.lib()
    host = np.zeros(4 * 64, dtype=np.uint8)
    off = np.array([0, 2, 4], dtype=np.int64)
    ids = np.array([[1]], dtype=np.int32)
    mo = np.zeros(2, dtype=np.int64)
    rc = L.msa_gather(host.ctypes.data, 64, 4, off.ctypes.data, 2, ids.ctypes.data, 1, 1, 1, 8,
                      mo.ctypes.data, None, None, None)
    assert rc == msa.MSA_ERR_INVALID_ARG and "pinned" in msa.msa_last_error()


def test_library_loads_next_to_torchs_hip_runtime():
    """torch brings its own libamdhip64; libmsa.so must not need a HIP
    symbol that runtime lacks (optional newer calls are looked up at run time)."""
    import subprocess
    import sys
    code = ("import torch, ctypes; ctypes.CDLL(%r); print('loaded')" % msa.LIB_PATH)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "loaded" in r.stdout, r.stderr[-2000:]


def test_gather_device_validates_before_launch():
    L = msa.lib()
    assert L.msa_gather_device(None, 1, 64, 4, 1, 2, 1, 1, 1, 1, 8, 1, 1, 256, None) == 1   # ctx NULL
    assert msa.msa_gather_device_workspace_size(0, 4, 100) == 0
    assert msa.msa_gather_device_workspace_size(3, 16, 1000) >= 3 * 64 * 3 * 8 + 1000 * 8
