"""ctypes binding of the device fill kernel and the streaming-read probe
(msa_synth/libmsasynth.so)."""

import ctypes
import os

_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsasynth.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError(f"{_LIB} is missing: build it with "
                               "`python -m long_context_memory_chunk_amd.build`")
        l = ctypes.CDLL(_LIB)
        l.msa_synth_fill_counter_bf16.restype = ctypes.c_int
        l.msa_synth_fill_counter_bf16.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                                  ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p]
        l.msa_synth_stream_key.restype = ctypes.c_uint64
        l.msa_synth_stream_key.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        l.msa_synth_read_probe.restype = ctypes.c_int
        l.msa_synth_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                           ctypes.c_void_p]
        _lib = l
    return _lib


def fill_counter_bf16(dst, seed, stream, start, count=None, hip_stream=None):
    """Fill a bf16 tensor (device, or pinned host given as (address, count))
    with counter-generator elements start .. start+count-1 of `stream`."""
    import torch
    if isinstance(dst, tuple):
        addr, n = dst
    else:
        addr, n = dst.data_ptr(), dst.numel()
    count = n if count is None else count
    hs = torch.cuda.current_stream().cuda_stream if hip_stream is None else hip_stream
    rc = lib().msa_synth_fill_counter_bf16(addr, seed, stream, start, count, hs)
    if rc != 0:
        raise RuntimeError(f"msa_synth_fill_counter_bf16 failed with HIP error {rc}")


def stream_key(seed, stream):
    return int(lib().msa_synth_stream_key(seed, stream))


def read_probe(src, sink, blocks, hip_stream=None):
    """Stream every byte of the device tensor `src` once (non-temporal 16-byte
    loads); sink: an int32 device tensor of at least blocks * 256 elements."""
    import torch
    nbytes = src.numel() * src.element_size()
    if sink.numel() < blocks * 256:
        raise ValueError("sink too small")
    hs = torch.cuda.current_stream().cuda_stream if hip_stream is None else hip_stream
    rc = lib().msa_synth_read_probe(src.data_ptr(), nbytes, sink.data_ptr(), blocks, hs)
    if rc != 0:
        raise RuntimeError(f"msa_synth_read_probe failed with HIP error {rc}")
