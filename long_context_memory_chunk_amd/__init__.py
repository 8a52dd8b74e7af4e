"""Python binding of the MSA C ABI (include/msa.h), argument marshalling only.

Every function here has the name of the C entry point it calls and does
nothing but turn torch tensors / numpy arrays into pointers and sizes, read
the current HIP stream, and raise MsaError on a non-zero status.  All
computation happens in the HIP kernels of libmsa.so.  There is no fallback:
if the library is missing, importing a function raises.

Build the library with ``python -m long_context_memory_chunk_amd.build``.
"""

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa.so")

MSA_OK, MSA_ERR_INVALID_ARG, MSA_ERR_UNSUPPORTED, MSA_ERR_HIP, MSA_ERR_WORKSPACE = range(5)
MSA_F32, MSA_BF16 = 0, 1
MSA_MAX_TOPK = 64

EXPORTS = [
    "msa_abi_version", "msa_last_error", "msa_status_string",
    "msa_ctx_create", "msa_ctx_destroy", "msa_chunk_offsets",
    "msa_encode_pool", "msa_encode_pool_bwd", "msa_route_workspace_size", "msa_route", "msa_route_time_next",
    "msa_route_bwd_workspace_size", "msa_route_bwd",
    "msa_gather", "msa_gather_device_workspace_size", "msa_gather_device",
    "msa_sparse_attn_workspace_size", "msa_sparse_attn", "msa_sparse_attn_noalloc",
    "msa_sparse_attn_lse", "msa_sparse_attn_bwd_workspace_size", "msa_sparse_attn_bwd",
    "msa_gather_attn_workspace_size", "msa_gather_attn",
]


class MsaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_STATUS = {0: "MSA_OK", 1: "MSA_ERR_INVALID_ARG", 2: "MSA_ERR_UNSUPPORTED", 3: "MSA_ERR_HIP",
           4: "MSA_ERR_WORKSPACE"}

_lib = None

P = ctypes.c_void_p
I32, I64, SZ, F32, F64 = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float, ctypes.c_double

_SIGS = {
    "msa_abi_version": (I32, []),
    "msa_last_error": (ctypes.c_char_p, []),
    "msa_status_string": (ctypes.c_char_p, [I32]),
    "msa_ctx_create": (I32, [I32, I32, F64, I32, ctypes.POINTER(P)]),
    "msa_ctx_destroy": (I32, [P]),
    "msa_chunk_offsets": (I32, [P, I64, I32, P, P]),
    "msa_encode_pool": (I32, [P, I32, P, P, P, P, P, I64, I64, I64, I32, I32, I64, P, P, P]),
    "msa_encode_pool_bwd": (I32, [P, I32, P, P, P, P, I64, I64, I64, I32, I32, I64, P, P, P, P]),
    "msa_route_workspace_size": (SZ, [I32, I64, I32, I32, I32, I64, I64, I32]),
    "msa_route": (I32, [P, I32, P, I64, I32, I32, P, I64, I32, P, I64, I32, P, P, P, P, P, SZ, P]),
    "msa_route_time_next": (I32, [P, P, P]),
    "msa_route_bwd_workspace_size": (SZ, [I64, I32, I32, I32, I64, I64]),
    "msa_route_bwd": (I32, [P, I32, P, I64, I32, I32, P, I64, I32, P, I64, P, P, P, P, P, SZ, P]),
    "msa_gather": (I32, [P, SZ, I64, P, I64, P, I64, I32, P, I64, P, P, P, P]),
    "msa_gather_device_workspace_size": (SZ, [I64, I32, I64]),
    "msa_gather_device": (I32, [P, P, SZ, I64, P, I64, P, I64, I32, P, I64, P, P, SZ, P]),
    "msa_sparse_attn_workspace_size": (SZ, [I32, I64, I32, I32, I32, I64, I32]),
    "msa_sparse_attn": (I32, [P, I32, P, I64, I32, I32, P, P, I64, I64, P, P, I32, I32, I32, F32, P,
                              P, SZ, P]),
    "msa_sparse_attn_noalloc": (I32, [P, I32, P, I64, I32, I32, P, P, I64, I64, P, P, I32, I32, I32, F32, P,
                                      P]),
    "msa_sparse_attn_lse": (I32, [P, I32, P, I64, I32, I32, P, P, I64, I64, P, P, I32, I32, I32, F32, P,
                                  P, P, SZ, P]),
    "msa_sparse_attn_bwd_workspace_size": (SZ, [I32, I64, I32, I32, I32, I64, I32]),
    "msa_sparse_attn_bwd": (I32, [P, I32, P, I64, I32, I32, P, P, I64, I64, P, P, I32, I32, I32, F32,
                                  P, P, P, P, P, P, P, P, SZ, P]),
    "msa_gather_attn_workspace_size": (SZ, [I32, I64, I32, I32, I32, I32, I64, I64, I32]),
    "msa_gather_attn": (I32, [P, I32, P, SZ, I64, P, I64, P, I32, P, I64, P, P, I64, I32, I32, I64, P, P,
                              I32, I32, I32, F32, P, P, SZ, P]),
}


def lib():
    """The loaded libmsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m long_context_memory_chunk_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _check(status):
    if status != MSA_OK:
        raise MsaError(status, lib().msa_last_error().decode())


def _ptr(x):
    """Device/host address of a torch tensor, numpy array, int or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        if not x.flags["C_CONTIGUOUS"]:
            raise ValueError("arrays must be C-contiguous")
        return x.ctypes.data
    if not x.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return x.data_ptr()


def _dtype(t):
    import torch
    if t.dtype == torch.bfloat16:
        return MSA_BF16
    if t.dtype == torch.float32:
        return MSA_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------- context

class Ctx:
    """Owns an msa_ctx*; destroyed by close() or garbage collection."""

    def __init__(self, handle, device, head_dim, rope_theta, max_pos):
        self.handle, self.device = handle, device
        self.head_dim, self.rope_theta, self.max_pos = head_dim, rope_theta, max_pos

    def close(self):
        if self.handle:
            _check(lib().msa_ctx_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def msa_abi_version():
    return lib().msa_abi_version()


def msa_last_error():
    return lib().msa_last_error().decode()


def msa_status_string(status):
    return lib().msa_status_string(status).decode()


def msa_ctx_create(device=0, head_dim=128, rope_theta=1e6, max_pos=16384):
    h = P()
    _check(lib().msa_ctx_create(device, head_dim, float(rope_theta), max_pos, ctypes.byref(h)))
    return Ctx(h.value, device, head_dim, rope_theta, max_pos)


def msa_ctx_destroy(ctx):
    ctx.close()


def msa_chunk_offsets(doc_tok_off, chunk_len, with_max_len=False):
    """Host helper: int64 numpy prefix sums of ceil(len / chunk_len); with
    with_max_len, also the longest document's length (msa_encode_pool's
    max_doc_len)."""
    tok = np.ascontiguousarray(doc_tok_off, dtype=np.int64)
    out = np.empty_like(tok)
    mx = ctypes.c_int64(0)
    _check(lib().msa_chunk_offsets(_ptr(tok), len(tok) - 1, chunk_len, _ptr(out), ctypes.addressof(mx)))
    return (out, mx.value) if with_max_len else out


# ---------------------------------------------------------------- stage 1

def msa_encode_pool(ctx, K, V, Kr, doc_tok_off, doc_chunk_off, KVbar, Krbar, chunk_len, max_doc_len,
                    stream=None):
    """K, V, Kr [T, Hkv, d]; offsets int64 device tensors [n_docs+1];
    KVbar [N, 2, Hkv, d], Krbar [N, Hkv, d] outputs; max_doc_len the longest
    document's token count (msa_chunk_offsets(..., with_max_len=True))."""
    T, Hkv, d = K.shape
    N = Krbar.shape[0]
    _check(lib().msa_encode_pool(ctx.handle, _dtype(K), _ptr(K), _ptr(V), _ptr(Kr), _ptr(doc_tok_off),
                                 _ptr(doc_chunk_off), doc_tok_off.numel() - 1, T, N, Hkv, chunk_len,
                                 int(max_doc_len), _ptr(KVbar), _ptr(Krbar), _stream(stream)))


def msa_encode_pool_bwd(ctx, dKVbar, dKrbar, doc_tok_off, doc_chunk_off, dK, dV, dKr, chunk_len, max_doc_len,
                        stream=None):
    """dKVbar [N, 2, Hkv, d], dKrbar [N, Hkv, d]; offsets int64 device [n_docs+1];
    dK, dV, dKr [T, Hkv, d] outputs; max_doc_len as for msa_encode_pool."""
    T, Hkv, d = dK.shape
    N = dKrbar.shape[0]
    _check(lib().msa_encode_pool_bwd(ctx.handle, _dtype(dK), _ptr(dKVbar), _ptr(dKrbar), _ptr(doc_tok_off),
                                     _ptr(doc_chunk_off), doc_tok_off.numel() - 1, T, N, Hkv, chunk_len,
                                     int(max_doc_len), _ptr(dK), _ptr(dV), _ptr(dKr), _stream(stream)))


# ---------------------------------------------------------------- stage 2

def msa_route_workspace_size(dtype, B, Tq, Hq, Hkv, N, n_docs, top_k):
    return lib().msa_route_workspace_size(dtype, B, Tq, Hq, Hkv, N, n_docs, top_k)


def msa_route(ctx, Qr, Krbar, doc_chunk_off, top_k, out_ids, workspace, out_scores=None,
              out_chunk=None, out_doc=None, stream=None):
    """Qr [B, Tq, Hq, d]; Krbar [N, Hkv, d]; doc_chunk_off int64 device [n_docs+1];
    out_ids int32 [B, top_k]; workspace uint8 device tensor."""
    B, Tq, Hq, d = Qr.shape
    N, Hkv, _ = Krbar.shape
    _check(lib().msa_route(ctx.handle, _dtype(Qr), _ptr(Qr), B, Tq, Hq, _ptr(Krbar), N, Hkv,
                           _ptr(doc_chunk_off), doc_chunk_off.numel() - 1, top_k, _ptr(out_ids),
                           _ptr(out_scores), _ptr(out_chunk), _ptr(out_doc), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(stream)))


def msa_route_time_next(ctx, start=None, stop=None):
    """start/stop: torch.cuda.Event(enable_timing=True) already recorded once
    (so the underlying event exists), or None to clear."""
    h = lambda e: None if e is None else e.cuda_event
    _check(lib().msa_route_time_next(ctx.handle, h(start), h(stop)))


def msa_route_bwd_workspace_size(B, Tq, Hq, Hkv, N, n_docs):
    return lib().msa_route_bwd_workspace_size(B, Tq, Hq, Hkv, N, n_docs)


def msa_route_bwd(ctx, Qr, Krbar, doc_chunk_off, dscore, dQr, dKrbar, workspace, out_arg=None, stream=None):
    """Qr [B, Tq, Hq, d]; Krbar [N, Hkv, d]; doc_chunk_off int64 device [n_docs+1];
    dscore float32 [B, n_docs]; dQr float32 like Qr; dKrbar float32 like Krbar;
    out_arg optional int32 [B, n_docs, 2]."""
    B, Tq, Hq, d = Qr.shape
    N, Hkv, _ = Krbar.shape
    _check(lib().msa_route_bwd(ctx.handle, _dtype(Qr), _ptr(Qr), B, Tq, Hq, _ptr(Krbar), N, Hkv,
                               _ptr(doc_chunk_off), doc_chunk_off.numel() - 1, _ptr(dscore), _ptr(dQr),
                               _ptr(dKrbar), _ptr(out_arg), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream)))


def msa_gather(host_KVbar, row_bytes, n_rows_host, doc_chunk_off_host, ids_host, top_k,
               dst_KVmem, cap_rows, mem_off_host, mem_off_dev=None, side=None, done=None):
    """host_KVbar: pinned host tensor (or address); doc_chunk_off_host int64
    numpy [n_docs+1]; ids_host int32 numpy/tensor [B, top_k] on the host;
    mem_off_host int64 host array [B+1] (written); mem_off_dev optional device
    int64 [B+1]; side: stream for the copies; done: raw hipEvent_t or None."""
    off = doc_chunk_off_host
    n_docs = (off.shape[0] if hasattr(off, "shape") else len(off)) - 1
    B = ids_host.shape[0]
    _check(lib().msa_gather(_ptr(host_KVbar), row_bytes, n_rows_host, _ptr(off), n_docs,
                            _ptr(ids_host), B, top_k, _ptr(dst_KVmem), cap_rows, _ptr(mem_off_host),
                            _ptr(mem_off_dev), _stream(side), done))


def msa_gather_device_workspace_size(B, top_k, cap_rows):
    return lib().msa_gather_device_workspace_size(B, top_k, cap_rows)


def msa_gather_device(ctx, host_KVbar, row_bytes, n_rows_host, doc_chunk_off, ids, dst_KVmem, cap_rows,
                      mem_off, workspace, stream=None):
    """host_KVbar: pinned host tensor or address; doc_chunk_off int64 device
    [n_docs+1]; ids int32 device [B, top_k]; mem_off int64 device [B+1]."""
    B, top_k = ids.shape
    _check(lib().msa_gather_device(ctx.handle, _ptr(host_KVbar), row_bytes, n_rows_host, _ptr(doc_chunk_off),
                                   doc_chunk_off.numel() - 1, _ptr(ids), B, top_k, _ptr(dst_KVmem), cap_rows,
                                   _ptr(mem_off), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)))


# ---------------------------------------------------------------- stage 3

def msa_sparse_attn_workspace_size(dtype, B, Tq, Hq, Hkv, max_rows_per_query, L):
    return lib().msa_sparse_attn_workspace_size(dtype, B, Tq, Hq, Hkv, max_rows_per_query, L)


def msa_sparse_attn(ctx, Q, KVmem, mem_off, max_rows_per_query, K_local, V_local, q_offset, scale,
                    O, workspace, stream=None):
    """Q [B, Tq, Hq, d]; KVmem [rows, 2, Hkv, d]; mem_off int64 device [B+1];
    K_local/V_local [B, L, Hkv, d]; O [B, Tq, Hq, d]."""
    B, Tq, Hq, d = Q.shape
    _, L, Hkv, _ = K_local.shape
    cap = KVmem.shape[0] if KVmem is not None else 0
    _check(lib().msa_sparse_attn(ctx.handle, _dtype(Q), _ptr(Q), B, Tq, Hq, _ptr(KVmem),
                                 _ptr(mem_off), cap, max_rows_per_query, _ptr(K_local),
                                 _ptr(V_local), L, Hkv, q_offset, float(scale), _ptr(O),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream)))


def msa_sparse_attn_noalloc(ctx, Q, KVmem, mem_off, max_rows_per_query, K_local, V_local, q_offset, scale,
                            O, stream=None):
    """msa_sparse_attn with the library's scratch array instead of a workspace
    (allocates nothing; see include/msa.h for the size limit)."""
    B, Tq, Hq, d = Q.shape
    _, L, Hkv, _ = K_local.shape
    cap = KVmem.shape[0] if KVmem is not None else 0
    _check(lib().msa_sparse_attn_noalloc(ctx.handle, _dtype(Q), _ptr(Q), B, Tq, Hq, _ptr(KVmem),
                                         _ptr(mem_off), cap, max_rows_per_query, _ptr(K_local),
                                         _ptr(V_local), L, Hkv, q_offset, float(scale), _ptr(O),
                                         _stream(stream)))


def msa_sparse_attn_lse(ctx, Q, KVmem, mem_off, max_rows_per_query, K_local, V_local, q_offset, scale,
                        O, lse, workspace, stream=None):
    """msa_sparse_attn plus lse float32 [B, Tq, Hq] (the saved row statistic)."""
    B, Tq, Hq, d = Q.shape
    _, L, Hkv, _ = K_local.shape
    cap = KVmem.shape[0] if KVmem is not None else 0
    _check(lib().msa_sparse_attn_lse(ctx.handle, _dtype(Q), _ptr(Q), B, Tq, Hq, _ptr(KVmem),
                                     _ptr(mem_off), cap, max_rows_per_query, _ptr(K_local),
                                     _ptr(V_local), L, Hkv, q_offset, float(scale), _ptr(O), _ptr(lse),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream)))


def msa_sparse_attn_bwd_workspace_size(dtype, B, Tq, Hq, Hkv, max_rows_per_query, L):
    return lib().msa_sparse_attn_bwd_workspace_size(dtype, B, Tq, Hq, Hkv, max_rows_per_query, L)


def msa_sparse_attn_bwd(ctx, Q, KVmem, mem_off, max_rows_per_query, K_local, V_local, q_offset, scale,
                        O, dO, lse, dQ, dKVmem, dK_local, dV_local, workspace, stream=None):
    """Gradients: dQ like Q, dKVmem like KVmem, dK_local/dV_local like K_local."""
    B, Tq, Hq, d = Q.shape
    _, L, Hkv, _ = K_local.shape
    cap = KVmem.shape[0] if KVmem is not None else 0
    _check(lib().msa_sparse_attn_bwd(ctx.handle, _dtype(Q), _ptr(Q), B, Tq, Hq, _ptr(KVmem),
                                     _ptr(mem_off), cap, max_rows_per_query, _ptr(K_local),
                                     _ptr(V_local), L, Hkv, q_offset, float(scale), _ptr(O), _ptr(dO),
                                     _ptr(lse), _ptr(dQ), _ptr(dKVmem), _ptr(dK_local), _ptr(dV_local),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream)))


def workspace(nbytes, device="cuda"):
    """A device byte buffer (torch allocations are 512-byte aligned)."""
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- stages 2b + 3

def msa_gather_attn_workspace_size(dtype, B, Tq, Hq, Hkv, top_k, cap_rows, max_rows_per_query, L):
    return lib().msa_gather_attn_workspace_size(dtype, B, Tq, Hq, Hkv, top_k, cap_rows, max_rows_per_query, L)


def msa_gather_attn(ctx, host_KVbar, row_bytes, n_rows_host, doc_chunk_off, ids, dst_KVmem, cap_rows, mem_off,
                    Q, max_rows_per_query, K_local, V_local, q_offset, scale, O, workspace, stream=None):
    """msa_gather_device then msa_sparse_attn over the gathered rows, in one
    call: host_KVbar pinned host tensor or address; doc_chunk_off int64 device
    [n_docs+1]; ids int32 device [B, top_k]; dst_KVmem [cap_rows, 2, Hkv, d];
    mem_off int64 device [B+1]; Q [B, Tq, Hq, d]; K_local/V_local
    [B, L, Hkv, d]; O [B, Tq, Hq, d]."""
    B, top_k = ids.shape
    _, Tq, Hq, _ = Q.shape
    _, L, Hkv, _ = K_local.shape
    _check(lib().msa_gather_attn(ctx.handle, _dtype(Q), _ptr(host_KVbar), row_bytes, n_rows_host,
                                 _ptr(doc_chunk_off), doc_chunk_off.numel() - 1, _ptr(ids), top_k, _ptr(dst_KVmem),
                                 cap_rows, _ptr(mem_off), _ptr(Q), B, Tq, Hq, max_rows_per_query, _ptr(K_local),
                                 _ptr(V_local), L, Hkv, q_offset, float(scale), _ptr(O), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))
