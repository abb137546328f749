"""Thin ctypes binding of libhierasparse.so (C ABI: include/hierasparse.h).

Argument marshalling only: every function forwards to the C entry point of the same name, passing
torch device tensors as raw pointers and the current torch stream as the HIP stream. Every step of
the compute path runs in the library's HIP kernels. If the library is missing the first call
raises; there is no fallback.
"""
import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhierasparse.so")

HS_OK, HS_ERR_NULL, HS_ERR_SHAPE, HS_ERR_COUNTS, HS_ERR_ALIGN = 0, 1, 2, 3, 4
HS_ERR_WORKSPACE, HS_ERR_UNSUPPORTED, HS_ERR_HIP, HS_ERR_OVERLAP = 5, 6, 7, 8
HS_OP_COMPRESS, HS_OP_DECODE, HS_OP_RECOMPRESS = 1, 2, 3
HS_BF16, HS_F16 = 0, 1
HS_PREFILL_SMFMAC, HS_PREFILL_DECOMPRESS = 0, 1
# Prefill variants of hs_prefill_attn_variant (one optimisation of the SMFMAC prefill left out).
(HS_PREFILL_VARIANT_NONE, HS_PREFILL_VARIANT_SYNC_LOADS, HS_PREFILL_VARIANT_NO_ALIAS,
 HS_PREFILL_VARIANT_GENERIC_WALK, HS_PREFILL_VARIANT_LOCKSTEP,
 HS_PREFILL_VARIANT_LDS_RELAYOUT) = 0, 1, 2, 4, 8, 16

EXPORTS = ("hs_cache_sizes", "hs_workspace_size", "hs_compress", "hs_compress_ex",
           "hs_compress_masked", "hs_recompress", "hs_decode_attn", "hs_decode_attn_noalloc",
           "hs_prefill_attn", "hs_prefill_attn_variant", "hs_status_string", "hs_last_error")

# Bytes of the device array hs_decode_attn_noalloc uses (HS_DECODE_NOALLOC_SCRATCH_BYTES).
HS_DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20

CACHE_FIELDS = ("map_k", "map_v", "k_dense", "k_nnz", "k_meta", "v_dense", "v_nnz", "v_meta")


class HsShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "q_heads", "kv_heads", "seq_len", "head_dim", "block", "dtype")]


class HsCounts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_pruned", "n_sparse_k", "n_sparse_v")]


class HsCache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in CACHE_FIELDS]


class HsCacheBytes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in CACHE_FIELDS]


class HsPolicy(ctypes.Structure):
    _fields_ = [("sink_tokens", ctypes.c_int32), ("local_tokens", ctypes.c_int32)]


class HsError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{hs_status_string(status)}: {detail}")
        self.status = status


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libhierasparse.so is not built ({LIB_PATH}); run "
                               "python -m sparse_kv_cache_magnitude_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, S = ctypes.c_void_p, ctypes.POINTER
        L.hs_cache_sizes.argtypes = [S(HsShape), S(HsCounts), S(HsCacheBytes)]
        L.hs_workspace_size.argtypes = [ctypes.c_int, S(HsShape), S(HsCounts), ctypes.c_int32,
                                        S(ctypes.c_size_t)]
        L.hs_compress.argtypes = [S(HsShape), S(HsCounts), P, P, S(HsCache), P, ctypes.c_size_t, P]
        L.hs_compress_ex.argtypes = [S(HsShape), S(HsCounts), S(HsPolicy), P, P, S(HsCache), P,
                                     ctypes.c_size_t, P]
        L.hs_compress_masked.argtypes = [S(HsShape), S(HsCounts), P, P, P, P, S(HsCache), P, P]
        L.hs_recompress.argtypes = [S(HsShape), S(HsCounts), S(HsCache), S(HsCounts), S(HsCache),
                                    P, ctypes.c_size_t, P]
        L.hs_decode_attn.argtypes = [S(HsShape), S(HsCounts), S(HsCache), P, P, P, ctypes.c_float,
                                     ctypes.c_int32, P, ctypes.c_size_t, P]
        L.hs_decode_attn_noalloc.argtypes = [S(HsShape), S(HsCounts), S(HsCache), P, P, P,
                                             ctypes.c_float, ctypes.c_int32, P]
        L.hs_prefill_attn.argtypes = [S(HsShape), S(HsCounts), S(HsCache), P, P, P,
                                      ctypes.c_float, ctypes.c_uint32, P]
        L.hs_prefill_attn_variant.argtypes = L.hs_prefill_attn.argtypes
        for f in ("hs_cache_sizes", "hs_workspace_size", "hs_compress", "hs_compress_ex",
                  "hs_compress_masked", "hs_recompress", "hs_decode_attn",
                  "hs_decode_attn_noalloc", "hs_prefill_attn", "hs_prefill_attn_variant"):
            getattr(L, f).restype = ctypes.c_int
        L.hs_status_string.argtypes = [ctypes.c_int]
        L.hs_status_string.restype = ctypes.c_char_p
        L.hs_last_error.argtypes = []
        L.hs_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status):
    if status != HS_OK:
        raise HsError(status, lib().hs_last_error().decode())


def shape(batch, q_heads, kv_heads, seq_len, head_dim=128, block=64, dtype=HS_BF16):
    return HsShape(batch, q_heads, kv_heads, seq_len, head_dim, block, dtype)


def counts(n_pruned, n_sparse_k, n_sparse_v):
    return HsCounts(n_pruned, n_sparse_k, n_sparse_v)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else None


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def hs_status_string(status):
    return lib().hs_status_string(status).decode()


def hs_last_error():
    return lib().hs_last_error().decode()


def hs_cache_sizes(shp, cnt):
    out = HsCacheBytes()
    _check(lib().hs_cache_sizes(ctypes.byref(shp), ctypes.byref(cnt), ctypes.byref(out)))
    return {f: int(getattr(out, f)) for f in CACHE_FIELDS}


def hs_workspace_size(op, shp, cnt, num_splits=0):
    n = ctypes.c_size_t()
    _check(lib().hs_workspace_size(op, ctypes.byref(shp), ctypes.byref(cnt), num_splits,
                                   ctypes.byref(n)))
    return int(n.value)


def _cache_struct(cache):
    return HsCache(*[_ptr(cache.get(f)) for f in CACHE_FIELDS])


def hs_compress(shp, cnt, k, v, cache, ws, stream=None):
    _check(lib().hs_compress(ctypes.byref(shp), ctypes.byref(cnt), _ptr(k), _ptr(v),
                             ctypes.byref(_cache_struct(cache)), _ptr(ws),
                             ws.numel() * ws.element_size() if ws is not None else 0,
                             _stream(stream)))


def policy(sink_tokens=64, local_tokens=256):
    return HsPolicy(sink_tokens, local_tokens)


def hs_compress_ex(shp, cnt, pol, k, v, cache, ws, stream=None):
    _check(lib().hs_compress_ex(ctypes.byref(shp), ctypes.byref(cnt),
                                ctypes.byref(pol) if pol is not None else None, _ptr(k), _ptr(v),
                                ctypes.byref(_cache_struct(cache)), _ptr(ws),
                                ws.numel() * ws.element_size() if ws is not None else 0,
                                _stream(stream)))


def hs_compress_masked(shp, cnt, k, v, mode_k, mode_v, cache, head_status=None, stream=None):
    _check(lib().hs_compress_masked(ctypes.byref(shp), ctypes.byref(cnt), _ptr(k), _ptr(v),
                                    _ptr(mode_k), _ptr(mode_v), ctypes.byref(_cache_struct(cache)),
                                    _ptr(head_status), _stream(stream)))


def hs_recompress(shp, in_cnt, cache_in, out_cnt, cache_out, ws, stream=None):
    _check(lib().hs_recompress(ctypes.byref(shp), ctypes.byref(in_cnt),
                               ctypes.byref(_cache_struct(cache_in)), ctypes.byref(out_cnt),
                               ctypes.byref(_cache_struct(cache_out)), _ptr(ws),
                               ws.numel() * ws.element_size() if ws is not None else 0,
                               _stream(stream)))


def hs_decode_attn(shp, cnt, cache, q, o, lse=None, softmax_scale=0.0, num_splits=0, ws=None,
                   stream=None):
    _check(lib().hs_decode_attn(ctypes.byref(shp), ctypes.byref(cnt),
                                ctypes.byref(_cache_struct(cache)), _ptr(q), _ptr(o), _ptr(lse),
                                float(softmax_scale), int(num_splits), _ptr(ws),
                                ws.numel() * ws.element_size() if ws is not None else 0,
                                _stream(stream)))


def hs_decode_attn_noalloc(shp, cnt, cache, q, o, lse=None, softmax_scale=0.0, num_splits=0,
                           stream=None):
    _check(lib().hs_decode_attn_noalloc(ctypes.byref(shp), ctypes.byref(cnt),
                                        ctypes.byref(_cache_struct(cache)), _ptr(q), _ptr(o),
                                        _ptr(lse), float(softmax_scale), int(num_splits),
                                        _stream(stream)))


def hs_prefill_attn(shp, cnt, cache, q, o, lse=None, softmax_scale=0.0,
                    flags=HS_PREFILL_SMFMAC, stream=None):
    _check(lib().hs_prefill_attn(ctypes.byref(shp), ctypes.byref(cnt),
                                 ctypes.byref(_cache_struct(cache)), _ptr(q), _ptr(o), _ptr(lse),
                                 float(softmax_scale), int(flags), _stream(stream)))


def hs_prefill_attn_variant(shp, cnt, cache, q, o, lse=None, softmax_scale=0.0,
                            variant=HS_PREFILL_VARIANT_NONE, stream=None):
    _check(lib().hs_prefill_attn_variant(ctypes.byref(shp), ctypes.byref(cnt),
                                         ctypes.byref(_cache_struct(cache)), _ptr(q), _ptr(o),
                                         _ptr(lse), float(softmax_scale), int(variant),
                                         _stream(stream)))


# ------------------------------------------------------------------------------------------------
# Allocation helpers (device memory is the caller's; torch provides it).

def alloc_cache(shp, cnt, device="cuda"):
    """The eight buffers of a compressed cache as torch tensors (int32 maps, int16 pools holding
    bf16 bits), sized by hs_cache_sizes."""
    sizes = hs_cache_sizes(shp, cnt)
    out = {}
    for f in CACHE_FIELDS:
        if f.startswith("map"):
            out[f] = torch.empty(sizes[f] // 4, dtype=torch.int32, device=device)
        else:
            out[f] = torch.empty(sizes[f] // 2, dtype=torch.int16, device=device)
    return out


def alloc_workspace(op, shp, cnt, num_splits=0, device="cuda"):
    n = hs_workspace_size(op, shp, cnt, num_splits)
    return torch.zeros(max(n, 16), dtype=torch.uint8, device=device)
