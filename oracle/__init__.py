"""fp64 CPU oracle for hierarchical semi-structured sparse KV attention (ctypes wrapper of hso.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package; the GPU library and its Python binding never import it.

What each function follows is cited in hso.c ("HieraSparse", arXiv 2604.16864v2: Eq. (1),
Eq. (2a)-(2d), §III-B, §IV-A/B) together with the readings R1-R8 taken where the paper is silent;
recompress (§III, Fig. 3) is the composition of unpack and compress (R9), compress_masked the
generic compressor fed by caller masks (§III-A, §IV-B; R10), compress(sink=, local=) the dense
policy of the quality runs (§V-A; R11), and Dims.dtype = 1 the fp16 element type (R12).
Parity is pinned by the tests under tests/ (brute force, closed forms, library routines, identities).
"""
import ctypes
import os
from dataclasses import dataclass

import numpy as np

from . import build as _build

_LIB = None

_ERR = {1: "bad shape", 2: "bad block counts", 3: "input value non-finite or |x| >= 2^24",
        4: "inconsistent index maps"}


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("b", "hkv", "L", "D", "B", "n_p", "n_sk", "n_sv", "dtype")]


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        P = ctypes.c_void_p
        lib.hso_pool_elems.argtypes = [ctypes.POINTER(_Dims), P]
        lib.hso_compress.argtypes = [ctypes.POINTER(_Dims)] + [P] * 12
        lib.hso_compress_ex.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int, ctypes.c_int] + [P] * 12
        lib.hso_unpack.argtypes = [ctypes.POINTER(_Dims)] + [P] * 11
        lib.hso_compress_masked.argtypes = [ctypes.POINTER(_Dims)] + [P] * 13
        lib.hso_attention.argtypes = [ctypes.c_int] * 9 + [P] * 4 + [ctypes.c_double,
                                                                      ctypes.c_int64, P, P, P]
        for f in (lib.hso_pool_elems, lib.hso_compress, lib.hso_unpack, lib.hso_attention,
                  lib.hso_compress_masked, lib.hso_compress_ex):
            f.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc):
    if rc != 0:
        raise ValueError(f"oracle: {_ERR.get(rc, rc)}")


@dataclass
class Dims:
    """b, Hkv, L tokens, head_dim D, block size B, per-(batch, KV head) block counts, and the
    element type of the 16-bit patterns (0 bf16, 1 IEEE binary16; hso.c R12)."""
    b: int
    hkv: int
    L: int
    D: int
    B: int
    n_p: int
    n_sk: int
    n_sv: int
    dtype: int = 0

    @property
    def nb(self):
        return self.L // self.B

    def c(self):
        return _Dims(self.b, self.hkv, self.L, self.D, self.B, self.n_p, self.n_sk, self.n_sv,
                     self.dtype)


POOLS = ("map_k", "map_v", "k_dense", "k_nnz", "k_meta", "v_dense", "v_nnz", "v_meta")


def pool_elems(d: Dims) -> dict:
    out = np.zeros(8, np.int64)
    _check(_lib().hso_pool_elems(ctypes.byref(d.c()), _ptr(out)))
    return dict(zip(POOLS, (int(x) for x in out)))


def pool_bytes(d: Dims) -> dict:
    """Bytes of each buffer: maps are int32, pools are bf16 bits (2 bytes)."""
    return {k: v * (4 if k.startswith("map") else 2) for k, v in pool_elems(d).items()}


def compress(d: Dims, K: np.ndarray, V: np.ndarray, with_loss: bool = False, sink: int = 0,
             local: int = 0) -> dict:
    """Compress bf16-bit tensors K, V [b][Hkv][L][D] (uint16). Returns the maps, the six pools
    (flat arrays) and 'keys' [b][Hkv][nb][3] uint64 (K 2:4 loss, V 2:4 loss, whole-block loss);
    with_loss adds the same losses in fp64 as 'loss'. sink / local: the dense policy of hso.c
    R11 (blocks holding one of the first sink or last local tokens stay dense, unranked)."""
    K = np.ascontiguousarray(K, dtype=np.uint16)
    V = np.ascontiguousarray(V, dtype=np.uint16)
    assert K.shape == V.shape == (d.b, d.hkv, d.L, d.D)
    n = pool_elems(d)
    out = {k: np.zeros(n[k], np.int32 if k.startswith("map") else np.uint16) for k in POOLS}
    keys = np.zeros((d.b, d.hkv, d.nb, 3), np.uint64)
    loss = np.zeros((d.b, d.hkv, d.nb, 3), np.float64) if with_loss else None
    _check(_lib().hso_compress_ex(ctypes.byref(d.c()), int(sink), int(local), _ptr(K), _ptr(V),
                                  *[_ptr(out[k]) for k in POOLS], _ptr(keys), _ptr(loss)))
    out["keys"] = keys
    if with_loss:
        out["loss"] = loss
    return out


def compress_masked(d: Dims, K: np.ndarray, V: np.ndarray, mode_k: np.ndarray,
                    mode_v: np.ndarray) -> dict:
    """Compression with caller masks ([HS] §III-A cache pruner, §IV-B generic kernel; hso.c R10).
    K, V [b][Hkv][L][D] bf16 bits with the element mask applied; mode_k, mode_v [b][Hkv][nb]
    uint8 (0 pruned, 1 dense, 2 2:4). Returns the maps, the six pools (zero where nothing is
    written) and 'head_status' [b][Hkv] int32."""
    K = np.ascontiguousarray(K, dtype=np.uint16)
    V = np.ascontiguousarray(V, dtype=np.uint16)
    assert K.shape == V.shape == (d.b, d.hkv, d.L, d.D)
    mk = np.ascontiguousarray(mode_k, dtype=np.uint8)
    mv = np.ascontiguousarray(mode_v, dtype=np.uint8)
    assert mk.shape == mv.shape == (d.b, d.hkv, d.nb)
    n = pool_elems(d)
    out = {k: np.zeros(n[k], np.int32 if k.startswith("map") else np.uint16) for k in POOLS}
    status = np.zeros((d.b, d.hkv), np.int32)
    _check(_lib().hso_compress_masked(ctypes.byref(d.c()), _ptr(K), _ptr(V), _ptr(mk), _ptr(mv),
                                      *[_ptr(out[k]) for k in POOLS], _ptr(status)))
    out["head_status"] = status
    return out


def unpack(d: Dims, cache: dict):
    """Dense stand-ins of a compressed cache: (Kt, Vt) [b][Hkv][L][D] bf16 bits with zeros where
    2:4 dropped or blocks were pruned, and visible [b][Hkv][nb] uint8."""
    Kt = np.zeros((d.b, d.hkv, d.L, d.D), np.uint16)
    Vt = np.zeros_like(Kt)
    vis = np.zeros((d.b, d.hkv, d.nb), np.uint8)
    arrs = [np.ascontiguousarray(cache[k]) for k in POOLS]
    _check(_lib().hso_unpack(ctypes.byref(d.c()), *[_ptr(a) for a in arrs], _ptr(Kt), _ptr(Vt),
                             _ptr(vis)))
    return Kt, Vt, vis


def recompress(d_in: Dims, cache: dict, d_out: Dims) -> dict:
    """Re-compression with other block counts ([HS] §III, Fig. 3: one compression for prefill,
    another for decode): the compressor applied to the dense tensors the compressed cache stands
    for. d_in and d_out differ only in their counts."""
    assert (d_in.b, d_in.hkv, d_in.L, d_in.D, d_in.B) == (d_out.b, d_out.hkv, d_out.L, d_out.D,
                                                           d_out.B)
    Kt, Vt, _ = unpack(d_in, cache)
    return compress(d_out, Kt, Vt)


def attention(Q, Kt, Vt, visible, B: int, causal: bool, scale: float = 0.0, rows=None,
              dtype: int = 0):
    """fp64 softmax attention over visible tokens. Q [b][Hq][Lq][D] 16-bit patterns of element type
    dtype (0 bf16, 1 fp16); Kt, Vt [b][Hkv][L][D] likewise; visible [b][Hkv][L/B]. rows: flat
    indices into [b][Hq][Lq] (None = all). Returns (O [nrows][D] fp64, lse [nrows] fp64)."""
    Q = np.ascontiguousarray(Q, dtype=np.uint16)
    Kt = np.ascontiguousarray(Kt, dtype=np.uint16)
    Vt = np.ascontiguousarray(Vt, dtype=np.uint16)
    visible = np.ascontiguousarray(visible, dtype=np.uint8)
    b, hq, lq, D = Q.shape
    _, hkv, L, _ = Kt.shape
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
    n = b * hq * lq if rows is None else len(rows)
    O = np.zeros((n, D), np.float64)
    lse = np.zeros(n, np.float64)
    _check(_lib().hso_attention(b, hq, hkv, L, D, B, lq, int(causal), int(dtype), _ptr(Q),
                                _ptr(Kt), _ptr(Vt), _ptr(visible), float(scale), n, _ptr(rows),
                                _ptr(O), _ptr(lse)))
    return O, lse


def decode(d: Dims, cache: dict, q, hq: int, scale: float = 0.0, rows=None):
    """Decode attention over a compressed cache: q [b][Hq][D] -> (O, lse) for the listed rows."""
    Kt, Vt, vis = unpack(d, cache)
    q = np.asarray(q).reshape(d.b, hq, 1, d.D)
    return attention(q, Kt, Vt, vis, d.B, False, scale, rows, d.dtype)


def prefill(d: Dims, cache: dict, Q, scale: float = 0.0, rows=None):
    """Causal prefill attention over a compressed cache: Q [b][Hq][L][D]."""
    Kt, Vt, vis = unpack(d, cache)
    return attention(Q, Kt, Vt, vis, d.B, True, scale, rows, d.dtype)
