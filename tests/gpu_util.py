"""Helpers for the GPU parity tests: host <-> device marshalling around the C-ABI binding."""
import functools

import numpy as np
import torch

import oracle

from sparse_kv_cache_magnitude_amd import hierasparse as hs
from sparse_kv_cache_magnitude_amd import synth

DEV = "cuda"


def to_dev(a: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bits -> int16 device tensor with the same bytes."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def to_host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def shape_of(w, b=None, L=None):
    return hs.shape(b or w.b, w.hq, w.hkv, L or w.L, w.D, w.B)


def counts_of(w):
    return hs.counts(w.n_p, w.n_sk, w.n_sv)


def gpu_compress(shp, cnt, Kd, Vd):
    cache = hs.alloc_cache(shp, cnt)
    ws = hs.alloc_workspace(hs.HS_OP_COMPRESS, shp, cnt)
    hs.hs_compress(shp, cnt, Kd, Vd, cache, ws)
    torch.cuda.synchronize()
    return cache


def compress_checked(shp, cnt, d, K, V):
    """Compress K, V (host 16-bit patterns) on the GPU and with the oracle; the two caches must be
    equal byte for byte. Returns (GPU cache, oracle cache): attention references are built from
    the oracle's cache, which the GPU cache has just been shown to equal."""
    cache = gpu_compress(shp, cnt, to_dev(K), to_dev(V))
    want = oracle.compress(d, K, V)
    compare_cache(cache_to_numpy(cache), want)
    return cache, want


def cache_to_numpy(cache):
    out = {}
    for f, t in cache.items():
        a = t.cpu().numpy()
        out[f] = a if f.startswith("map") else a.view(np.uint16)
    return out


@functools.lru_cache(maxsize=2)
def workload_kv(name):
    w = synth.workload(name)
    K, V = synth.make_kv(w.seed, w.b, w.hkv, w.L, w.D, outliers=w.outliers)
    return K, V


def compare_cache(got, want, fields=hs.CACHE_FIELDS):
    for f in fields:
        g, e = np.asarray(got[f]), np.asarray(want[f])
        assert g.shape == e.shape, (f, g.shape, e.shape)
        if not np.array_equal(g, e):
            bad = np.flatnonzero(g != e)
            raise AssertionError(f"{f}: {bad.size} of {g.size} differ; first at {bad[:8]}: "
                                 f"got {g[bad[:8]]} want {e[bad[:8]]}")
