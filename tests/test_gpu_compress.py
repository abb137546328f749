"""GPU compressor (hs_compress) against the oracle: maps and all six pools bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from oracle import Dims
from sparse_kv_cache_magnitude_amd import hierasparse as hs
from sparse_kv_cache_magnitude_amd import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _check(b, hkv, L, B, counts, K, V, hq=None):
    hq = hq or hkv
    shp = hs.shape(b, hq, hkv, L, 128, B)
    cnt = hs.counts(*counts)
    print(f"[compress] b={b} hkv={hkv} L={L} B={B} counts={counts}", flush=True)
    cache = gu.gpu_compress(shp, cnt, gu.to_dev(K), gu.to_dev(V))
    want = oracle.compress(Dims(b, hkv, L, 128, B, *counts), K, V)
    gu.compare_cache(gu.cache_to_numpy(cache), want)
    return cache


@pytest.mark.parametrize("name", ["decode_1h_4k_all24", "prefill_16k_b1_B128",
                                  "decode_llama8b_32k_b8", "decode_128k_b4"])
def test_compress_workloads_bit_exact(name):
    w = synth.workload(name)
    K, V = gu.workload_kv(name)
    _check(w.b, w.hkv, w.L, w.B, w.counts(), K, V, hq=w.hq)


@pytest.mark.parametrize("B", [64, 128])
@pytest.mark.parametrize("counts_fn", [
    lambda nb: (0, 0, 0),            # all dense
    lambda nb: (0, nb, nb),          # all 2:4
    lambda nb: (nb, 0, 0),           # all pruned
    lambda nb: (1, nb - 1, 0),       # K all sparse, V all dense among survivors
    lambda nb: (nb // 3, nb // 2, nb // 5),
])
def test_compress_edge_counts(B, counts_fn):
    rng = np.random.default_rng(B)
    b, hkv, L = 3, 2, 9 * B   # nb = 9: not a power of two
    K = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    V = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32) * 3)
    _check(b, hkv, L, B, counts_fn(L // B), K, V)


def test_compress_single_block_and_ties():
    rng = np.random.default_rng(7)
    vals = np.array([0.0, -0.0, 1.0, -1.0, 2.0, 0.5, -2.0], np.float32)
    b, hkv, L, B = 2, 3, 64 * 6, 64
    K = synth.bf16_bits(vals[rng.integers(0, len(vals), (b, hkv, L, 128))])
    V = synth.bf16_bits(vals[rng.integers(0, len(vals), (b, hkv, L, 128))])
    K[:, :, 64:128] = K[:, :, 256:320]     # duplicated blocks -> tied block losses
    V[:, :, 64:128] = V[:, :, 256:320]
    _check(b, hkv, L, B, (2, 2, 3), K, V)
    _check(1, 1, 64, 64, (0, 1, 0), K[:1, :1, :64], V[:1, :1, :64])   # nb = 1


def test_compress_extreme_magnitudes():
    rng = np.random.default_rng(11)
    b, hkv, L, B = 1, 2, 512, 64
    mag = np.exp2(rng.integers(-130, 24, (b, hkv, L, 128))).astype(np.float32)
    sign = np.where(rng.random((b, hkv, L, 128)) < 0.5, -1.0, 1.0).astype(np.float32)
    K = synth.bf16_bits(mag * sign * rng.uniform(1, 1.99, (b, hkv, L, 128)).astype(np.float32))
    V = synth.bf16_bits(np.flip(mag, axis=2) * sign)
    K = np.where(np.abs(synth.bf16_to_f32(K)) >= 2.0 ** 24, 0, K).astype(np.uint16)
    _check(b, hkv, L, B, (2, 3, 3), K, V)


def test_compress_deterministic():
    w = synth.workload("decode_1h_4k_all24")
    K, V = gu.workload_kv(w.name)
    shp, cnt = hs.shape(1, 1, 1, w.L, 128, w.B), hs.counts(0, 40, 20)
    Kd, Vd = gu.to_dev(K), gu.to_dev(V)
    a = gu.cache_to_numpy(gu.gpu_compress(shp, cnt, Kd, Vd))
    b = gu.cache_to_numpy(gu.gpu_compress(shp, cnt, Kd, Vd))
    gu.compare_cache(a, b)


@pytest.mark.parametrize("B", [64, 128])
def test_compress_keys_bit_exact(B):
    """The per-block loss keys themselves (not only the ranking they lead to) equal the oracle's:
    N(0,1) data with a few magnitudes of 256 and more in some blocks, so that within one launch
    some waves take the 32-bit key path and others its 64-bit fallback."""
    rng = np.random.default_rng(31 + B)
    b, hkv, L = 2, 2, B * 9
    Kf = rng.standard_normal((b, hkv, L, 128), dtype=np.float32)
    Vf = rng.standard_normal((b, hkv, L, 128), dtype=np.float32)
    Kf[0, 0, 3, 5] = 300.0
    Kf[1, 1, 4 * B + 7, 100] = -4096.0
    Vf[0, 1, 2 * B + 1, 64] = 257.0
    Vf[1, 0, 5 * B, 0] = 1.0e6
    Kf[0, 1, 6 * B + 2, 9] = 255.0  # the largest magnitude of the fast path
    K, V = synth.bf16_bits(Kf), synth.bf16_bits(Vf)
    counts = (1, 3, 4)
    shp, cnt = hs.shape(b, hkv, hkv, L, 128, B), hs.counts(*counts)
    cache = hs.alloc_cache(shp, cnt)
    ws = hs.alloc_workspace(hs.HS_OP_COMPRESS, shp, cnt)
    hs.hs_compress(shp, cnt, gu.to_dev(K), gu.to_dev(V), cache, ws)
    torch.cuda.synchronize()
    nb = L // B
    got = ws[: b * hkv * nb * 3 * 8].cpu().numpy().view(np.uint64).reshape(b, hkv, nb, 3)
    want = oracle.compress(Dims(b, hkv, L, 128, B, *counts), K, V)
    assert np.array_equal(got, want["keys"]), np.argwhere(got != want["keys"])[:8]
    gu.compare_cache(gu.cache_to_numpy(cache), want)


def _check_policy(b, hkv, L, B, counts, sink, local, K, V, hq=None):
    hq = hq or hkv
    shp, cnt = hs.shape(b, hq, hkv, L, 128, B), hs.counts(*counts)
    print(f"[compress_ex] b={b} hkv={hkv} L={L} B={B} counts={counts} sink={sink} "
          f"local={local}", flush=True)
    cache = hs.alloc_cache(shp, cnt)
    ws = hs.alloc_workspace(hs.HS_OP_COMPRESS, shp, cnt)
    hs.hs_compress_ex(shp, cnt, hs.policy(sink, local), gu.to_dev(K), gu.to_dev(V), cache, ws)
    torch.cuda.synchronize()
    want = oracle.compress(Dims(b, hkv, L, 128, B, *counts), K, V, sink=sink, local=local)
    gu.compare_cache(gu.cache_to_numpy(cache), want)


@pytest.mark.parametrize("B", [64, 128])
@pytest.mark.parametrize("sink,local", [(0, 0), (64, 256), (1, 1), (65, 0), (0, 129),
                                        (300, 500)])
def test_compress_dense_policy(B, sink, local):
    rng = np.random.default_rng(B + sink + local)
    b, hkv, L = 2, 2, 16 * B
    K = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    V = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    held = len({i for i in range(16) for t in (i * B, i * B + B - 1)
                if i * B < sink or i * B + B - 1 >= L - local})
    r = 16 - held
    _check_policy(b, hkv, L, B, (r // 4, r - r // 4, r // 2), sink, local, K, V)


def test_compress_dense_policy_workload():
    """The 32K batch-8 cache with the quality runs' policy (64 sink, 256 local-window tokens)."""
    w = synth.workload("decode_llama8b_32k_b8")
    K, V = gu.workload_kv(w.name)
    _check_policy(w.b, w.hkv, w.L, w.B, w.counts(), 64, 256, K, V, hq=w.hq)
