"""The fp16 element type (hs_shape.dtype = HS_F16) on the GPU against the oracle: compressor, re-
compression and caller-mask compressor bit-exact; decode and causal prefill (both 2:4 paths), over
the oracle's own compressed cache (checked equal to the GPU's first), to max |o - o_ref| <= 1e-2
beyond the fp16 output rounding and relative L2 <= 5e-3."""
import numpy as np
import pytest
import torch

import oracle
from oracle import Dims
from sparse_kv_cache_magnitude_amd import hierasparse as hs
from sparse_kv_cache_magnitude_amd import synth
from tests import gpu_util as gu
from tests.test_gpu_prefill import sample_rows

pytestmark = pytest.mark.gpu

F16 = hs.HS_F16
MAX_ABS, REL_L2 = 1e-2, 5e-3


def half_ulp_f16(x):
    """Half an fp16 ulp at |x|: the error of rounding an exact result to the fp16 output."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -14)))
    return 2.0 ** (e - 11)


def assert_close_f16(o_gpu, o_ref, lse_gpu, lse_ref, tag):
    o_gpu = np.asarray(o_gpu, np.float64).reshape(o_ref.shape)
    err = np.abs(o_gpu - o_ref)
    rel = np.linalg.norm(o_gpu - o_ref) / max(np.linalg.norm(o_ref), 1e-30)
    excess = (err - half_ulp_f16(o_ref)).max()
    print(f"[{tag}] max_abs={err.max():.3e} max_abs_beyond_output_rounding={excess:.3e} "
          f"rel_l2={rel:.3e}", flush=True)
    assert excess <= MAX_ABS and rel <= REL_L2, (err.max(), excess, rel)
    lg = np.asarray(lse_gpu, np.float64).reshape(lse_ref.shape)
    fin = np.isfinite(lse_ref)
    assert (np.isfinite(lg) == fin).all()
    if fin.any():
        assert np.abs(lg[fin] - lse_ref[fin]).max() < 2e-2


def compress_f16(b, hq, hkv, L, B, counts, K, V):
    """GPU and oracle compression of fp16 K, V, checked equal; returns the oracle's cache too."""
    shp = hs.shape(b, hq, hkv, L, 128, B, dtype=F16)
    cnt = hs.counts(*counts)
    cache, want = gu.compress_checked(shp, cnt, Dims(b, hkv, L, 128, B, *counts, dtype=1), K, V)
    return shp, cnt, cache, want


@pytest.mark.parametrize("B", [64, 128])
@pytest.mark.parametrize("scale", [1.0, 300.0])   # 300: magnitudes past 256 take the 64-bit keys
def test_f16_compress_bit_exact(B, scale):
    rng = np.random.default_rng(B)
    b, hkv, L = 3, 2, 9 * B
    K = synth.f16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32) * scale)
    V = synth.f16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    K[0, 0, :7, :5] = synth.f16_bits(np.float32(6e-8))          # subnormal keys
    V[1, 1, 3, :] = 0x8000                                        # -0
    print(f"[f16 compress] B={B} scale={scale}", flush=True)
    compress_f16(b, 4, hkv, L, B, (2, 4, 5), K, V)


def test_f16_compress_workload():
    w = synth.workload("decode_llama8b_32k_b8")
    K, V = synth.make_kv(w.seed, w.b, w.hkv, w.L, w.D, outliers=w.outliers, dtype=1)
    print("[f16 compress] 32K batch 8", flush=True)
    compress_f16(w.b, w.hq, w.hkv, w.L, w.B, w.counts(), K, V)


def run_decode_f16(b, hq, hkv, L, B, counts, K, V, q):
    shp, cnt, cache, want = compress_f16(b, hq, hkv, L, B, counts, K, V)
    o = torch.empty((b, hq, 128), dtype=torch.int16, device="cuda")
    lse = torch.empty((b, hq), dtype=torch.float32, device="cuda")
    ws = hs.alloc_workspace(hs.HS_OP_DECODE, shp, cnt)
    hs.hs_decode_attn(shp, cnt, cache, gu.to_dev(q), o, lse, 0.0, 0, ws)
    torch.cuda.synchronize()
    d = Dims(b, hkv, L, 128, B, *counts, dtype=1)
    ref, ref_lse = oracle.decode(d, want, q, hq)
    return synth.f16_to_f32(gu.to_host_u16(o)), lse.cpu().numpy(), ref, ref_lse


@pytest.mark.parametrize("B,counts", [(64, (5, 20, 11)), (128, (2, 9, 14)), (64, (0, 0, 0)),
                                      (64, (4, 28, 28)), (128, (3, 29, 29))])
def test_f16_decode_small(B, counts):
    rng = np.random.default_rng(B + 1)
    b, hq, hkv, L = 2, 8, 2, 32 * B
    K = synth.f16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    V = synth.f16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    q = synth.f16_bits(rng.standard_normal((b, hq, 1, 128), dtype=np.float32))
    print(f"[f16 decode] B={B} counts={counts}", flush=True)
    o, lse, ref, ref_lse = run_decode_f16(b, hq, hkv, L, B, counts, K, V, q)
    assert_close_f16(o, ref, lse, ref_lse, f"f16 decode B={B} {counts}")


def test_f16_decode_workload():
    w = synth.workload("decode_llama8b_32k_b8")
    K, V = synth.make_kv(w.seed, w.b, w.hkv, w.L, w.D, outliers=w.outliers, dtype=1)
    q = synth.make_q(w.seed, w.b, w.hq, 1, w.D, dtype=1)
    print("[f16 decode] 32K batch 8", flush=True)
    o, lse, ref, ref_lse = run_decode_f16(w.b, w.hq, w.hkv, w.L, w.B, w.counts(), K, V, q)
    assert_close_f16(o, ref, lse, ref_lse, "f16 decode 32K b8")


def run_prefill_f16(b, hq, hkv, L, B, counts, K, V, Q, flags, rows=None):
    shp, cnt, cache, want = compress_f16(b, hq, hkv, L, B, counts, K, V)
    o = torch.empty((b, hq, L, 128), dtype=torch.int16, device="cuda")
    lse = torch.empty((b, hq, L), dtype=torch.float32, device="cuda")
    hs.hs_prefill_attn(shp, cnt, cache, gu.to_dev(Q), o, lse, 0.0, flags)
    torch.cuda.synchronize()
    d = Dims(b, hkv, L, 128, B, *counts, dtype=1)
    ref, ref_lse = oracle.prefill(d, want, Q, rows=rows)
    of = synth.f16_to_f32(gu.to_host_u16(o)).reshape(-1, 128)
    lf = lse.cpu().numpy().reshape(-1)
    if rows is not None:
        of, lf = of[rows], lf[rows]
    return of, lf, ref, ref_lse


@pytest.mark.parametrize("path", ["smfmac", "decompress"])
@pytest.mark.parametrize("B,counts", [(64, (3, 9, 5)), (128, (1, 5, 2)), (64, (0, 0, 0))])
def test_f16_prefill_small(path, B, counts):
    rng = np.random.default_rng(B + sum(counts) + 7)
    b, hq, hkv, L = 2, 8, 2, 16 * 64 if B == 64 else 8 * 128
    K = synth.f16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    V = synth.f16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    Q = synth.f16_bits(rng.standard_normal((b, hq, L, 128), dtype=np.float32))
    flags = hs.HS_PREFILL_SMFMAC if path == "smfmac" else hs.HS_PREFILL_DECOMPRESS
    print(f"[f16 prefill] {path} B={B} counts={counts}", flush=True)
    o, lse, ref, ref_lse = run_prefill_f16(b, hq, hkv, L, B, counts, K, V, Q, flags)
    assert_close_f16(o, ref, lse, ref_lse, f"f16 prefill {path} B={B} {counts}")


def test_f16_prefill_16k_sampled():
    w = synth.workload("prefill_16k_b1_B128")
    K, V = synth.make_kv(w.seed, w.b, w.hkv, w.L, w.D, outliers=w.outliers, dtype=1)
    Q = synth.make_q(w.seed + 100, w.b, w.hq, w.L, w.D, dtype=1)
    rows = sample_rows(w.b, w.hq, w.L, 4, 9)
    print("[f16 prefill] 16K B128 sampled", flush=True)
    o, lse, ref, ref_lse = run_prefill_f16(w.b, w.hq, w.hkv, w.L, w.B, w.counts(), K, V, Q,
                                           hs.HS_PREFILL_SMFMAC, rows)
    assert_close_f16(o, ref, lse, ref_lse, "f16 prefill 16K")


def test_f16_recompress_and_masked():
    rng = np.random.default_rng(91)
    b, hkv, L, B = 2, 2, 12 * 64, 64
    K = synth.f16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    V = synth.f16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    first, second = (2, 0, 6), (2, 6, 6)
    shp, c1, cache, want1 = compress_f16(b, hkv, hkv, L, B, first, K, V)
    c2 = hs.counts(*second)
    out = hs.alloc_cache(shp, c2)
    ws = hs.alloc_workspace(hs.HS_OP_RECOMPRESS, shp, c2)
    hs.hs_recompress(shp, c1, cache, c2, out, ws)
    torch.cuda.synchronize()
    d1, d2 = Dims(b, hkv, L, 128, B, *first, dtype=1), Dims(b, hkv, L, 128, B, *second, dtype=1)
    want = oracle.recompress(d1, want1, d2)
    gu.compare_cache(gu.cache_to_numpy(out), want)
    # the caller-mask compressor on the same shape
    mk, mv = synth.random_modes(92, b, hkv, L // B, *second)
    Km = synth.random_element_mask(93, K, mk, B, False)
    Vm = synth.random_element_mask(94, V, mv, B, True)
    cache_m = {f: t.zero_() for f, t in hs.alloc_cache(shp, c2).items()}
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    hs.hs_compress_masked(shp, c2, gu.to_dev(Km), gu.to_dev(Vm), dev(mk), dev(mv), cache_m)
    torch.cuda.synchronize()
    want_m = oracle.compress_masked(d2, Km, Vm, mk, mv)
    gu.compare_cache(gu.cache_to_numpy(cache_m), want_m)
