"""GPU causal prefill (hs_prefill_attn) against the oracle's fp64 causal attention over the oracle's
own compressed cache (the GPU cache is first checked equal to it byte for byte, in the same test),
for both ways 2:4 tiles reach the matrix cores (SMFMAC and decompress-to-LDS).
Gate: max |o - o_ref| <= 1e-2 beyond the bf16 output rounding and relative L2 <= 5e-3 (sampled
query rows at full size)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import Dims
from sparse_kv_cache_magnitude_amd import hierasparse as hs
from sparse_kv_cache_magnitude_amd import synth
from tests import gpu_util as gu
from tests.test_gpu_decode import assert_close

pytestmark = pytest.mark.gpu

FLAGS = {"smfmac": hs.HS_PREFILL_SMFMAC, "decompress": hs.HS_PREFILL_DECOMPRESS}


def run_prefill(b, hq, hkv, L, B, counts, K, V, Q, flags, scale=0.0, cache=None, want=None,
                rows=None, variant=None):
    """GPU causal prefill over the GPU compression of K, V and the oracle's over the oracle's
    compression (checked equal); rows: flat indices into [b][hq][L] to compare (None = all).
    Returns (o, lse, ref, ref_lse, cache, want) with o, lse restricted to the rows."""
    shp = hs.shape(b, hq, hkv, L, 128, B)
    cnt = hs.counts(*counts)
    d = Dims(b, hkv, L, 128, B, *counts)
    if cache is None:
        cache, want = gu.compress_checked(shp, cnt, d, K, V)
    qd = gu.to_dev(Q)
    o = torch.empty((b, hq, L, 128), dtype=torch.int16, device="cuda")
    lse = torch.empty((b, hq, L), dtype=torch.float32, device="cuda")
    if variant is None:
        hs.hs_prefill_attn(shp, cnt, cache, qd, o, lse, scale, flags)
    else:
        hs.hs_prefill_attn_variant(shp, cnt, cache, qd, o, lse, scale, variant)
    torch.cuda.synchronize()
    of = synth.bf16_to_f32(gu.to_host_u16(o)).reshape(-1, 128)
    lf = lse.cpu().numpy().reshape(-1)
    ref, ref_lse = oracle.prefill(d, want, Q, scale, rows=rows)
    if rows is not None:
        of, lf = of[rows], lf[rows]
    return of, lf, ref, ref_lse, cache, want


def sample_rows(b, hq, L, per_head, seed):
    """Flat row ids into [b][hq][L]: per head the first and last rows, the rows on both sides of
    the 32-query wave tiles and 64-token key tiles near both ends (0/1, 31/32, 63/64/65, 95/96,
    and their mirrors from the end), plus random rows."""
    rng = np.random.default_rng(seed)
    edges = {0, 1, 31, 32, 33, 63, 64, 65, 95, 96, 127, 128}
    edges |= {L - 1 - e for e in edges}
    rows = []
    for bi in range(b):
        for h in range(hq):
            base = (bi * hq + h) * L
            pick = set(edges)
            pick.update(rng.integers(0, L, per_head).tolist())
            rows += [base + r for r in sorted(pick) if 0 <= r < L]
    return np.array(rows, np.int64)


@pytest.mark.parametrize("path", ["smfmac", "decompress"])
@pytest.mark.parametrize("B,counts", [(64, (0, 0, 0)), (64, (3, 9, 5)), (64, (0, 16, 16)),
                                      (128, (1, 5, 2)), (128, (0, 0, 8))])
def test_prefill_small_full_compare(path, B, counts):
    rng = np.random.default_rng(B + sum(counts))
    b, hq, hkv, L = 2, 8, 2, 16 * 64 if B == 64 else 8 * 128
    K = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    V = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    Q = synth.bf16_bits(rng.standard_normal((b, hq, L, 128), dtype=np.float32))
    print(f"[prefill] {path} B={B} counts={counts}", flush=True)
    o, lse, ref, ref_lse, _, _ = run_prefill(b, hq, hkv, L, B, counts, K, V, Q, FLAGS[path])
    assert_close(o, ref, lse, ref_lse, f"{path} B={B} {counts}")


@pytest.mark.parametrize("path", ["smfmac", "decompress"])
@pytest.mark.parametrize("G", [1, 2, 3, 4, 8])
def test_prefill_gqa_groups(path, G):
    rng = np.random.default_rng(100 + G)
    b, hkv, L, B = 1, 2, 5 * 64, 64
    hq = G * hkv
    counts = (1, 2, 2)
    K = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    V = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    Q = synth.bf16_bits(rng.standard_normal((b, hq, L, 128), dtype=np.float32))
    o, lse, ref, ref_lse, _, _ = run_prefill(b, hq, hkv, L, B, counts, K, V, Q, FLAGS[path],
                                             scale=0.07)
    assert_close(o, ref, lse, ref_lse, f"{path} G={G}")


@pytest.mark.parametrize("path", ["smfmac", "decompress"])
def test_prefill_pruned_prefix_rows_are_empty(path):
    """Rows whose visible set is empty (their own and all earlier blocks pruned) give 0 / -inf."""
    rng = np.random.default_rng(3)
    b, hq, hkv, L, B = 1, 4, 1, 4 * 64, 64
    scale = np.ones((1, 1, L, 1), np.float32)
    scale[:, :, :128] = 1e-3   # blocks 0 and 1 have the smallest magnitude -> pruned
    K = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32) * scale)
    V = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32) * scale)
    Q = synth.bf16_bits(rng.standard_normal((b, hq, L, 128), dtype=np.float32))
    counts = (2, 1, 1)
    o, lse, ref, ref_lse, _, _ = run_prefill(b, hq, hkv, L, B, counts, K, V, Q, FLAGS[path])
    assert np.isneginf(ref_lse).any()   # the data makes the first blocks' rows empty
    assert_close(o, ref, lse, ref_lse, f"{path} empty rows")


@pytest.mark.parametrize("path", ["smfmac", "decompress"])
def test_prefill_workload_sampled(path):
    """Full-size causal prefill (16K tokens, 32/8 heads, 128-token blocks, 70% 2:4) on sampled
    rows, in the launch configuration the benchmark times."""
    w = synth.workload("prefill_16k_b1_B128")
    K, V = gu.workload_kv(w.name)
    Q = synth.make_q(w.seed, w.b, w.hq, w.L, w.D)
    print(f"[prefill] {w.name} {path}", flush=True)
    rows = sample_rows(w.b, w.hq, w.L, 6, 7)
    o, lse, ref, ref_lse, _, _ = run_prefill(w.b, w.hq, w.hkv, w.L, w.B, w.counts(), K, V, Q,
                                             FLAGS[path], rows=rows)
    assert_close(o, ref, lse, ref_lse, f"{w.name} {path}")


@pytest.mark.parametrize("path", ["smfmac", "decompress"])
def test_prefill_bench_workload_sampled(path):
    """Full-size causal prefill at the benchmark's prefill shape (32K tokens, batch 8, 32/8 heads,
    64-token blocks, 77 pruned / 307 2:4 / 128 dense blocks per head, K outlier channels) on
    sampled rows (the wave- and key-tile edges near both ends of every head, and two random rows
    per head), on both 2:4 paths (the benchmark times the SMFMAC one)."""
    w = synth.workload("decode_llama8b_32k_b8")
    K, V = gu.workload_kv(w.name)
    Q = synth.make_q(w.seed + 100, w.b, w.hq, w.L, w.D)
    print(f"[prefill] {w.name} full-size sampled, {path}", flush=True)
    rows = sample_rows(w.b, w.hq, w.L, 2, 8)
    o, lse, ref, ref_lse, _, _ = run_prefill(w.b, w.hq, w.hkv, w.L, w.B, w.counts(), K, V, Q,
                                             FLAGS[path], rows=rows)
    assert_close(o, ref, lse, ref_lse, f"{w.name} prefill {path}")


def test_prefill_paths_agree_and_deterministic():
    rng = np.random.default_rng(21)
    b, hq, hkv, L, B = 1, 8, 2, 1024, 64
    counts = (2, 6, 9)
    K = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    V = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    Q = synth.bf16_bits(rng.standard_normal((b, hq, L, 128), dtype=np.float32))
    o1, l1, _, _, cache, want = run_prefill(b, hq, hkv, L, B, counts, K, V, Q,
                                            hs.HS_PREFILL_SMFMAC)
    o1b, l1b, _, _, _, _ = run_prefill(b, hq, hkv, L, B, counts, K, V, Q, hs.HS_PREFILL_SMFMAC,
                                       cache=cache, want=want)
    o2, l2, _, _, _, _ = run_prefill(b, hq, hkv, L, B, counts, K, V, Q, hs.HS_PREFILL_DECOMPRESS,
                                     cache=cache, want=want)
    assert np.array_equal(o1, o1b) and np.array_equal(l1, l1b)
    # the two paths multiply the same bf16 values; only accumulation order may differ
    assert np.abs(o1 - o2).max() <= 1e-2


def test_prefill_dense_equals_library_attention():
    rng = np.random.default_rng(22)
    b, hq, hkv, L, B = 1, 4, 1, 512, 64
    K = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    V = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    Q = synth.bf16_bits(rng.standard_normal((b, hq, L, 128), dtype=np.float32))
    o, _, _, _, _, _ = run_prefill(b, hq, hkv, L, B, (0, 0, 0), K, V, Q, hs.HS_PREFILL_SMFMAC)
    qt = torch.from_numpy(synth.bf16_to_f32(Q))
    kt = torch.from_numpy(synth.bf16_to_f32(K)).repeat_interleave(hq // hkv, dim=1)
    vt = torch.from_numpy(synth.bf16_to_f32(V)).repeat_interleave(hq // hkv, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True).numpy()
    assert_close(o, ref.astype(np.float64).reshape(-1, 128), tag="prefill dense vs sdpa fp32")


@pytest.mark.parametrize("path", ["smfmac", "decompress"])
def test_prefill_long_head_eight_wave_path(path):
    """A head of 2049 64-token blocks (131136 tokens): more blocks than the four-wave SMFMAC
    workgroups list, so the SMFMAC path runs the eight-wave kernel; sampled rows (the tile edges
    near both ends and random rows) against the oracle."""
    rng = np.random.default_rng(31)
    b, hq, hkv, B, nb = 1, 2, 1, 64, 2049
    L = nb * B
    counts = (205, 1024, 1024)
    K = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    V = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    Q = synth.bf16_bits(rng.standard_normal((b, hq, L, 128), dtype=np.float32))
    print(f"[prefill] {path} L={L} (2049 blocks)", flush=True)
    rows = sample_rows(b, hq, L, 12, 9)
    o, lse, ref, ref_lse, _, _ = run_prefill(b, hq, hkv, L, B, counts, K, V, Q, FLAGS[path],
                                             rows=rows)
    assert_close(o, ref, lse, ref_lse, f"{path} L={L}")


VARIANTS = {"sync_loads": hs.HS_PREFILL_VARIANT_SYNC_LOADS,
            "no_alias": hs.HS_PREFILL_VARIANT_NO_ALIAS,
            "generic_walk": hs.HS_PREFILL_VARIANT_GENERIC_WALK,
            "lockstep": hs.HS_PREFILL_VARIANT_LOCKSTEP,
            "lds_relayout": hs.HS_PREFILL_VARIANT_LDS_RELAYOUT}


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("B,counts", [(64, (0, 16, 16)), (64, (3, 9, 5)), (64, (0, 0, 0)),
                                      (128, (1, 5, 2)), (128, (0, 8, 8))])
def test_prefill_ablation_variants(variant, B, counts):
    """The measurement variants of the SMFMAC prefill (each with one optimisation left out) against
    the oracle. The variants that only change where and when operands are staged, or which copy of
    the tile body runs, compute every product and sum of the default kernel in the same order:
    their outputs equal its outputs bit for bit. The eight-wave variant issues GEMM2 one tile late,
    and the LDS re-layout variant gives each lane other tokens to sum, so they are held to the
    oracle only."""
    rng = np.random.default_rng(B * 7 + sum(counts))
    b, hq, hkv, L = 2, 8, 2, 16 * 64 if B == 64 else 8 * 128
    K = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    V = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    Q = synth.bf16_bits(rng.standard_normal((b, hq, L, 128), dtype=np.float32))
    print(f"[prefill variant] {variant} B={B} counts={counts}", flush=True)
    o0, l0, _, _, cache, want = run_prefill(b, hq, hkv, L, B, counts, K, V, Q,
                                            hs.HS_PREFILL_SMFMAC)
    o, lse, ref, ref_lse, _, _ = run_prefill(b, hq, hkv, L, B, counts, K, V, Q, None,
                                             cache=cache, want=want, variant=VARIANTS[variant])
    assert_close(o, ref, lse, ref_lse, f"{variant} B={B} {counts}")
    if variant not in ("lockstep", "lds_relayout"):
        assert np.array_equal(o, o0) and np.array_equal(lse, l0)
