"""Pins of the CPU oracle against what the paper and the mathematics fix (no GPU).

Each test checks the oracle against something other than itself: brute-force enumeration, exact
rational arithmetic, the paper's printed worked values (tests/golden), a library routine
(torch scaled_dot_product_attention in float64), or an identity that holds exactly.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import Dims
from sparse_kv_cache_magnitude_amd import synth
from tests import pinlib

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hierasparse_worked_values.json")


def tie_heavy(shape, seed):
    """bf16 bits drawn from a tiny value set so that equal magnitudes are common."""
    rng = np.random.default_rng(seed)
    vals = np.array([0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0, 3.0], np.float32)
    return synth.bf16_bits(vals[rng.integers(0, len(vals), size=shape)])


def normal(shape, seed):
    return synth.bf16_bits(np.random.default_rng(seed).standard_normal(shape, dtype=np.float32))


# ------------------------------------------------------------------------------------------------
# C1: element selection (Eq. 2a-2b, fused top-2 of §IV-B)

@pytest.mark.parametrize("maker", [tie_heavy, normal])
def test_kept_pairs_match_brute_force(maker):
    d = Dims(b=1, hkv=2, L=32, D=32, B=16, n_p=0, n_sk=2, n_sv=2)   # every block 2:4
    K = maker((d.b, d.hkv, d.L, d.D), 1)
    V = maker((d.b, d.hkv, d.L, d.D), 2)
    cache = oracle.compress(d, K, V)
    _, _, _, keepK, keepV = pinlib.decode_cache(d.b, d.hkv, d.L, d.D, d.B, cache)
    for h in range(d.hkv):
        for is_v, X, keep in ((0, K[0, h], keepK[0, h]), (1, V[0, h], keepV[0, h])):
            for i in range(d.nb):
                for row, g, x4 in pinlib.groups_of_block(X, is_v, d.B, d.D, i):
                    if not is_v:
                        got = keep[i * d.B + row, 4 * g:4 * g + 4]
                    else:
                        got = keep[i * d.B + 4 * g:i * d.B + 4 * g + 4, row]
                    want = pinlib.kept_pair_brute(x4)
                    assert tuple(np.flatnonzero(got)) == want, (h, is_v, i, row, g, x4)


def test_exactly_two_kept_and_magnitude_order():
    d = Dims(b=2, hkv=1, L=64, D=64, B=32, n_p=0, n_sk=2, n_sv=2)
    K = normal((d.b, d.hkv, d.L, d.D), 3)
    V = tie_heavy((d.b, d.hkv, d.L, d.D), 4)
    cache = oracle.compress(d, K, V)
    Kt, Vt, _, keepK, keepV = pinlib.decode_cache(d.b, d.hkv, d.L, d.D, d.B, cache)
    # K groups: 4 consecutive channels; V groups: 4 consecutive tokens
    gk = keepK.reshape(d.b, d.hkv, d.L, d.D // 4, 4)
    gv = keepV.reshape(d.b, d.hkv, d.L // 4, 4, d.D)
    assert (gk.sum(-1) == 2).all() and (gv.sum(-2) == 2).all()
    ak = np.abs(synth.bf16_to_f32(K)).reshape(gk.shape)
    av = np.abs(synth.bf16_to_f32(V)).reshape(gv.shape)
    kept_min = np.where(gk, ak, np.inf).min(-1)
    drop_max = np.where(~gk, ak, -np.inf).max(-1)
    assert (kept_min >= drop_max).all()
    kept_min = np.where(gv, av, np.inf).min(-2)
    drop_max = np.where(~gv, av, -np.inf).max(-2)
    assert (kept_min >= drop_max).all()
    # kept values are the input values, dropped ones read back as zero
    assert (Kt == np.where(keepK, K, 0)).all() and (Vt == np.where(keepV, V, 0)).all()


# ------------------------------------------------------------------------------------------------
# C2-C3: block losses (Eq. 2c) and block modes (Eq. 2d + pruned state)

def test_block_keys_exact_arithmetic():
    d = Dims(b=1, hkv=2, L=64, D=16, B=16, n_p=1, n_sk=1, n_sv=2)
    K = tie_heavy((d.b, d.hkv, d.L, d.D), 5)
    V = normal((d.b, d.hkv, d.L, d.D), 6)
    V[0, 1, 5, 3] = synth.bf16_bits(np.float32(3e-6))   # below 2^-17: truncated by the key
    V[0, 1, 6, 3] = synth.bf16_bits(np.float32(1e-30))
    out = oracle.compress(d, K, V, with_loss=True)
    for h in range(d.hkv):
        want = pinlib.block_keys_exact(K[0, h], V[0, h], d.B, d.D)
        got = [tuple(int(x) for x in row) for row in out["keys"][0, h]]
        assert got == want
        # the fp64 L1 sums are the exact losses up to rounding
        exact = []
        for i in range(d.nb):
            row = []
            for is_v, X in ((0, K[0, h]), (1, V[0, h])):
                s = 0
                for _, _, x4 in pinlib.groups_of_block(X, is_v, d.B, d.D, i):
                    keep = pinlib.kept_pair_brute(x4)
                    s += sum(pinlib.mag(x4[j]) for j in range(4) if j not in keep)
                row.append(float(s))
            exact.append(row)
        np.testing.assert_allclose(out["loss"][0, h, :, :2], np.array(exact), rtol=1e-13)


@pytest.mark.parametrize("counts", [(0, 3, 5), (2, 3, 4), (3, 5, 0), (8, 0, 0), (0, 8, 8),
                                    (1, 7, 7)])
def test_block_modes_brute_force(counts):
    n_p, n_sk, n_sv = counts
    d = Dims(b=2, hkv=2, L=8 * 16, D=16, B=16, n_p=n_p, n_sk=n_sk, n_sv=n_sv)
    K = tie_heavy((d.b, d.hkv, d.L, d.D), 7)
    V = tie_heavy((d.b, d.hkv, d.L, d.D), 8)
    # duplicate some blocks so whole-block and 2:4 keys tie exactly
    K[:, :, 16:32] = K[:, :, 48:64]
    V[:, :, 16:32] = V[:, :, 48:64]
    K[:, :, 96:112] = K[:, :, 0:16]
    V[:, :, 96:112] = V[:, :, 0:16]
    out = oracle.compress(d, K, V)
    mk = out["map_k"].reshape(d.b, d.hkv, d.nb)
    mv = out["map_v"].reshape(d.b, d.hkv, d.nb)
    for bi in range(d.b):
        for h in range(d.hkv):
            keys = [tuple(int(x) for x in r) for r in out["keys"][bi, h]]
            want_k, want_v = pinlib.modes_brute(keys, n_p, n_sk, n_sv)
            got_k = [0 if x == 0 else (1 if x > 0 else 2) for x in mk[bi, h]]
            got_v = [0 if x == 0 else (1 if x > 0 else 2) for x in mv[bi, h]]
            assert got_k == want_k and got_v == want_v


def test_fp64_loss_ranking_agrees_with_integer_keys():
    w = synth.workload("decode_llama8b_32k_b8")
    d = Dims(b=1, hkv=2, L=8192, D=128, B=64, n_p=19, n_sk=77, n_sv=77)
    K, V = synth.make_kv(w.seed, 1, 2, d.L, d.D, outliers=4)
    out = oracle.compress(d, K, V, with_loss=True)
    for h in range(2):
        for j in range(3):
            ki = np.lexsort((np.arange(d.nb), out["keys"][0, h, :, j]))
            kf = np.lexsort((np.arange(d.nb), out["loss"][0, h, :, j]))
            assert (ki == kf).all()


# ------------------------------------------------------------------------------------------------
# C4-C5: index map and pools

def test_round_trip_and_map_is_a_bijection():
    d = Dims(b=2, hkv=3, L=256, D=32, B=32, n_p=2, n_sk=3, n_sv=4)
    K = normal((d.b, d.hkv, d.L, d.D), 9)
    V = normal((d.b, d.hkv, d.L, d.D), 10)
    cache = oracle.compress(d, K, V)
    Kt, Vt, vis, keepK, keepV = pinlib.decode_cache(d.b, d.hkv, d.L, d.D, d.B, cache)
    # unpack(pack(X)) = X on kept elements and 0 elsewhere, bit for bit
    assert (Kt == np.where(keepK, K, 0)).all() and (Vt == np.where(keepV, V, 0)).all()
    # dense blocks keep everything, pruned blocks nothing, 2:4 blocks exactly half
    nb = d.nb
    mk = cache["map_k"].reshape(d.b, d.hkv, nb)
    mv = cache["map_v"].reshape(d.b, d.hkv, nb)
    kb = keepK.reshape(d.b, d.hkv, nb, -1).mean(-1)
    vb = keepV.reshape(d.b, d.hkv, nb, -1).mean(-1)
    assert (kb == np.where(mk > 0, 1.0, np.where(mk < 0, 0.5, 0.0))).all()
    assert (vb == np.where(mv > 0, 1.0, np.where(mv < 0, 0.5, 0.0))).all()
    assert ((mk == 0) == (mv == 0)).all() and ((mk == 0).sum(-1) == d.n_p).all()
    # every pool slot is used exactly once, and a head's slots increase with block index
    for m, n_s in ((mk, d.n_sk), (mv, d.n_sv)):
        n_d = nb - d.n_p - n_s
        for bi in range(d.b):
            for h in range(d.hkv):
                head = bi * d.hkv + h
                dense = m[bi, h][m[bi, h] > 0]
                sparse = -m[bi, h][m[bi, h] < 0]
                assert list(dense) == list(range(head * n_d + 1, head * n_d + n_d + 1))
                assert list(sparse) == list(range(head * n_s + 1, head * n_s + n_s + 1))
    # the oracle's own decompression agrees with the test-side decoder
    Kt2, Vt2, vis2 = oracle.unpack(d, cache)
    assert (Kt2 == Kt).all() and (Vt2 == Vt).all() and (vis2 == vis).all()


# ------------------------------------------------------------------------------------------------
# fp16 element type (hso.c R12; [HS] §IV-A computes in fp16)

def f16_normal(shape, seed):
    return synth.f16_bits(np.random.default_rng(seed).standard_normal(shape, dtype=np.float32))


def test_f16_values_match_numpy_for_every_pattern():
    """Attention over one visible token returns that token's V row exactly, so every finite fp16
    pattern passes through the oracle's decoding once and must equal numpy's float16 value."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = bits[(bits & 0x7C00) != 0x7C00]                   # 63488 patterns
    L = -(-len(finite) // 128)
    V = np.zeros(L * 128, np.uint16)
    V[:len(finite)] = finite
    V = V.reshape(1, 1, L, 128)                                 # one token per 128 patterns
    K = np.zeros_like(V)
    Q = np.zeros((1, 1, 1, 128), np.uint16)
    for t in range(L):
        vis = np.zeros((1, 1, L), np.uint8)                     # block size 1: token t alone
        vis[0, 0, t] = 1
        O, _ = oracle.attention(Q, K, V, vis, 1, False, dtype=1)
        assert np.array_equal(O[0], V[0, 0, t].view(np.float16).astype(np.float64)), t


def test_f16_kept_pairs_and_keys_exact():
    d = Dims(b=1, hkv=2, L=64, D=16, B=16, n_p=1, n_sk=1, n_sv=2, dtype=1)
    vals = np.array([0.0, -0.0, 6e-8, -6e-8, 1e-5, 0.5, -0.5, 3.0, 65504.0, -1000.0],
                    np.float32)
    rng = np.random.default_rng(81)
    K = synth.f16_bits(vals[rng.integers(0, len(vals), (1, 2, 64, 16))])
    V = f16_normal((1, 2, 64, 16), 82)
    V[0, 1, 5, 3] = synth.f16_bits(np.float32(6e-8))          # subnormal: key 1
    out = oracle.compress(d, K, V, with_loss=True)
    _, _, _, keepK, keepV = pinlib.decode_cache(1, 2, 64, 16, 16, out)
    for h in range(2):
        want = pinlib.block_keys_exact(K[0, h], V[0, h], 16, 16, dtype=1)
        assert [tuple(int(x) for x in r) for r in out["keys"][0, h]] == want
        keys = [tuple(int(x) for x in r) for r in out["keys"][0, h]]
        mk = out["map_k"].reshape(2, 4)[h]
        mv = out["map_v"].reshape(2, 4)[h]
        wk, wv = pinlib.modes_brute(keys, 1, 1, 2)
        assert [0 if m == 0 else (1 if m > 0 else 2) for m in mk] == wk
        assert [0 if m == 0 else (1 if m > 0 else 2) for m in mv] == wv
        for is_v, X, keep in ((0, K[0, h], keepK[0, h]), (1, V[0, h], keepV[0, h])):
            m = mv if is_v else mk
            for i in range(4):
                if m[i] >= 0:
                    continue
                for row, g, x4 in pinlib.groups_of_block(X, is_v, 16, 16, i):
                    got = (keep[i * 16 + row, 4 * g:4 * g + 4] if not is_v
                           else keep[i * 16 + 4 * g:i * 16 + 4 * g + 4, row])
                    assert tuple(np.flatnonzero(got)) == pinlib.kept_pair_brute(x4, 1)


@pytest.mark.parametrize("causal", [False, True])
def test_f16_sparsity_zero_equals_library_attention(causal):
    B, L, D = 16, 64, 32
    d = Dims(b=1, hkv=2, L=L, D=D, B=B, n_p=0, n_sk=0, n_sv=0, dtype=1)
    K, V = f16_normal((1, 2, L, D), 83), f16_normal((1, 2, L, D), 84)
    Q = f16_normal((1, 4, L, D), 85)
    cache = oracle.compress(d, K, V)
    o, _ = oracle.prefill(d, cache, Q) if causal else oracle.attention(
        Q, *oracle.unpack(d, cache), B, False, dtype=1)
    f = lambda a: torch.from_numpy(a.view(np.float16).astype(np.float64))
    kq = f(K).repeat_interleave(2, dim=1)
    vq = f(V).repeat_interleave(2, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(f(Q), kq, vq, is_causal=causal)
    np.testing.assert_allclose(o.reshape(ref.shape), ref.numpy(), rtol=1e-10, atol=1e-12)


def test_f16_rejects_non_finite():
    d = Dims(b=1, hkv=1, L=16, D=16, B=16, n_p=0, n_sk=1, n_sv=0, dtype=1)
    K = np.zeros((1, 1, 16, 16), np.uint16)
    oracle.compress(d, K, K)
    K[0, 0, 3, 3] = 0x7C00                                       # +inf
    with pytest.raises(ValueError):
        oracle.compress(d, K, np.zeros_like(K))


# ------------------------------------------------------------------------------------------------
# Dense policy of the quality runs ([HS] §V-A): sink and local-window blocks stay dense

@pytest.mark.parametrize("sink,local", [(0, 0), (1, 0), (16, 0), (17, 40), (0, 16), (0, 33),
                                        (48, 48)])
def test_dense_policy_brute_force(sink, local):
    # a block is held when any of its tokens is a sink or local-window token
    held = {i for i in range(8)
            if any(t < sink or t >= 128 - local for t in range(16 * i, 16 * i + 16))}
    r = 8 - len(held)
    n_p = r // 3
    n_sk, n_sv = r - n_p - (r > 3), min(r - n_p, 3)
    d = Dims(b=1, hkv=2, L=128, D=16, B=16, n_p=n_p, n_sk=n_sk, n_sv=n_sv)
    K = tie_heavy((1, 2, 128, 16), 71)
    V = tie_heavy((1, 2, 128, 16), 72)
    got = oracle.compress(d, K, V, sink=sink, local=local)
    mk = got["map_k"].reshape(2, 8)
    mv = got["map_v"].reshape(2, 8)
    for h in range(2):
        keys = pinlib.block_keys_exact(K[0, h], V[0, h], 16, 16)
        want_k, want_v = pinlib.modes_brute(keys, n_p, n_sk, n_sv, held)
        got_k = [0 if m == 0 else (1 if m > 0 else 2) for m in mk[h]]
        got_v = [0 if m == 0 else (1 if m > 0 else 2) for m in mv[h]]
        assert got_k == want_k and got_v == want_v, (h, held)
        assert all(mk[h, i] > 0 and mv[h, i] > 0 for i in held)
    if not held:
        _same_cache(got, oracle.compress(d, K, V))
    # the pools still hold what the modes say
    Kt, Vt, _, keepK, keepV = pinlib.decode_cache(1, 2, 128, 16, 16, got)
    assert (Kt == np.where(keepK, K, 0)).all() and (Vt == np.where(keepV, V, 0)).all()


def test_dense_policy_rejects_counts_that_do_not_fit():
    d = Dims(b=1, hkv=1, L=128, D=16, B=16, n_p=3, n_sk=3, n_sv=0)   # 6 ranked blocks needed
    K = tie_heavy((1, 1, 128, 16), 73)
    oracle.compress(d, K, K, sink=16, local=16)                      # 6 blocks left: fits
    with pytest.raises(ValueError):
        oracle.compress(d, K, K, sink=17, local=16)                  # 5 left
    with pytest.raises(ValueError):
        oracle.compress(d, K, K, sink=-1)


# ------------------------------------------------------------------------------------------------
# Re-compression ([HS] §III, Fig. 3): compress(unpack(cache), counts')

def _same_cache(a, b):
    for k in oracle.POOLS:
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("maker", [tie_heavy, normal])
@pytest.mark.parametrize("counts", [(0, 3, 5), (2, 3, 4), (3, 5, 0), (0, 8, 8), (8, 0, 0)])
def test_recompress_identities(maker, counts):
    d = Dims(b=2, hkv=2, L=256, D=32, B=32, n_p=0, n_sk=0, n_sv=0)
    K = maker((d.b, d.hkv, d.L, d.D), 21)
    V = maker((d.b, d.hkv, d.L, d.D), 22)
    dc = Dims(d.b, d.hkv, d.L, d.D, d.B, *counts)
    want = oracle.compress(dc, K, V)
    # an all-dense cache holds every value: re-compressing it is compressing from scratch
    _same_cache(oracle.recompress(d, oracle.compress(d, K, V), dc), want)
    # a 2:4 or pruned block has zero loss for its own mode, so the same counts change nothing
    _same_cache(oracle.recompress(dc, want, dc), want)
    # the prefill-to-decode phase change (one tensor 2:4 first, then both) loses nothing against
    # compressing the original values with the decode counts
    n_p, n_sk, n_sv = counts
    for first in ((n_p, 0, n_sv), (n_p, n_sk, 0)):
        d1 = Dims(d.b, d.hkv, d.L, d.D, d.B, *first)
        _same_cache(oracle.recompress(d1, oracle.compress(d1, K, V), dc), want)
    # towards dense nothing is recovered: the cache stands for the same tensors as before
    d0 = Dims(d.b, d.hkv, d.L, d.D, d.B, n_p, 0, 0)
    back = oracle.recompress(dc, want, d0)
    Kt, Vt, vis, _, _ = pinlib.decode_cache(d.b, d.hkv, d.L, d.D, d.B, want)
    Kt0, Vt0, vis0, keepK0, keepV0 = pinlib.decode_cache(d.b, d.hkv, d.L, d.D, d.B, back)
    assert (Kt0 == Kt).all() and (Vt0 == Vt).all() and (vis0 == vis).all()
    assert (back["map_k"] >= 0).all() and (back["map_v"] >= 0).all()


def test_recompress_changes_modes_by_the_held_values():
    # a block whose 2:4 loss was high in the original still ranks by what the cache holds
    d = Dims(b=1, hkv=1, L=128, D=16, B=16, n_p=0, n_sk=0, n_sv=0)
    K = normal((1, 1, d.L, d.D), 31)
    V = normal((1, 1, d.L, d.D), 32)
    K[..., 16:32, :] = synth.bf16_bits(np.float32(40.0) * np.ones((16, 16), np.float32))
    d_first = Dims(1, 1, d.L, d.D, d.B, 0, 3, 0)
    first = oracle.compress(d_first, K, V)
    # block 1 holds large equal values: its K 2:4 loss is the largest, so it stays dense
    assert first["map_k"][1] > 0
    again = oracle.recompress(d_first, first, Dims(1, 1, d.L, d.D, d.B, 0, 4, 0))
    # the three 2:4 blocks keep their mode (zero loss) and one more is chosen among the rest
    assert ((first["map_k"] < 0) <= (again["map_k"] < 0)).all() and (again["map_k"] < 0).sum() == 4


# ------------------------------------------------------------------------------------------------
# Compression with caller masks ([HS] §III-A cache pruner, §IV-B generic kernel)

def modes_of(d, cache):
    """Block modes (0 pruned, 1 dense, 2 2:4) read off a compressed cache's maps."""
    out = []
    for m in (cache["map_k"], cache["map_v"]):
        m = np.asarray(m).reshape(d.b, d.hkv, d.nb)
        out.append(np.where(m == 0, 0, np.where(m > 0, 1, 2)).astype(np.uint8))
    return out


@pytest.mark.parametrize("maker", [tie_heavy, normal])
@pytest.mark.parametrize("counts", [(0, 3, 5), (2, 3, 4), (3, 5, 0), (0, 8, 8), (8, 0, 0)])
def test_masked_reproduces_the_magnitude_compressor(maker, counts):
    d = Dims(2, 2, 256, 32, 32, *counts)
    K = maker((d.b, d.hkv, d.L, d.D), 41)
    V = maker((d.b, d.hkv, d.L, d.D), 42)
    want = oracle.compress(d, K, V)
    mk, mv = modes_of(d, want)
    # fed the magnitude compressor's own block modes and its masked (unpacked) values, the
    # generic path writes the same cache: the non-zeros of a thinned group are its top two
    Kt, Vt, _ = oracle.unpack(d, want)
    got = oracle.compress_masked(d, Kt, Vt, mk, mv)
    assert not got["head_status"].any()
    _same_cache(got, want)
    # unmasked input: groups with more than two non-zeros fall back to the top-2 rule
    _same_cache(oracle.compress_masked(d, K, V, mk, mv), want)


def test_masked_element_rule_brute_force():
    """Every group over {+0, -0, 1, -2} (256 of them), stored by the generic kernel's rule: the
    non-zeros padded with the lowest zero positions, or the top-2 pair when more than two."""
    vals = np.array([0x0000, 0x8000, 0x3F80, 0xC000], np.uint16)
    groups = np.array(list(itertools.product(range(4), repeat=4)))
    X4 = vals[groups]                                              # [256][4]
    blockK = X4.reshape(64, 16)                                    # 64 tokens x 4 groups
    K = np.zeros((1, 1, 64, 16), np.uint16)
    K[0, 0] = blockK
    V = np.zeros((1, 1, 64, 16), np.uint16)
    V[0, 0] = X4.reshape(16, 64).T            # channel c, token group g holds group 16 c + g
    d = Dims(1, 1, 64, 16, 64, 0, 1, 1)
    two = np.full((1, 1, 1), 2, np.uint8)
    got = oracle.compress_masked(d, K, V, two, two)
    _, _, _, keepK, keepV = pinlib.decode_cache(1, 1, 64, 16, 64, got)

    def expected(x4):
        nz = [j for j in range(4) if x4[j] & 0x7FFF]
        if len(nz) > 2:
            return set(pinlib.kept_pair_brute(x4))
        return set(nz) | set([j for j in range(4) if not x4[j] & 0x7FFF][:2 - len(nz)])

    kk = keepK[0, 0].reshape(64, 4, 4)
    vv = keepV[0, 0].T.reshape(16, 16, 4)
    for n, x4 in enumerate(X4):
        want = expected(x4)
        assert set(np.flatnonzero(kk[n // 4, n % 4])) == want, x4
    Vg = V[0, 0].T.reshape(16, 16, 4)
    for c in range(16):
        for g in range(16):
            assert set(np.flatnonzero(vv[c, g])) == expected(Vg[c, g]), Vg[c, g]


def test_masked_channel_mask_closed_form():
    """A channel mask (K keeps channels 4g, 4g+1 of every group; V keeps tokens 4g, 4g+2): every
    K metadata word is 0x4444 (positions 0 and 1 in each nibble), every V word 0x8888 (0, 2),
    and the kept values are the unmasked ones in order."""
    d = Dims(1, 2, 128, 32, 32, 0, 4, 4)
    K = normal((1, 2, 128, 32), 51)
    V = normal((1, 2, 128, 32), 52)
    K[..., 2::4] = 0
    K[..., 3::4] = 0
    V[:, :, 1::4] = 0
    V[:, :, 3::4] = 0
    two = np.full((1, 2, 4), 2, np.uint8)
    got = oracle.compress_masked(d, K, V, two, two)
    assert (got["k_meta"] == 0x4444).all() and (got["v_meta"] == 0x8888).all()
    kn = got["k_nnz"].reshape(2, 4, 32, 8, 2)                      # [head][block][token][group][2]
    want_k = K[0].reshape(2, 4, 32, 8, 4)[..., :2]
    assert (kn == want_k).all()
    vn = got["v_nnz"].reshape(2, 4, 32, 8, 2)                      # [head][block][chan][group][2]
    want_v = V[0].reshape(2, 4, 32, 32).transpose(0, 1, 3, 2).reshape(2, 4, 32, 8, 4)[..., [0, 2]]
    assert (vn == want_v).all()


def test_masked_rejects_heads_whose_modes_do_not_fit():
    d = Dims(2, 3, 256, 32, 32, 2, 3, 4)
    K = normal((2, 3, 256, 32), 61)
    V = normal((2, 3, 256, 32), 62)
    mk, mv = synth.random_modes(63, 2, 3, 8, 2, 3, 4)
    good = oracle.compress_masked(d, K, V, mk, mv)
    assert not good["head_status"].any()
    bk, bv = mk.copy(), mv.copy()
    bk[0, 1, np.flatnonzero(bk[0, 1] == 1)[0]] = 3                 # a byte above 2 (counts of 0
                                                                   # and 2 unchanged)
    i = np.flatnonzero(bk[1, 0] == 0)[0]
    bk[1, 0, i] = 1                                                # K kept where V pruned: 2 | 4
    j = np.flatnonzero(bv[1, 2] == 1)[0]
    bv[1, 2, j] = 2                                                # one 2:4 V block too many
    got = oracle.compress_masked(d, K, V, bk, bv)
    st = got["head_status"]
    assert st[0, 1] == 1 and st[1, 0] == 2 | 4 and st[1, 2] == 4
    assert st[0, 0] == st[0, 2] == st[1, 1] == 0
    for m in ("map_k", "map_v"):
        gm, wm = got[m].reshape(2, 3, 8), good[m].reshape(2, 3, 8)
        ok = st == 0
        assert (gm[~ok] == 0).all() and (gm[ok] == wm[ok]).all()
    # accepted heads' pool slots are written exactly as before; rejected ones are left zero
    Kt, Vt, _, _, _ = pinlib.decode_cache(2, 3, 256, 32, 32, got)
    Kg, Vg, _, _, _ = pinlib.decode_cache(2, 3, 256, 32, 32, good)
    ok = (st == 0)[..., None, None]
    assert (np.where(ok, Kt, 0) == np.where(ok, Kg, 0)).all()
    assert (np.where(ok, Vt, 0) == np.where(ok, Vg, 0)).all()


def test_rejects_out_of_range_inputs():
    d = Dims(b=1, hkv=1, L=16, D=16, B=16, n_p=0, n_sk=1, n_sv=0)
    K = np.zeros((1, 1, 16, 16), np.uint16)
    V = K.copy()
    K[0, 0, 3, 3] = synth.bf16_bits(np.float32(2.0 ** 24))
    with pytest.raises(ValueError):
        oracle.compress(d, K, V)
    K[0, 0, 3, 3] = 0x7F80  # +inf
    with pytest.raises(ValueError):
        oracle.compress(d, K, V)
    with pytest.raises(ValueError):
        oracle.compress(Dims(1, 1, 16, 16, 16, 1, 1, 0), K * 0, V)   # n_p + n_sk > nb


# ------------------------------------------------------------------------------------------------
# Sizes: Eq. (4)-(6), Table V

def _bytes_no_prune(L, D, B, n_sk, n_sv):
    return oracle.pool_bytes(Dims(1, 1, L, D, B, 0, n_sk, n_sv))


@pytest.mark.parametrize("L,B,SK,SV", [(4096, 64, 0.5, 1.0), (4096, 64, 1.0, 1.0),
                                       (8192, 128, 0.25, 0.75), (2048, 16, 0.0, 1.0)])
def test_byte_count_equals_closed_form(L, B, SK, SV):
    D = 128
    nb = L // B
    n_sk, n_sv = int(SK * nb), int(SV * nb)
    got = _bytes_no_prune(L, D, B, n_sk, n_sv)
    e = 2  # bytes per element
    size_den = e * (L * D * (1 - SK) + L * D * (1 - SV))        # Eq. (5b)
    size_nnz = e * (0.5 * L * D * SK + 0.5 * L * D * SV)         # Eq. (5c)
    size_e = e * (L * D * SK / 16 + L * D * SV / 16)             # Eq. (5d)
    size_idx = 4 * 2 * L / B                                      # Eq. (5a), int32 entries
    assert got["k_dense"] + got["v_dense"] == size_den
    assert got["k_nnz"] + got["v_nnz"] == size_nnz
    assert got["k_meta"] + got["v_meta"] == size_e
    assert got["map_k"] + got["map_v"] == size_idx


def test_eq6_worked_compression_ratios():
    g = json.load(open(GOLDEN))["compression_ratio_eq6"]
    L, D, B = 32768, 128, 64
    nb = L // B
    for case in g["cases"]:
        got = _bytes_no_prune(L, D, B, int(case["S_K"] * nb), int(case["S_V"] * nb))
        r = 2 * L * D * 2 / sum(got.values())                    # Eq. (3)-(4)
        assert f"{r:.2f}" == f"{case['r_comp']:.2f}"


def test_table_v_memory_column():
    g = json.load(open(GOLDEN))["table_v_key_value_memory_gib"]
    for row in g["rows"]:
        L = row["context"]
        per_head = _bytes_no_prune(L, g["head_dim"], 64, L // 64, 0)
        scale = g["layers"] * g["kv_heads"] / 2 ** 30
        dense = per_head["v_dense"] * scale
        sparse = (per_head["k_nnz"] + per_head["k_meta"]) * scale
        assert f"{dense:.2f}" == f"{row['dense']:.2f}"
        assert f"{sparse:.2f}" == f"{row['sparse_S1']:.2f}"


# ------------------------------------------------------------------------------------------------
# C7-C8: attention (Eq. 1)

def _sdpa(q, k, v, causal, G):
    q = torch.from_numpy(synth.bf16_to_f32(q).astype(np.float64))
    k = torch.from_numpy(synth.bf16_to_f32(k).astype(np.float64)).repeat_interleave(G, dim=1)
    v = torch.from_numpy(synth.bf16_to_f32(v).astype(np.float64)).repeat_interleave(G, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal).numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_sparsity_zero_equals_library_attention(causal):
    d = Dims(b=2, hkv=2, L=128, D=32, B=16, n_p=0, n_sk=0, n_sv=0)
    hq = 8
    K = normal((d.b, d.hkv, d.L, d.D), 11)
    V = normal((d.b, d.hkv, d.L, d.D), 12)
    cache = oracle.compress(d, K, V)
    lq = d.L if causal else 1
    Q = normal((d.b, hq, lq, d.D), 13)
    if causal:
        O, _ = oracle.prefill(d, cache, Q)
    else:
        O, _ = oracle.decode(d, cache, Q, hq)
    want = _sdpa(Q, K, V, causal, hq // d.hkv)
    np.testing.assert_allclose(O.reshape(want.shape), want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("counts", [(0, 2, 2), (1, 1, 0), (1, 0, 1)])
def test_brute_force_tiny_heads(causal, counts):
    d = Dims(b=1, hkv=1, L=32, D=16, B=16, n_p=counts[0], n_sk=counts[1], n_sv=counts[2])
    hq = 2
    K = normal((1, 1, d.L, d.D), 14)
    V = normal((1, 1, d.L, d.D), 15)
    cache = oracle.compress(d, K, V)
    Kt, Vt, vis, _, _ = pinlib.decode_cache(1, 1, d.L, d.D, d.B, cache)
    Q = normal((1, hq, d.L if causal else 1, d.D), 16)
    want, want_lse = pinlib.attention_full_matrix(Q, Kt, Vt, vis, d.B, causal)
    if causal:
        O, lse = oracle.prefill(d, cache, Q)
    else:
        O, lse = oracle.decode(d, cache, Q, hq)
    np.testing.assert_allclose(O.reshape(want.shape), want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse.reshape(want_lse.shape), want_lse, rtol=0, atol=1e-12)


def test_special_cases():
    D, B, L = 16, 16, 64
    d = Dims(1, 1, L, D, B, 0, 0, 0)
    K = normal((1, 1, L, D), 17)
    row = normal((D,), 18)
    V = np.broadcast_to(row, (1, 1, L, D)).copy()
    cache = oracle.compress(d, K, V)
    # all value rows equal -> the output is that row
    O, _ = oracle.decode(d, cache, normal((1, 1, D), 19), 1)
    np.testing.assert_allclose(O[0], synth.bf16_to_f32(row), atol=1e-12)
    # q = 0 -> uniform weights -> mean of the visible value rows
    d2 = Dims(1, 1, L, D, B, 1, 1, 1)
    V2 = normal((1, 1, L, D), 20)
    cache2 = oracle.compress(d2, K, V2)
    Kt, Vt, vis, _, _ = pinlib.decode_cache(1, 1, L, D, B, cache2)
    O, lse = oracle.decode(d2, cache2, np.zeros((1, 1, D), np.uint16), 1)
    tok = np.repeat(vis[0, 0].astype(bool), B)
    np.testing.assert_allclose(O[0], synth.bf16_to_f32(Vt[0, 0][tok]).astype(np.float64).mean(0),
                               atol=1e-12)
    assert abs(lse[0] - math.log(tok.sum())) < 1e-12
    # a single visible token -> its value row (prefill row 0 sees only token 0)
    O, lse = oracle.prefill(d, cache, normal((1, 1, L, D), 21), rows=[0])
    np.testing.assert_allclose(O[0], synth.bf16_to_f32(V[0, 0, 0]), atol=1e-12)
    # everything pruned -> zero output, lse = -inf
    d3 = Dims(1, 1, L, D, B, L // B, 0, 0)
    cache3 = oracle.compress(d3, K, V2)
    O, lse = oracle.decode(d3, cache3, normal((1, 1, D), 22), 1)
    assert (O == 0).all() and np.isneginf(lse).all()
    O, lse = oracle.prefill(d3, cache3, normal((1, 1, L, D), 23))
    assert (O == 0).all() and np.isneginf(lse).all()


def test_dropped_mass_identity():
    """Dropping tokens of softmax mass eps moves the output by exactly eps * (o_dropped - o_kept)
    (Jet-QSparse, arXiv 2611.01022, §3.4 'Effect of omitted mass', Eq. 5), and by at most eps times
    the diameter of the value set."""
    D, B, L, hq = 32, 16, 256, 4
    K = normal((1, 2, L, D), 24)
    V = normal((1, 2, L, D), 25)
    Q = normal((1, hq, 1, D), 26)
    nb = L // B
    kept = np.zeros((1, 2, nb), np.uint8)
    kept[..., ::3] = 1
    kept[..., 5] = 1
    allv = np.ones_like(kept)
    o_all, lse_all = oracle.attention(Q, K, V, allv, B, False)
    o_kept, _ = oracle.attention(Q, K, V, kept, B, False)
    o_drop, lse_drop = oracle.attention(Q, K, V, 1 - kept, B, False)
    eps = np.exp(lse_drop - lse_all)[:, None]
    np.testing.assert_allclose(o_all - o_kept, eps * (o_drop - o_kept), atol=1e-12)
    vv = synth.bf16_to_f32(V).astype(np.float64)
    for r in range(hq):
        vals = vv[0, r // 2]
        diam = max(np.linalg.norm(vals[i] - vals[j]) for i in range(0, L, 7) for j in range(L))
        assert np.linalg.norm(o_all[r] - o_kept[r]) <= eps[r, 0] * diam + 1e-12
    # and the compressed cache's pruned blocks behave exactly as those dropped tokens
    d = Dims(1, 2, L, D, B, 6, 0, 0)
    cache = oracle.compress(d, K, V)
    vis = (cache["map_k"].reshape(1, 2, nb) != 0).astype(np.uint8)
    o_c, _ = oracle.decode(d, cache, Q, hq)
    o_v, _ = oracle.attention(Q, K, V, vis, B, False)
    np.testing.assert_allclose(o_c, o_v, atol=1e-15)


def test_split_merge_by_log_sum_exp():
    """Partial outputs over a partition of the visible blocks, merged by their log-sum-exp, equal
    the unsplit result (the combine step of the split-KV decode)."""
    D, B, L, hq = 32, 16, 512, 4
    K = normal((2, 1, L, D), 27)
    V = normal((2, 1, L, D), 28)
    Q = normal((2, hq, 1, D), 29)
    nb = L // B
    vis = np.ones((2, 1, nb), np.uint8)
    vis[..., 3] = 0
    o_full, lse_full = oracle.attention(Q, K, V, vis, B, False)
    parts = []
    for s in range(5):
        m = np.zeros_like(vis)
        m[..., s::5] = vis[..., s::5]
        parts.append(oracle.attention(Q, K, V, m, B, False))
    lses = np.stack([p[1] for p in parts])
    mstar = lses.max(0)
    w = np.exp(lses - mstar)
    o = sum(w[i][:, None] * parts[i][0] for i in range(5)) / w.sum(0)[:, None]
    np.testing.assert_allclose(o, o_full, atol=1e-12)
    np.testing.assert_allclose(mstar + np.log(w.sum(0)), lse_full, atol=1e-12)


def test_gqa_mapping():
    D, B, L = 32, 16, 128
    K = normal((1, 2, L, D), 30)
    V = normal((1, 2, L, D), 31)
    Q = normal((1, 8, 1, D), 32)
    vis = np.ones((1, 2, L // B), np.uint8)
    o, _ = oracle.attention(Q, K, V, vis, B, False)
    # G = 4: query head h reads KV head h // 4, i.e. replicating KV heads gives the same result
    Kr, Vr = np.repeat(K, 4, axis=1), np.repeat(V, 4, axis=1)
    o_rep, _ = oracle.attention(Q, Kr, Vr, np.ones((1, 8, L // B), np.uint8), B, False)
    np.testing.assert_allclose(o, o_rep, atol=0)
    # G = 1 equals running each head on its own
    for h in range(8):
        oh, _ = oracle.attention(Q[:, h:h + 1], Kr[:, h:h + 1], Vr[:, h:h + 1],
                                 np.ones((1, 1, L // B), np.uint8), B, False)
        np.testing.assert_allclose(oh[0], o_rep[h], atol=0)
