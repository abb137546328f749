"""Pins of the benchmark's work model (no GPU): the executed-flop count behind the reported MFMA
utilisation and ideal prefill speedup reproduces HieraSparse §III-D2 Eq. (10) and its worked values
(§III-D3: 1.6x at S_K = 0.5, S_V = 1; 2.0x at S_K = S_V = 1), and the decode byte count reproduces
Eq. (11) (the compression ratio of §III-D1 Eq. (6))."""
import json
import os

import numpy as np
import pytest

import bench
from sparse_kv_cache_magnitude_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hierasparse_worked_values.json")


def _maps(nb, sparse_k, sparse_v, pruned=()):
    """Index maps of one head with the given 2:4 (negative) and pruned (0) block sets."""
    mk = np.array([0 if i in pruned else (-(i + 1) if i in sparse_k else i + 1)
                   for i in range(nb)], np.int32)
    mv = np.array([0 if i in pruned else (-(i + 1) if i in sparse_v else i + 1)
                   for i in range(nb)], np.int32)
    return mk, mv


def _workload(nb, B=64):
    return synth.Workload("pin", "prefill", 1, 1, 1, 128, nb * B, B, 0, 0, 0, 0)


def test_prefill_speedup_eq10_worked_values():
    """Eq. (10) is written for full (non-causal) attention, where every block carries the same
    work. Under the causal mask block i carries work linear in i, so a block set carries exactly
    half of it when it is made of whole mirror pairs (i, nb - 1 - i); with such a set as the 2:4 K
    blocks (S_K = 0.5) and every V block 2:4 (S_V = 1), the causal ratio equals Eq. (10)'s."""
    cases = json.load(open(GOLDEN))["prefill_speedup_eq10"]["cases"]
    nb = 8
    w = _workload(nb)
    for case in cases:
        S_K, S_V = case["S_K"], case["S_V"]
        n_k = int(round(S_K * nb))
        sparse_k = set()
        for i in range(n_k // 2):
            sparse_k |= {i, nb - 1 - i}
        sparse_v = set(range(int(round(S_V * nb))))
        assert len(sparse_k) == n_k
        mk, mv = _maps(nb, sparse_k, sparse_v)
        dense_eq, executed, full = bench.prefill_flops(w, mk, mv, smfmac=True)
        assert dense_eq == pytest.approx(full, rel=1e-15)          # nothing pruned
        eq10 = 4.0 / (4.0 - (S_K + S_V))
        assert full / executed == pytest.approx(eq10, rel=1e-12)
        assert round(eq10, 1) == case["speedup"]                   # the printed value
        # the decompress path executes every flop densely
        _, executed_d, _ = bench.prefill_flops(w, mk, mv, smfmac=False)
        assert executed_d == pytest.approx(full, rel=1e-15)


def test_prefill_flops_closed_form():
    """Dense-equivalent causal work: 4 D flops per (query, key <= query) pair with the key's block
    not pruned, for every query head; brute force over all pairs of a small shape."""
    nb, B = 5, 64
    w = synth.Workload("pin", "prefill", 2, 8, 2, 128, nb * B, B, 0, 0, 0, 0)
    rng = np.random.default_rng(3)
    maps_k, maps_v = [], []
    for _ in range(w.b * w.hkv):
        pruned = set(rng.choice(nb, 1, replace=False).tolist())
        mk, mv = _maps(nb, set(rng.choice(nb, 2, replace=False).tolist()),
                       set(rng.choice(nb, 3, replace=False).tolist()), pruned)
        maps_k.append(mk)
        maps_v.append(mv)
    mk, mv = np.stack(maps_k), np.stack(maps_v)
    dense_eq, executed, _ = bench.prefill_flops(w, mk, mv, smfmac=True)
    G = w.hq // w.hkv
    want_eq = want_ex = 0.0
    for h in range(w.b * w.hkv):
        for q in range(w.L):
            for k in range(q + 1):
                i = k // B
                if mk[h, i] == 0:
                    continue
                want_eq += 4 * w.D * G
                want_ex += 2 * w.D * G * ((0.5 if mk[h, i] < 0 else 1.0)
                                          + (0.5 if mv[h, i] < 0 else 1.0))
    assert dense_eq == pytest.approx(want_eq, rel=1e-12)
    assert executed == pytest.approx(want_ex, rel=1e-12)


@pytest.mark.parametrize("S_K,S_V", [(0.5, 1.0), (1.0, 1.0), (0.25, 0.75)])
def test_decode_bytes_eq11(S_K, S_V):
    """The K/V part of the decode's algorithmic bytes gives Eq. (11)'s ratio exactly (the index
    maps and q/o, which the benchmark also counts, are subtracted here)."""
    nb = 512
    w0 = synth.Workload("pin", "decode", 2, 8, 2, 128, nb * 64, 64, 0, 0, 0, 0)
    w = w0.with_counts(0, int(S_K * nb), int(S_V * nb))
    G = w.hq // w.hkv
    extra = (2 * 4 * nb + 2 * G * w.D * 2) * w.b * w.hkv
    r = (bench.decode_bytes(w0, G) - extra) / (bench.decode_bytes(w, G) - extra)
    assert r == pytest.approx(1.0 / (1.0 - 0.21875 * (S_K + S_V)), rel=1e-12)
