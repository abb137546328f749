"""GPU compression with caller masks (hs_compress_masked) against the oracle: head status, maps
and all six pools bit-exact. Output pools start zeroed on both sides (a rejected head's slots are
left as they were)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import Dims
from sparse_kv_cache_magnitude_amd import hierasparse as hs
from sparse_kv_cache_magnitude_amd import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _run(b, hkv, L, B, counts, K, V, mk, mv, with_status=True, hq=None):
    hq = hq or hkv
    shp, cnt = hs.shape(b, hq, hkv, L, 128, B), hs.counts(*counts)
    print(f"[masked] b={b} hkv={hkv} L={L} B={B} counts={counts}", flush=True)
    cache = {f: t.zero_() for f, t in hs.alloc_cache(shp, cnt).items()}
    status = torch.full((b * hkv,), -1, dtype=torch.int32, device="cuda") if with_status else None
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    hs.hs_compress_masked(shp, cnt, gu.to_dev(K), gu.to_dev(V), dev(mk), dev(mv), cache, status)
    torch.cuda.synchronize()
    want = oracle.compress_masked(Dims(b, hkv, L, 128, B, *counts), K, V, mk, mv)
    gu.compare_cache(gu.cache_to_numpy(cache), want)
    if with_status:
        assert np.array_equal(status.cpu().numpy().reshape(b, hkv), want["head_status"])
    return want


def _normal(seed, shape, scale=1.0):
    rng = np.random.default_rng(seed)
    return synth.bf16_bits(rng.standard_normal(shape, dtype=np.float32) * scale)


@pytest.mark.parametrize("B", [64, 128])
@pytest.mark.parametrize("counts_fn", [
    lambda nb: (0, 0, 0),
    lambda nb: (0, nb, nb),
    lambda nb: (nb, 0, 0),
    lambda nb: (2, 3, 5),
    lambda nb: (1, nb - 1, 0),
])
def test_masked_random_masks(B, counts_fn):
    b, hkv, L = 3, 2, 9 * B
    nb = L // B
    counts = counts_fn(nb)
    mk, mv = synth.random_modes(B + 7, b, hkv, nb, *counts)
    K = synth.random_element_mask(B + 8, _normal(B + 1, (b, hkv, L, 128)), mk, B, False)
    V = synth.random_element_mask(B + 9, _normal(B + 2, (b, hkv, L, 128), 3), mv, B, True)
    want = _run(b, hkv, L, B, counts, K, V, mk, mv)
    assert not want["head_status"].any()


def test_masked_thinned_groups_and_unmasked_fallback():
    """Groups with one or no non-zero (padding with the lowest zero positions), -0 values, and an
    unmasked tensor whose 2:4 groups fall back to the top-2 rule."""
    b, hkv, L, B = 2, 2, 6 * 64, 64
    mk, mv = synth.random_modes(21, b, hkv, 6, 1, 3, 4)
    K = synth.random_element_mask(22, _normal(23, (b, hkv, L, 128)), mk, B, False, keep=1)
    V = synth.random_element_mask(24, _normal(25, (b, hkv, L, 128)), mv, B, True, keep=0)
    K[0, 0, :64, ::7] = 0x8000
    _run(b, hkv, L, B, (1, 3, 4), K, V, mk, mv)
    _run(b, hkv, L, B, (1, 3, 4), _normal(26, (b, hkv, L, 128)), _normal(27, (b, hkv, L, 128)),
         mk, mv, with_status=False)


def test_masked_rejected_heads():
    b, hkv, L, B = 2, 3, 8 * 64, 64
    counts = (2, 3, 4)
    mk, mv = synth.random_modes(31, b, hkv, 8, *counts)
    mk[0, 1, np.flatnonzero(mk[0, 1] == 1)[0]] = 7
    mk[1, 0, np.flatnonzero(mk[1, 0] == 0)[0]] = 2
    mv[1, 2, np.flatnonzero(mv[1, 2] == 1)[0]] = 0
    K, V = _normal(32, (b, hkv, L, 128)), _normal(33, (b, hkv, L, 128))
    want = _run(b, hkv, L, B, counts, K, V, mk, mv)
    st = want["head_status"]
    assert st[0, 1] and st[1, 0] and st[1, 2] and not st[0, 0] and not st[1, 1]


def test_masked_workload_size():
    """The 32K batch-8 cache shape with random block masks at its counts and random 2:4 element
    masks in the 2:4 blocks."""
    w = synth.workload("decode_llama8b_32k_b8")
    K, V = gu.workload_kv(w.name)
    mk, mv = synth.random_modes(41, w.b, w.hkv, w.nb, *w.counts())
    K = synth.random_element_mask(42, K, mk, w.B, False)
    V = synth.random_element_mask(43, V, mv, w.B, True)
    want = _run(w.b, w.hkv, w.L, w.B, w.counts(), K, V, mk, mv, hq=w.hq)
    assert not want["head_status"].any()
