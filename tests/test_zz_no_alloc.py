"""GPU check of hs_decode_attn_noalloc (the decode entry point that allocates nothing and keeps its
splits' partials in the library's fixed device array) through the C ABI: on calls in a row, the
second with a smaller input, its output and log-sum-exp equal those of hs_decode_attn with a
caller workspace bit for bit (same kernels, same split count)."""
import numpy as np
import pytest
import torch

from sparse_kv_cache_magnitude_amd import hierasparse as hs
from sparse_kv_cache_magnitude_amd import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# (batch, q_heads, kv_heads, tokens, block, counts, splits): calls in this order
CASES = [(4, 32, 8, 64 * 48, 64, (6, 24, 20), 0),    # larger first call
         (2, 8, 2, 128 * 9, 128, (1, 4, 3), 0),      # smaller second call
         (1, 40, 2, 64 * 11, 64, (2, 5, 3), 7),      # G = 20: two column groups, fixed splits
         (2, 8, 2, 64 * 6, 64, (1, 2, 3), 1)]        # one split: no combine launch


def _decode_both(case, rng):
    b, hq, hkv, L, B, counts, splits = case
    K = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    V = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    q = synth.bf16_bits(rng.standard_normal((b, hq, 1, 128), dtype=np.float32))
    shp, cnt = hs.shape(b, hq, hkv, L, 128, B), hs.counts(*counts)
    cache = gu.gpu_compress(shp, cnt, gu.to_dev(K), gu.to_dev(V))
    qd = gu.to_dev(q)
    o_ws = torch.empty((b, hq, 128), dtype=torch.int16, device="cuda")
    l_ws = torch.empty((b, hq), dtype=torch.float32, device="cuda")
    ws = hs.alloc_workspace(hs.HS_OP_DECODE, shp, cnt, splits)
    hs.hs_decode_attn(shp, cnt, cache, qd, o_ws, l_ws, 0.0, splits, ws)
    o_na = torch.full((b, hq, 128), -1, dtype=torch.int16, device="cuda")
    l_na = torch.full((b, hq), float("nan"), dtype=torch.float32, device="cuda")
    hs.hs_decode_attn_noalloc(shp, cnt, cache, qd, o_na, l_na, 0.0, splits)
    torch.cuda.synchronize()
    return o_ws.cpu().numpy(), l_ws.cpu().numpy(), o_na.cpu().numpy(), l_na.cpu().numpy()


def test_noalloc_decode_matches_workspace_decode():
    rng = np.random.default_rng(77)
    for case in CASES + CASES[:1]:
        print(f"[noalloc] {case}", flush=True)
        o_ws, l_ws, o_na, l_na = _decode_both(case, rng)
        assert np.array_equal(o_ws, o_na), case
        assert np.array_equal(l_ws.view(np.uint32), l_na.view(np.uint32)), case
