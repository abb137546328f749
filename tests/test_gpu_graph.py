"""The decode and prefill entry points inside a captured HIP graph (torch.cuda.CUDAGraph on ROCm):
every replay, with eager work and synchronisations between replays, gives the eager result bit
for bit. The library issues no memset and allocates nothing, and the decode's workspace needs no
contents (each call writes the partials it reads), so a captured call can be replayed as is."""
import numpy as np
import pytest
import torch

from sparse_kv_cache_magnitude_amd import hierasparse as hs
from sparse_kv_cache_magnitude_amd import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _setup(b, hq, hkv, L, B, counts, seed):
    rng = np.random.default_rng(seed)
    K = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    V = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    shp, cnt = hs.shape(b, hq, hkv, L, 128, B), hs.counts(*counts)
    cache = gu.gpu_compress(shp, cnt, gu.to_dev(K), gu.to_dev(V))
    return rng, shp, cnt, cache


def test_decode_graph_replays():
    rng, shp, cnt, cache = _setup(2, 8, 2, 64 * 40, 64, (6, 20, 14), 1)
    q = gu.to_dev(synth.bf16_bits(rng.standard_normal((2, 8, 1, 128), dtype=np.float32)))
    ws = hs.alloc_workspace(hs.HS_OP_DECODE, shp, cnt)
    o = torch.empty((2, 8, 128), dtype=torch.int16, device="cuda")
    lse = torch.empty((2, 8), dtype=torch.float32, device="cuda")
    hs.hs_decode_attn(shp, cnt, cache, q, o, lse, 0.0, 0, ws)
    torch.cuda.synchronize()
    want_o, want_lse = o.clone(), lse.clone()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            hs.hs_decode_attn(shp, cnt, cache, q, o, lse, 0.0, 0, ws)
    torch.cuda.current_stream().wait_stream(s)
    for r in range(4):
        o.fill_(0)
        lse.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph decode] replay {r}", flush=True)
        assert torch.equal(o, want_o) and torch.equal(lse, want_lse), r
        # eager work between replays, on the same workspace
        hs.hs_decode_attn(shp, cnt, cache, q, o, lse, 0.0, 0, ws)
        torch.cuda.synchronize()
        assert torch.equal(o, want_o)


def test_prefill_graph_replays():
    rng, shp, cnt, cache = _setup(1, 8, 2, 64 * 12, 64, (2, 6, 5), 2)
    Q = gu.to_dev(synth.bf16_bits(rng.standard_normal((1, 8, 64 * 12, 128), dtype=np.float32)))
    O = torch.empty_like(Q)
    lse = torch.empty((1, 8, 64 * 12), dtype=torch.float32, device="cuda")
    hs.hs_prefill_attn(shp, cnt, cache, Q, O, lse, 0.0, hs.HS_PREFILL_SMFMAC)
    torch.cuda.synchronize()
    want_o, want_lse = O.clone(), lse.clone()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            hs.hs_prefill_attn(shp, cnt, cache, Q, O, lse, 0.0, hs.HS_PREFILL_SMFMAC)
    torch.cuda.current_stream().wait_stream(s)
    for r in range(3):
        O.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph prefill] replay {r}", flush=True)
        assert torch.equal(O, want_o) and torch.equal(lse, want_lse), r
