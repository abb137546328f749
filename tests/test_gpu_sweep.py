"""The sparsity sweep at full size against the oracle (HieraSparse §V-B1, Fig. 8a: 0%, 50% all
2:4, 62.5% and 75% with the extra sparsity from pruned blocks), in the launch configurations the
benchmark times:
  - decode and compressor at 64K context, batch 16, 32/8 heads: every pool and map bit-exact, and
    the whole decode output within the attention gate;
  - causal prefill at 32K, batch 1, on the SMFMAC path, on sampled query rows (the wave- and
    key-tile edges near both ends of every head and four random rows per head).
Inputs come from the benchmark's own seeded device generator (synth.make_inputs_device) and are
copied to the host for the oracle."""
import numpy as np
import pytest
import torch

import oracle
from oracle import Dims
from sparse_kv_cache_magnitude_amd import hierasparse as hs
from sparse_kv_cache_magnitude_amd import synth
from tests import gpu_util as gu
from tests.test_gpu_decode import assert_close
from tests.test_gpu_prefill import sample_rows

pytestmark = pytest.mark.gpu

POINTS = ("0", "50", "62p5", "75")


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("tag", POINTS)
def test_sweep_decode_64k_b16(tag):
    w = synth.workload(f"sweep_decode_64k_b16_s{tag}")
    print(f"[sweep] {w.name} counts={w.counts()}", flush=True)
    K, V, Q, q = synth.make_inputs_device(w)
    del Q
    shp, cnt = hs.shape(w.b, w.hq, w.hkv, w.L, w.D, w.B), hs.counts(*w.counts())
    cache = hs.alloc_cache(shp, cnt)
    hs.hs_compress(shp, cnt, K, V, cache, hs.alloc_workspace(hs.HS_OP_COMPRESS, shp, cnt))
    o = torch.empty((w.b, w.hq, w.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.b, w.hq), dtype=torch.float32, device="cuda")
    hs.hs_decode_attn(shp, cnt, cache, q, o, lse, 0.0, 0,
                      hs.alloc_workspace(hs.HS_OP_DECODE, shp, cnt))
    torch.cuda.synchronize()
    Kh, Vh, qh = host_bits(K), host_bits(V), host_bits(q)
    del K, V
    d = Dims(w.b, w.hkv, w.L, w.D, w.B, *w.counts())
    want = oracle.compress(d, Kh, Vh)
    del Kh, Vh
    gu.compare_cache(gu.cache_to_numpy(cache), want)
    ref, ref_lse = oracle.decode(d, want, qh, w.hq)
    assert_close(synth.bf16_to_f32(host_bits(o)), ref, lse.cpu().numpy(), ref_lse, w.name)


@pytest.mark.parametrize("tag", POINTS)
def test_sweep_prefill_32k_b1(tag):
    w = synth.workload(f"sweep_prefill_32k_b1_s{tag}")
    print(f"[sweep] {w.name} counts={w.counts()}", flush=True)
    K, V, Q, _ = synth.make_inputs_device(w)
    shp, cnt = hs.shape(w.b, w.hq, w.hkv, w.L, w.D, w.B), hs.counts(*w.counts())
    cache = hs.alloc_cache(shp, cnt)
    hs.hs_compress(shp, cnt, K, V, cache, hs.alloc_workspace(hs.HS_OP_COMPRESS, shp, cnt))
    O = torch.empty_like(Q)
    lse = torch.empty((w.b, w.hq, w.L), dtype=torch.float32, device="cuda")
    hs.hs_prefill_attn(shp, cnt, cache, Q, O, lse, 0.0, hs.HS_PREFILL_SMFMAC)
    torch.cuda.synchronize()
    d = Dims(w.b, w.hkv, w.L, w.D, w.B, *w.counts())
    want = oracle.compress(d, host_bits(K), host_bits(V))
    gu.compare_cache(gu.cache_to_numpy(cache), want)
    rows = sample_rows(w.b, w.hq, w.L, 4, 11)
    ref, ref_lse = oracle.prefill(d, want, host_bits(Q), rows=rows)
    o = synth.bf16_to_f32(host_bits(O)).reshape(-1, w.D)[rows]
    assert_close(o, ref, lse.cpu().numpy().reshape(-1)[rows], ref_lse, w.name)
