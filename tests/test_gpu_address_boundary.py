"""Cache arrays that straddle 4 GiB boundaries of the device address space.

Every 64-bit source address the kernels form must carry into its high half. The direct-load runs
of the prefill once overwrote the carry of a 64-bit address add that the compiler had split around
them (their M0 additions write SCC), which only shows when a block's address crosses a 4 GiB
boundary. Here each of the cache's eight arrays is placed across its own 4 GiB boundary inside one
large allocation; compress (bit-exact), decode and both prefill paths are compared with the
oracle."""
import numpy as np
import pytest
import torch

import oracle
from oracle import Dims
from sparse_kv_cache_magnitude_amd import hierasparse as hs
from sparse_kv_cache_magnitude_amd import synth
from tests import gpu_util as gu
from tests.test_gpu_decode import assert_close, run_decode
from tests.test_gpu_prefill import FLAGS, run_prefill

pytestmark = pytest.mark.gpu

GIB4 = 1 << 32


def test_cache_arrays_across_4gib_boundaries():
    rng = np.random.default_rng(43)
    b, hq, hkv, L, B, counts = 2, 8, 2, 64 * 24, 64, (3, 9, 7)
    shp, cnt = hs.shape(b, hq, hkv, L, 128, B), hs.counts(*counts)
    d = Dims(b, hkv, L, 128, B, *counts)
    K = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    V = synth.bf16_bits(rng.standard_normal((b, hkv, L, 128), dtype=np.float32))
    sizes = hs.hs_cache_sizes(shp, cnt)
    n = len(hs.CACHE_FIELDS)
    print(f"[boundary] b={b} hq={hq} hkv={hkv} L={L} B={B} counts={counts} sizes={sizes}",
          flush=True)
    big = torch.empty((n + 1) * GIB4 + (1 << 20), dtype=torch.uint8, device="cuda")
    base = big.data_ptr()
    first = (base + (1 << 20) + GIB4 - 1) // GIB4 * GIB4  # 4 GiB-aligned, 1 MiB in or more
    cache = {}
    for i, f in enumerate(hs.CACHE_FIELDS):
        nbytes = sizes[f]
        start = first + i * GIB4 - max(256, (nbytes // 2) // 256 * 256)
        assert base <= start and start + nbytes <= base + big.numel()
        dt = torch.int32 if f.startswith("map") else torch.int16
        cache[f] = big[start - base:start - base + nbytes].view(dt)
        print(f"[boundary] {f}: {nbytes} bytes at 0x{start:x} (boundary 0x{first + i * GIB4:x})",
              flush=True)

    ws = hs.alloc_workspace(hs.HS_OP_COMPRESS, shp, cnt)
    hs.hs_compress(shp, cnt, gu.to_dev(K), gu.to_dev(V), cache, ws)
    torch.cuda.synchronize()
    want = oracle.compress(d, K, V)
    gu.compare_cache(gu.cache_to_numpy(cache), want)

    q = synth.bf16_bits(rng.standard_normal((b, hq, 1, 128), dtype=np.float32))
    print("[boundary] decode", flush=True)
    o, lse, ref, ref_lse, _, _ = run_decode(b, hq, hkv, L, B, counts, K, V, q, cache=cache,
                                            want=want)
    assert_close(o, ref, lse, ref_lse, "decode across 4 GiB boundaries")

    Q = synth.bf16_bits(rng.standard_normal((b, hq, L, 128), dtype=np.float32))
    for path in ("smfmac", "decompress"):
        print(f"[boundary] prefill {path}", flush=True)
        o, lse, ref, ref_lse, _, _ = run_prefill(b, hq, hkv, L, B, counts, K, V, Q, FLAGS[path],
                                                 cache=cache, want=want)
        assert_close(o, ref, lse, ref_lse, f"prefill {path} across 4 GiB boundaries")
    del cache, big
    torch.cuda.empty_cache()
