"""Seeded synthetic inputs and the named workloads they are drawn for.

This module holds no step of the method: it only draws N(0,1) tensors, rounds them to bf16, adds
the key outlier channels, and turns block fractions into integer block counts. Both the GPU path
(tests, benchmark) and the CPU oracle (tests) consume what it returns.

Stand-in: the paper times its kernels on the Llama-3.1-8B-Instruct attention shape (32 query
heads, 8 KV heads, head_dim 128) at batch 8 and 32K context, independently of which pruning
algorithm picks the blocks (HieraSparse v2, §V-B1). These seeded N(0,1) tensors stand in for that
KV cache. Keys get a few large-magnitude channels that are the same for every token, as the key
caches pictured in §II, Fig. 2 show.
"""
from dataclasses import dataclass, field

import numpy as np

QKV_STREAMS = 4  # Q, K, V, outlier channels


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even. Inputs are finite."""
    u = np.array(x, dtype=np.float32, order="C", copy=True).view(np.uint32)
    return ((u + (0x7FFF + ((u >> 16) & 1))) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> IEEE binary16 bit patterns (uint16), numpy's round to nearest even."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def to_bits(x: np.ndarray, dtype: int = 0) -> np.ndarray:
    """float32 -> 16-bit patterns of element type dtype (0 bf16, 1 fp16)."""
    return f16_bits(x) if dtype else bf16_bits(x)


def to_f32(bits: np.ndarray, dtype: int = 0) -> np.ndarray:
    return f16_to_f32(bits) if dtype else bf16_to_f32(bits)


def _streams(seed: int):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(QKV_STREAMS)]


def make_kv(seed: int, b: int, hkv: int, L: int, D: int, outliers: int = 0,
            outlier_scale: float = 8.0, dtype: int = 0):
    """K, V [b][hkv][L][D] 16-bit patterns (dtype 0 bf16, 1 fp16) ~ N(0,1), drawn head by head.
    With outliers > 0, each KV head gets that many distinct key channels (shared by every batch
    entry and token) scaled by outlier_scale after rounding (a power of two, so exact)."""
    _, rk, rv, ro = _streams(seed)
    K = np.empty((b, hkv, L, D), np.uint16)
    V = np.empty((b, hkv, L, D), np.uint16)
    for bi in range(b):
        for h in range(hkv):
            K[bi, h] = to_bits(rk.standard_normal((L, D), dtype=np.float32), dtype)
    for bi in range(b):
        for h in range(hkv):
            V[bi, h] = to_bits(rv.standard_normal((L, D), dtype=np.float32), dtype)
    if outliers:
        for h in range(hkv):
            ch = ro.choice(D, outliers, replace=False)
            for c in ch:
                K[:, h, :, c] = to_bits(to_f32(K[:, h, :, c], dtype) * np.float32(outlier_scale),
                                        dtype)
    return K, V


def make_q(seed: int, b: int, hq: int, lq: int, D: int, dtype: int = 0):
    """Q [b][hq][lq][D] 16-bit patterns (dtype 0 bf16, 1 fp16) ~ N(0,1) (lq = 1 for decode)."""
    rq = _streams(seed)[0]
    return to_bits(rq.standard_normal((b, hq, lq, D), dtype=np.float32), dtype)


def random_modes(seed: int, b: int, hkv: int, nb: int, n_p: int, n_sk: int, n_sv: int):
    """Caller-side block-level masks with exact per-head counts: uint8 [b][hkv][nb] for K and V
    (0 pruned, 1 dense, 2 2:4), the pruned blocks shared, placed uniformly at random."""
    rng = np.random.default_rng(seed)
    mk = np.ones((b, hkv, nb), np.uint8)
    mv = np.ones((b, hkv, nb), np.uint8)
    for bi in range(b):
        for h in range(hkv):
            perm = rng.permutation(nb)
            mk[bi, h, perm[:n_p]] = 0
            mv[bi, h, perm[:n_p]] = 0
            rest = perm[n_p:]
            mk[bi, h, rng.permutation(rest)[:n_sk]] = 2
            mv[bi, h, rng.permutation(rest)[:n_sv]] = 2
    return mk, mv


def random_element_mask(seed: int, X: np.ndarray, modes: np.ndarray, B: int, along_tokens: bool,
                        keep: int = 2):
    """X [b][hkv][L][D] bf16 bits with a random caller-side element mask applied in the blocks
    whose mode is 2: in each group of four (consecutive channels of a token, or consecutive
    tokens of a channel if along_tokens) all but `keep` random positions are set to +0."""
    rng = np.random.default_rng(seed)
    b, hkv, L, D = X.shape
    out = X.copy()
    for bi in range(b):
        for h in range(hkv):
            for i in np.flatnonzero(modes[bi, h] == 2):
                blk = out[bi, h, i * B:(i + 1) * B]
                g = blk.T.reshape(D, B // 4, 4) if along_tokens else blk.reshape(B, D // 4, 4)
                r = rng.random(g.shape).argsort(axis=-1)      # a random order of the 4 positions
                g[r >= keep] = 0
                blk[...] = g.reshape(D, B).T if along_tokens else g.reshape(B, D)
    return out


def make_inputs_device(w, dtype=None, dev="cuda"):
    """The same recipe drawn on the device, for workloads too large to draw on the host in the
    time a test or a benchmark run has: K, V [b][hkv][L][D], prompt Q [b][hq][L][D] and decode q
    [b][hq][D] ~ N(0,1) as torch tensors of `dtype` (default bf16, rounded from fp32), from
    torch's generator seeded with the workload seed (K, then the outlier channels, then V, Q, q),
    with the workload's key outlier channels (per KV head, shared by every batch entry and token)
    scaled by 8 after rounding."""
    import torch
    dtype = dtype or torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    K = torch.randn((w.b, w.hkv, w.L, w.D), generator=g, device=dev, dtype=torch.float32)
    K = K.to(dtype)
    if w.outliers:
        for h in range(w.hkv):
            ch = torch.randperm(w.D, generator=g, device=dev)[:w.outliers]
            K[:, h, :, ch] *= 8
    V = torch.randn((w.b, w.hkv, w.L, w.D), generator=g, device=dev,
                    dtype=torch.float32).to(dtype)
    Q = torch.empty((w.b, w.hq, w.L, w.D), device=dev, dtype=dtype)
    for bi in range(w.b):
        Q[bi] = torch.randn((w.hq, w.L, w.D), generator=g, device=dev, dtype=torch.float32)
    q = torch.randn((w.b, w.hq, w.D), generator=g, device=dev, dtype=torch.float32)
    return K, V, Q, q.to(dtype)


def block_count(frac: float, nb: int) -> int:
    """Block fraction -> integer count, round half up."""
    return int(np.floor(frac * nb + 0.5))


@dataclass
class Workload:
    name: str
    phase: str              # "decode" or "prefill"
    b: int
    hq: int
    hkv: int
    D: int
    L: int
    B: int
    n_p: int
    n_sk: int
    n_sv: int
    seed: int
    outliers: int = 0
    note: str = field(default="")

    @property
    def nb(self):
        return self.L // self.B

    def counts(self):
        return self.n_p, self.n_sk, self.n_sv

    def with_counts(self, n_p, n_sk, n_sv, name=None):
        w = Workload(**{**self.__dict__})
        w.n_p, w.n_sk, w.n_sv = n_p, n_sk, n_sv
        if name:
            w.name = name
        return w


def _frac(name, phase, b, hq, hkv, L, B, dense, sparse, pruned, seed, outliers=0, note=""):
    nb = L // B
    n_p, n_s = block_count(pruned, nb), block_count(sparse, nb)
    assert n_p + n_s <= nb
    return Workload(name, phase, b, hq, hkv, 128, L, B, n_p, n_s, n_s, seed, outliers, note)


WORKLOADS = {}


def _add(w):
    WORKLOADS[w.name] = w


# one KV head, 4K tokens, every block 2:4 (50% sparsity), decode batch 1
_add(_frac("decode_1h_4k_all24", "decode", 1, 1, 1, 4096, 64, 0.0, 1.0, 0.0, 1001,
           note="single head parity case"))
# Llama-3.1-8B attention shape, 32K context, batch 8: 25% dense, 60% 2:4, 15% pruned blocks
_add(_frac("decode_llama8b_32k_b8", "decode", 8, 32, 8, 32768, 64, 0.25, 0.60, 0.15, 1002,
           outliers=4))
# causal prefill 16K, 128-token blocks: 30% dense, 70% 2:4
_add(_frac("prefill_16k_b1_B128", "prefill", 1, 32, 8, 16384, 128, 0.30, 0.70, 0.0, 1003))
# long-context decode 128K, batch 4: 10% dense, 50% 2:4, 40% pruned
_add(_frac("decode_128k_b4", "decode", 4, 32, 8, 131072, 64, 0.10, 0.50, 0.40, 1004))
# sparsity sweep: 0% / 50% (all 2:4) / 62.5% / 75% (extra sparsity from pruned blocks)
for k, (p, s) in enumerate([(0.0, 0.0), (0.0, 1.0), (0.25, 0.75), (0.5, 0.5)]):
    tag = ("0", "50", "62p5", "75")[k]
    _add(_frac(f"sweep_decode_64k_b16_s{tag}", "decode", 16, 32, 8, 65536, 64, 1 - p - s, s, p,
               1050 + k, outliers=4))
    _add(_frac(f"sweep_prefill_32k_b1_s{tag}", "prefill", 1, 32, 8, 32768, 64, 1 - p - s, s, p,
               1050 + k, outliers=4))


def workload(name: str) -> Workload:
    return WORKLOADS[name]
