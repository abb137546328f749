#!/usr/bin/env python3
"""Benchmark of the hierarchical sparse KV attention hot path on one MI355X.

One step = the whole hot path over one batch of the Llama-3.1-8B attention workload (32 query /
8 KV heads, head_dim 128, 32K context, batch 8, 64-token blocks, 25% dense / 60% 2:4 / 15% pruned
blocks -- the batch-8, 32K kernel benchmark setting of HieraSparse v2 §V-B1):
  hs_compress (score, rank, pack) of the 32K-token K/V cache,
  hs_prefill_attn causal over the 32K prompt (2:4 blocks on SMFMAC),
  hs_decode_attn of one new token per query head over the compressed cache.
Each call is bracketed by HIP events on the stream the kernels run on. Between prefill and decode a
read pass over 1 GiB (part of the step, outside both windows) settles the dirty cache lines of the
prefill's 2 GiB output, so the decode window holds the decode's own HBM traffic. The same kernels
on a cache compressed with every block dense give the same-kernel dense baseline.

Output: one JSON line. value = decode HBM throughput (GB/s) on the compressed bytes the decode
must read; roofline = the step's dominant kernel (prefill, matrix cores); the other kernels'
rooflines, times and speedups vs dense are extra keys. The CPU oracle is timed on a bounded sample
of the same workload on the host cores (cpu_baseline).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "decode_llama8b_32k_b8"
HBM_PEAK_GBS = 8000.0
BF16_DENSE_PEAK_TFLOPS = 2500.0
SETTLE_BYTES = 1 << 30  # read pass that settles dirty last-level-cache lines (cache: 256 MiB)
SUITE_PARTS = ("prefill16k", "decode128k", "sweeps", "recompress", "masked", "policy", "f16",
               "ablation")
COPY_BYTES = 1 << 30    # calibration copy for the byte counters (--copy-probe)
COPY_KERNEL = "neg_kernel"  # torch's elementwise kernel that the calibration copy runs

# Kernels whose HBM traffic is summarised, with the sources their digest covers.
TRAFFIC_KERNELS = {"k_prefill": ("hs_prefill.hip", "hs_device.h"),
                   "k_decode_split": ("hs_decode.hip", "hs_device.h"),
                   "k_score": ("hs_compress.hip", "hs_device.h"),
                   "k_rank": ("hs_compress.hip", "hs_device.h"),
                   "k_pack": ("hs_compress.hip", "hs_device.h")}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--prefill-path", choices=["smfmac", "decompress"], default="smfmac")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-dense-baseline", action="store_true")
    p.add_argument("--cpu-sample-heads", type=int, default=16,
                   help="(batch, KV head) pairs the oracle runs for the CPU baseline")
    p.add_argument("--cpu-leg", action="store_true",
                   help="(internal) run one CPU-oracle leg and print its JSON line")
    p.add_argument("--copy-probe", action="store_true",
                   help="first run a plain device copy of COPY_BYTES (reads and writes a known "
                        "number of bytes: the calibration of rocprofv3's byte counters)")
    p.add_argument("--suite", nargs="?", const=",".join(SUITE_PARTS), default=None,
                   metavar="PARTS",
                   help="instead of the headline step: one JSON line per further workload; PARTS "
                        "is a comma list of " + ", ".join(SUITE_PARTS) + " (default: all): 16K "
                        "prefill with both 2:4 paths, 128K decode, the sparsity sweeps, the "
                        "prefill-to-decode re-compression, the caller-mask compressor, the "
                        "sink/local dense policy, the fp16 element type at 32K batch 8 and the "
                        "prefill ablation (each optimisation left out in turn) at 32K batch 8")
    p.add_argument("--peaks", action="store_true",
                   help="instead of the headline step: the measured ceilings of the GPU "
                        "(libhspeaks.so): matrix-core issue loops (MFMA and SMFMAC), vector-ALU "
                        "loops (exp2, FMA, max3, bf16 pack), matrix-core and vector work sharing "
                        "a SIMD, and streaming HBM reads; one JSON line each")
    p.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no GPU work: turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, "
                        "then WRITE_SIZE, each with --copy-probe) into profiles/traffic.json")
    return p.parse_args()


# ------------------------------------------------------------------------------------------------
# Algorithmic work (bytes and flops the method must move / execute), from the mode table.

def decode_bytes(w, G):
    """Compressed K/V blocks the decode must stream, both index maps, q in and o out."""
    B, D, nb = w.B, w.D, w.nb
    ndk, ndv = nb - w.n_p - w.n_sk, nb - w.n_p - w.n_sv
    per_head = (ndk + ndv) * 2 * B * D + (w.n_sk + w.n_sv) * (B * D + B * D // 8) \
        + 2 * 4 * nb + 2 * G * D * 2
    return per_head * w.b * w.hkv


def compress_bytes(w, cache_bytes):
    """Two passes over K and V (score, pack) plus the compressed output."""
    return 2 * 2 * w.b * w.hkv * w.L * w.D * 2 + sum(cache_bytes.values())


def prefill_flops(w, map_k, map_v, smfmac=True):
    """Causal attention work over visible (query, key) pairs with key <= query: dense-equivalent
    flops (4*D per pair) and the flops the matrix cores must execute, where a 2:4 operand costs
    half (Eq. 9 of HieraSparse v2 §III-D2) on the SMFMAC path and full on the decompress path."""
    import numpy as np
    B, D, L = w.B, w.D, w.L
    nb = L // B
    i = np.arange(nb, dtype=np.float64)
    # pairs (q, k) with k in block i and q >= k: sum over the block's tokens of (L - k)
    pairs = B * L - B * i * B - B * (B - 1) / 2.0
    mk = np.asarray(map_k).reshape(-1, nb)
    mv = np.asarray(map_v).reshape(-1, nb)
    vis = mk != 0
    ck = np.where(mk > 0, 1.0, 0.5 if smfmac else 1.0)
    cv = np.where(mv > 0, 1.0, 0.5 if smfmac else 1.0)
    G = w.hq // w.hkv
    dense_eq = float((vis * pairs).sum()) * 4 * D * G
    executed = float((vis * pairs * (ck + cv)).sum()) * 2 * D * G
    full_causal = 4 * D * L * (L + 1) / 2 * w.hq * w.b
    return dense_eq, executed, full_causal


def source_digest(*names):
    """Digest of the code of kernel sources: line comments, trailing blanks and empty lines are
    dropped, so a comment edit does not void counters taken on the same code."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sparse_kv_cache_magnitude_amd", "csrc", n)) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(kernel_key, digest):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on the
    current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


def summarize_counters(fetch_dir, write_dir):
    """HBM bytes per launch of the hot-path kernels from two rocprofv3 --pmc runs (FETCH_SIZE and
    WRITE_SIZE, KiB per dispatch), over the launches of each kernel's largest grid. Each counter is
    scaled by the bytes the calibration copy really moves over what the same counter reads for
    it. Writes profiles/traffic.json."""
    import csv
    import glob
    from collections import defaultdict

    def per_kernel(d, counter):
        paths = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not paths:
            raise SystemExit(f"no counter_collection.csv under {d}")
        vals = defaultdict(lambda: defaultdict(float))
        grid = {}
        for path in paths:
            with open(path) as f:
                for r in csv.DictReader(f):
                    if r["Counter_Name"] == counter:
                        vals[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
                        grid[r["Dispatch_Id"]] = int(r["Grid_Size"])
        # per kernel, the launches of the largest grid: the headline workload's (the small
        # workload the bench also times runs the same kernels)
        launches = defaultdict(list)
        for name, per_dispatch in vals.items():
            key = next((k for k in list(TRAFFIC_KERNELS) + [COPY_KERNEL] if k in name), None)
            if key:
                launches[key] += [(grid[d], v) for d, v in per_dispatch.items()]
        out = {}
        for key, gv in launches.items():
            top = max(g for g, _ in gv)
            out[key] = [v for g, v in gv if g == top]
        return out

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    if COPY_KERNEL not in fetch or COPY_KERNEL not in write:
        raise SystemExit("the calibration copy is missing: run the profiled command with "
                         "--copy-probe")
    kib = lambda xs: sum(xs) / len(xs)
    f_scale = COPY_BYTES / (kib(fetch[COPY_KERNEL]) * 1024)
    w_scale = COPY_BYTES / (kib(write[COPY_KERNEL]) * 1024)
    rec = {"calibration": {"kernel": COPY_KERNEL, "bytes_read": COPY_BYTES,
                           "bytes_written": COPY_BYTES,
                           "fetch_kib": round(kib(fetch[COPY_KERNEL]), 1),
                           "write_kib": round(kib(write[COPY_KERNEL]), 1),
                           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)}}
    for k, srcs in TRAFFIC_KERNELS.items():
        if k in fetch and k in write:
            fb, wb = kib(fetch[k]) * 1024 * f_scale, kib(write[k]) * 1024 * w_scale
            rec[k] = {"source_digest": source_digest(*srcs), "dispatches": len(fetch[k]),
                      "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
                      "hbm_bytes_per_launch": round(fb + wb)}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))
    return 0


# ------------------------------------------------------------------------------------------------

def make_inputs(w, torch, dev, dtype=None):
    """Seeded N(0,1) K, V, prompt Q and decode q of the workload shape (bf16, or the torch dtype
    given), drawn on the device with the workload's key outlier channels scaled by 8
    (synth.make_inputs_device; the timing does not depend on the values)."""
    from sparse_kv_cache_magnitude_amd import synth
    return synth.make_inputs_device(w, dtype, dev)


def cpu_baseline(w, heads, min_seconds=10.0):
    """The oracle (C, fp64, OpenMP) on `heads` (batch, KV head) pairs of the workload: compress
    their K/V, then decode their query heads over the result. Reported in the metric's unit: GB/s
    of compressed decode bytes, i.e. decode_bytes of the sample / oracle decode time."""
    import numpy as np
    import oracle
    from oracle import Dims
    from sparse_kv_cache_magnitude_amd import synth
    G = w.hq // w.hkv
    K, V = synth.make_kv(w.seed, 1, heads, w.L, w.D, outliers=w.outliers)
    q = synth.make_q(w.seed, 1, heads * G, 1, w.D)
    d = Dims(1, heads, w.L, w.D, w.B, w.n_p, w.n_sk, w.n_sv)
    t0 = time.perf_counter()
    cache = oracle.compress(d, K, V)
    t1 = time.perf_counter()
    reps = 0
    while True:  # repeat the decode for about ten seconds of CPU time
        oracle.decode(d, cache, q, heads * G)
        reps += 1
        t2 = time.perf_counter()
        if t2 - t1 >= min_seconds:
            break
    per = (t2 - t1) / reps
    sample_w = synth.Workload(**{**w.__dict__, "b": 1, "hkv": heads, "hq": heads * G})
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(decode_bytes(sample_w, G) / per / 1e9, 3), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{heads} of {w.b * w.hkv} (batch, KV head) pairs of {w.name}: fp64 decode "
                      f"(decompress + attention) of their {heads * G} query heads over "
                      f"{w.L} tokens, repeated {reps}x; compress of the same heads took "
                      f"{t1 - t0:.2f} s",
            "decode_s_per_rep": round(per, 4), "compress_s": round(t1 - t0, 3)}


def cpu_prefill_sample(q_heads=4, stride=64):
    """The oracle's causal prefill on the 16K, 128-token-block workload, on a row sample: the first
    q_heads query heads, every stride-th query row plus every row of the first and the last block.
    The full time is extrapolated by visible (query, key) pairs (the workload prunes no block, so
    row i sees i + 1 keys); the sampled call includes the oracle's decompression of the whole
    cache, which the extrapolation scales with the rest (an overestimate)."""
    import numpy as np
    import oracle
    from oracle import Dims
    from sparse_kv_cache_magnitude_amd import synth
    w = synth.workload("prefill_16k_b1_B128")
    K, V = synth.make_kv(w.seed, w.b, w.hkv, w.L, w.D, outliers=w.outliers)
    d = Dims(w.b, w.hkv, w.L, w.D, w.B, *w.counts())
    cache = oracle.compress(d, K, V)
    Q = synth.make_q(w.seed, w.b, w.hq, w.L, w.D)
    per_head = sorted(set(range(0, w.L, stride)) | set(range(w.B)) |
                      set(range(w.L - w.B, w.L)))
    rows = np.array([h * w.L + r for h in range(q_heads) for r in per_head], np.int64)
    t0 = time.perf_counter()
    oracle.prefill(d, cache, Q, rows=rows)
    t = time.perf_counter() - t0
    pairs_sample = float(sum(r + 1 for r in per_head)) * q_heads
    pairs_total = float(w.L) * (w.L + 1) / 2 * w.hq * w.b
    return {"workload": w.name, "sample_rows": int(len(rows)), "sample_s": round(t, 3),
            "extrapolated_ms": round(t * pairs_total / pairs_sample * 1e3, 1),
            "method": f"{q_heads} of {w.hq} query heads, every {stride}th row and the first and "
                      f"last {w.B}-token blocks; scaled by visible (query, key) pairs "
                      f"({pairs_total / pairs_sample:.1f}x); extrapolated"}


def cpu_leg(heads):
    """One CPU-oracle leg (run in a child process, whose OMP_NUM_THREADS sets its threads): the
    decode/compress baseline of the headline workload and the sampled 16K prefill; one JSON line."""
    from sparse_kv_cache_magnitude_amd import synth
    rec = cpu_baseline(synth.workload(WORKLOAD), heads)
    rec["prefill_16k"] = cpu_prefill_sample()
    print(json.dumps(rec), flush=True)
    return 0


def cpu_legs(heads):
    """The oracle timed at one thread and at all the threads it may use (OMP_NUM_THREADS, else the
    CPU count), each in a child process started before this process touches the GPU."""
    import subprocess
    all_threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    out = {}
    for n in sorted({1, all_threads}):
        env = dict(os.environ, OMP_NUM_THREADS=str(n))
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-leg",
                            "--cpu-sample-heads", str(heads)], env=env, capture_output=True,
                           text=True, timeout=600)
        if r.returncode != 0:
            raise RuntimeError(f"CPU oracle leg ({n} threads) failed:\n{r.stderr[-2000:]}")
        out[n] = json.loads(r.stdout.strip().splitlines()[-1])
    return out[all_threads], out[1]


def run_suite(parts=SUITE_PARTS, reps=7):
    """The further measured workloads, one JSON line each: the 16K causal prefill with 128-token
    blocks on both 2:4 paths, the 128K long-context decode, the sparsity sweeps (decode and
    compressor at 64K / batch 16, prefill at 32K / batch 1) and the re-compression of the 32K
    batch-8 cache from its prefill counts (K dense) to its decode counts. Every timing is the
    median of `reps` HIP-event windows around one call; each decode window follows a 1 GiB read
    pass (the settled, cold-cache state). Workloads are also run on an all-dense cache (same
    kernels)."""
    import numpy as np
    import torch
    from sparse_kv_cache_magnitude_amd import hierasparse as hs
    from sparse_kv_cache_magnitude_amd import synth
    dev = "cuda"
    stream = torch.cuda.current_stream()
    settle = torch.ones(SETTLE_BYTES // 4, device=dev, dtype=torch.float32)

    def timed(fn, pre=None):
        ts = []
        for _ in range(reps + 1):
            if pre:
                pre()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / 1e3)
        return float(np.median(ts[1:]))

    def setup(w, counts=None):
        K, V, Q, q = make_inputs(w, torch, dev)
        shp = hs.shape(w.b, w.hq, w.hkv, w.L, w.D, w.B)
        cnt = hs.counts(*(counts or (w.n_p, w.n_sk, w.n_sv)))
        cache = hs.alloc_cache(shp, cnt)
        ws_c = hs.alloc_workspace(hs.HS_OP_COMPRESS, shp, cnt)
        comp = timed(lambda: hs.hs_compress(shp, cnt, K, V, cache, ws_c))
        return K, V, Q, q, shp, cnt, cache, comp

    def decode_time(shp, cnt, cache, q):
        ws = hs.alloc_workspace(hs.HS_OP_DECODE, shp, cnt)
        o = torch.empty_like(q)
        return timed(lambda: hs.hs_decode_attn(shp, cnt, cache, q, o, None, 0.0, 0, ws),
                     pre=lambda: settle.sum())

    def prefill_time(shp, cnt, cache, Q, flags):
        O = torch.empty_like(Q)
        return timed(lambda: hs.hs_prefill_attn(shp, cnt, cache, Q, O, None, 0.0, flags))

    def emit(rec):
        print(json.dumps(rec), flush=True)

    if "prefill16k" in parts:
        suite_prefill16k(hs, synth, setup, prefill_time, emit)
    if "decode128k" in parts:
        suite_decode128k(hs, synth, setup, decode_time, emit)
    if "sweeps" in parts:
        suite_sweeps(hs, synth, setup, decode_time, prefill_time, emit)
    if "recompress" in parts:
        suite_recompress(hs, synth, setup, timed, emit, torch)
    if "masked" in parts:
        suite_masked(hs, synth, setup, timed, emit, torch)
    if "policy" in parts:
        suite_policy(hs, synth, setup, timed, decode_time, emit)
    if "f16" in parts:
        suite_f16(hs, synth, timed, decode_time, prefill_time, emit, torch)
    if "ablation" in parts:
        suite_ablation(hs, synth, setup, timed, emit, torch)
    return 0


def suite_prefill16k(hs, synth, setup, prefill_time, emit):
    """16K causal prefill, 128-token blocks, both 2:4 paths, against the all-dense cache."""
    w = synth.workload("prefill_16k_b1_B128")
    K, V, Q, q, shp, cnt, cache, comp = setup(w)
    mk, mv = cache["map_k"].cpu().numpy(), cache["map_v"].cpu().numpy()
    t_s = prefill_time(shp, cnt, cache, Q, hs.HS_PREFILL_SMFMAC)
    t_d = prefill_time(shp, cnt, cache, Q, hs.HS_PREFILL_DECOMPRESS)
    dense_eq, ex_s, full = prefill_flops(w, mk, mv, True)
    _, ex_d, _ = prefill_flops(w, mk, mv, False)
    _, _, _, _, shp0, cnt0, cache0, _ = setup(w, (0, 0, 0))
    t0 = prefill_time(shp0, cnt0, cache0, Q, hs.HS_PREFILL_SMFMAC)
    t0_d = prefill_time(shp0, cnt0, cache0, Q, hs.HS_PREFILL_DECOMPRESS)
    peak = BF16_DENSE_PEAK_TFLOPS * 1e12
    emit({"suite": w.name, "prefill_ms_smfmac": round(t_s * 1e3, 3),
          "prefill_ms_decompress": round(t_d * 1e3, 3), "prefill_ms_dense_cache": round(t0 * 1e3, 3),
          "prefill_ms_dense_cache_decompress_kernel": round(t0_d * 1e3, 3),
          "speedup_vs_fastest_dense_smfmac": round(min(t0, t0_d) / t_s, 3),
          "tflops_dense_equivalent_smfmac": round(dense_eq / t_s / 1e12, 1),
          "mfma_utilisation_smfmac": round(ex_s / peak / t_s, 4),
          "mfma_utilisation_decompress": round(ex_d / peak / t_d, 4),
          "mfma_utilisation_dense_cache": round(full / peak / t0, 4),
          "speedup_vs_dense_smfmac": round(t0 / t_s, 3),
          "speedup_vs_dense_decompress": round(t0 / t_d, 3),
          "smfmac_over_decompress_speed": round(t_d / t_s, 3),
          "ideal_speedup_executed_flops": round(full / ex_s, 3),
          "compress_us": round(comp * 1e6, 1), "compress_share_of_prefill": round(comp / t_s, 5)})
    del K, V, Q, q, cache, cache0


def suite_decode128k(hs, synth, setup, decode_time, emit):
    """128K long-context decode against the all-dense cache."""
    w = synth.workload("decode_128k_b4")
    G = w.hq // w.hkv
    K, V, Q, q, shp, cnt, cache, comp = setup(w)
    del Q
    t = decode_time(shp, cnt, cache, q)
    _, _, _, _, shp0, cnt0, cache0, _ = setup(w, (0, 0, 0))
    t0 = decode_time(shp0, cnt0, cache0, q)
    nbytes, nbytes0 = decode_bytes(w, G), decode_bytes(w.with_counts(0, 0, 0), G)
    emit({"suite": w.name, "decode_us": round(t * 1e6, 2), "decode_gbs": round(nbytes / t / 1e9, 1),
          "frac_hbm_peak": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4), "decode_bytes": nbytes,
          "dense_cache_us": round(t0 * 1e6, 2), "speedup_vs_dense": round(t0 / t, 3),
          "ideal_speedup_bytes": round(nbytes0 / nbytes, 3), "compress_us": round(comp * 1e6, 1)})
    del K, V, q, cache, cache0


def suite_sweeps(hs, synth, setup, decode_time, prefill_time, emit):
    """Sparsity sweeps: decode and compressor at 64K / batch 16, causal prefill at 32K / batch 1."""
    base = None
    for tag in ("0", "50", "62p5", "75"):
        w = synth.workload(f"sweep_decode_64k_b16_s{tag}")
        G = w.hq // w.hkv
        K, V, Q, q, shp, cnt, cache, comp = setup(w)
        del Q
        t = decode_time(shp, cnt, cache, q)
        base = base or (t, decode_bytes(w, G))
        nbytes = decode_bytes(w, G)
        emit({"suite": w.name, "decode_us": round(t * 1e6, 2),
              "decode_gbs": round(nbytes / t / 1e9, 1),
              "frac_hbm_peak": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
              "speedup_vs_0pct": round(base[0] / t, 3),
              "ideal_speedup_bytes": round(base[1] / nbytes, 3),
              "compress_us": round(comp * 1e6, 1),
              "compress_gbs": round(compress_bytes(w, hs.hs_cache_sizes(shp, cnt)) / comp / 1e9, 1)})
        del K, V, q, cache
    base = None
    for tag in ("0", "50", "62p5", "75"):
        w = synth.workload(f"sweep_prefill_32k_b1_s{tag}")
        K, V, Q, q, shp, cnt, cache, comp = setup(w)
        mk, mv = cache["map_k"].cpu().numpy(), cache["map_v"].cpu().numpy()
        t = prefill_time(shp, cnt, cache, Q, hs.HS_PREFILL_SMFMAC)
        dense_eq, ex, full = prefill_flops(w, mk, mv, True)
        base = base or (t, ex)
        emit({"suite": w.name, "prefill_ms": round(t * 1e3, 3),
              "tflops_dense_equivalent": round(dense_eq / t / 1e12, 1),
              "mfma_utilisation": round(ex / (BF16_DENSE_PEAK_TFLOPS * 1e12) / t, 4),
              "speedup_vs_0pct": round(base[0] / t, 3),
              "ideal_speedup_executed_flops": round(base[1] / ex, 3),
              "compress_us": round(comp * 1e6, 1), "compress_share_of_prefill": round(comp / t, 5)})
        del K, V, Q, q, cache


def suite_recompress(hs, synth, setup, timed, emit, torch):
    """The 32K batch-8 cache compressed for prefill (K dense, V 2:4) and re-compressed to its
    decode counts (K and V 2:4). Re-compression = expansion of the cache to dense K, V in the
    workspace, then the compressor; its bytes by design are the compressed input, the dense
    intermediate written once and the compressor's own bytes."""
    w = synth.workload("decode_llama8b_32k_b8")
    first = (w.n_p, 0, w.n_sv)
    K, V, Q, q, shp, cnt1, cache1, comp1 = setup(w, first)
    del Q, q
    cnt2 = hs.counts(*w.counts())
    cache2 = hs.alloc_cache(shp, cnt2)
    ws_c = hs.alloc_workspace(hs.HS_OP_COMPRESS, shp, cnt2)
    comp2 = timed(lambda: hs.hs_compress(shp, cnt2, K, V, cache2, ws_c))
    ws = hs.alloc_workspace(hs.HS_OP_RECOMPRESS, shp, cnt2)
    t = timed(lambda: hs.hs_recompress(shp, cnt1, cache1, cnt2, cache2, ws))
    in_bytes = sum(hs.hs_cache_sizes(shp, cnt1).values())
    dense = 2 * w.b * w.hkv * w.L * w.D * 2
    design = in_bytes + dense + compress_bytes(w, hs.hs_cache_sizes(shp, cnt2))
    emit({"suite": w.name + "_recompress", "from_counts": list(first),
          "to_counts": list(w.counts()), "recompress_us": round(t * 1e6, 1),
          "compress_from_dense_us": round(comp2 * 1e6, 1),
          "compress_prefill_counts_us": round(comp1 * 1e6, 1),
          "design_bytes": design, "design_gbs": round(design / t / 1e9, 1),
          "frac_hbm_peak": round(design / t / 1e9 / HBM_PEAK_GBS, 4)})
    del K, V, cache1, cache2, ws


def suite_masked(hs, synth, setup, timed, emit, torch):
    """The caller-mask compressor on the 32K batch-8 shape: random block masks at the workload's
    counts, random 2:4 element masks applied in the 2:4 blocks (drawn on the host), against the
    magnitude compressor on the same tensors. Algorithmic bytes: K and V of the blocks that are not
    pruned, both mode arrays, and the compressed cache written."""
    import numpy as np
    w = synth.workload("decode_llama8b_32k_b8")
    K, V, Q, q, shp, cnt, cache, comp = setup(w)
    del Q, q
    mk, mv = synth.random_modes(41, w.b, w.hkv, w.nb, *w.counts())
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    Kh = K.view(torch.int16).cpu().numpy().view(np.uint16)
    Vh = V.view(torch.int16).cpu().numpy().view(np.uint16)
    Km = dev(synth.random_element_mask(42, Kh, mk, w.B, False).view(np.int16))
    Vm = dev(synth.random_element_mask(43, Vh, mv, w.B, True).view(np.int16))
    del Kh, Vh
    mkd, mvd = dev(mk), dev(mv)
    status = torch.empty(w.b * w.hkv, dtype=torch.int32, device="cuda")
    t = timed(lambda: hs.hs_compress_masked(shp, cnt, Km, Vm, mkd, mvd, cache, status))
    assert int(status.abs().sum()) == 0
    kept = w.nb - w.n_p
    nbytes = (2 * w.b * w.hkv * kept * w.B * w.D * 2 + 2 * mk.size
              + sum(hs.hs_cache_sizes(shp, cnt).values()))
    emit({"suite": w.name + "_masked", "masked_compress_us": round(t * 1e6, 1),
          "magnitude_compress_us": round(comp * 1e6, 1), "bytes": nbytes,
          "gbs": round(nbytes / t / 1e9, 1), "frac_hbm_peak": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)})
    del K, V, Km, Vm, cache

def suite_policy(hs, synth, setup, timed, decode_time, emit):
    """The 32K batch-8 cache compressed with the quality runs' dense policy (first 64 and last 256
    tokens dense, unranked) at the workload's counts, against the plain compressor, and the decode
    on both caches."""
    w = synth.workload("decode_llama8b_32k_b8")
    G = w.hq // w.hkv
    K, V, Q, q, shp, cnt, cache, comp = setup(w)
    del Q
    pol = hs.policy(64, 256)
    cache_p = hs.alloc_cache(shp, cnt)
    ws = hs.alloc_workspace(hs.HS_OP_COMPRESS, shp, cnt)
    t_c = timed(lambda: hs.hs_compress_ex(shp, cnt, pol, K, V, cache_p, ws))
    t = decode_time(shp, cnt, cache, q)
    t_p = decode_time(shp, cnt, cache_p, q)
    nbytes = decode_bytes(w, G)
    emit({"suite": w.name + "_policy_sink64_local256", "compress_policy_us": round(t_c * 1e6, 1),
          "compress_us": round(comp * 1e6, 1), "decode_policy_us": round(t_p * 1e6, 2),
          "decode_us": round(t * 1e6, 2), "decode_bytes": nbytes,
          "decode_policy_gbs": round(nbytes / t_p / 1e9, 1)})
    del K, V, q, cache, cache_p

def suite_f16(hs, synth, timed, decode_time, prefill_time, emit, torch):
    """The 32K batch-8 workload in fp16 (the pages' precision): compressor, decode and causal
    prefill on the sparse cache and on the all-dense cache, so that the speedups can be set beside
    the pages' fp16 ratios."""
    w = synth.workload("decode_llama8b_32k_b8")
    G = w.hq // w.hkv
    K, V, Q, q = make_inputs(w, torch, "cuda", torch.float16)
    shp = hs.shape(w.b, w.hq, w.hkv, w.L, w.D, w.B, dtype=hs.HS_F16)
    res = {}
    for tag, counts in (("sparse", w.counts()), ("dense", (0, 0, 0))):
        cnt = hs.counts(*counts)
        cache = hs.alloc_cache(shp, cnt)
        ws = hs.alloc_workspace(hs.HS_OP_COMPRESS, shp, cnt)
        comp = timed(lambda: hs.hs_compress(shp, cnt, K, V, cache, ws))
        t_d = decode_time(shp, cnt, cache, q)
        t_p = prefill_time(shp, cnt, cache, Q, hs.HS_PREFILL_SMFMAC)
        mk, mv = cache["map_k"].cpu().numpy(), cache["map_v"].cpu().numpy()
        res[tag] = (comp, t_d, t_p, prefill_flops(w, mk, mv, True))
        del cache
    comp, t_d, t_p, (dense_eq, ex, _) = res["sparse"]
    _, t_d0, t_p0, _ = res["dense"]
    nbytes = decode_bytes(w, G)
    emit({"suite": w.name + "_f16", "decode_us": round(t_d * 1e6, 2),
          "decode_gbs": round(nbytes / t_d / 1e9, 1),
          "frac_hbm_peak": round(nbytes / t_d / 1e9 / HBM_PEAK_GBS, 4),
          "decode_dense_cache_us": round(t_d0 * 1e6, 2), "decode_speedup": round(t_d0 / t_d, 3),
          "prefill_ms": round(t_p * 1e3, 3), "prefill_dense_cache_ms": round(t_p0 * 1e3, 3),
          "prefill_speedup": round(t_p0 / t_p, 3),
          "prefill_tflops_dense_equivalent": round(dense_eq / t_p / 1e12, 1),
          "mfma_utilisation": round(ex / (BF16_DENSE_PEAK_TFLOPS * 1e12) / t_p, 4),
          "compress_us": round(comp * 1e6, 1)})
    del K, V, Q, q

def suite_ablation(hs, synth, setup, timed, emit, torch):
    """What each optimisation of the SMFMAC prefill is worth (the ablation of the HieraSparse
    paper's §IV-C, Fig. 4, at its setting: Llama-3.1-8B attention shape, 32K context, batch 8):
    the default kernel and its variants that leave out one optimisation each (loads pipelined a
    tile ahead, the dense and 2:4 stage buffers aliased, the walks specialised for all-2:4 and
    all-dense workgroups, four-wave workgroups two per CU, and the token order that lets P^T stay
    in registers instead of a round trip through LDS), on the decode workload's mixed cache
    (25% dense, 60% 2:4, 15% pruned blocks) and on an all-2:4 cache."""
    base = synth.workload(WORKLOAD)
    variants = (("default", hs.HS_PREFILL_VARIANT_NONE),
                ("sync_loads", hs.HS_PREFILL_VARIANT_SYNC_LOADS),
                ("no_alias", hs.HS_PREFILL_VARIANT_NO_ALIAS),
                ("generic_walk", hs.HS_PREFILL_VARIANT_GENERIC_WALK),
                ("lockstep_8wave", hs.HS_PREFILL_VARIANT_LOCKSTEP),
                ("lds_relayout", hs.HS_PREFILL_VARIANT_LDS_RELAYOUT))
    gains = {"sync_loads": "gain_pipelining", "no_alias": "gain_aliasing",
             "generic_walk": "gain_specialised_walk", "lockstep_8wave": "gain_four_wave",
             "lds_relayout": "gain_in_register_relayout"}
    for tag, counts in (("mixed", None), ("all24", (0, base.nb, base.nb))):
        w = base if counts is None else base.with_counts(*counts)
        K, V, Q, q, shp, cnt, cache, _ = setup(w)
        del K, V, q
        O = torch.empty_like(Q)
        ms = {}
        for name, v in variants:
            ms[name] = timed(lambda: hs.hs_prefill_attn_variant(shp, cnt, cache, Q, O, None, 0.0,
                                                                v)) * 1e3
        rec = {"suite": f"ablation_prefill_32k_b8_{tag}",
               "counts": [w.n_p, w.n_sk, w.n_sv]}
        rec.update({f"{n}_ms": round(t, 3) for n, t in ms.items()})
        rec.update({g: round(ms[n] / ms["default"], 3) for n, g in gains.items()})
        emit(rec)
        del Q, O, cache


def run_peaks(reps=3):
    """Measured ceilings of the GPU. Each probe is timed with HIP events (median of `reps` after
    one warm-up launch); cycle counts are per SIMD at the shader clock the probe's own clock
    samples give (s_memtime against the 100 MHz counter). Every loop kernel runs one workgroup
    per CU, so w waves per workgroup put w/4 waves on each of the 1024 SIMDs."""
    import numpy as np
    import torch
    from sparse_kv_cache_magnitude_amd import peaks as pk
    dev = "cuda"
    stream = torch.cuda.current_stream()
    n_simd = 1024
    out = torch.empty(1024 * 1024, device=dev, dtype=torch.float32)
    clk = torch.zeros(4, device=dev, dtype=torch.int64)

    def timed(fn):
        ts = []
        for _ in range(reps + 1):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / 1e3)
        return float(np.median(ts[1:]))

    def clock_hz():
        c = clk.cpu().numpy().astype(np.float64)
        return (c[2] - c[0]) / max(c[3] - c[1], 1.0) * 1e8

    def emit(rec):
        print(json.dumps(rec), flush=True)

    grid = 1024  # four waves of workgroups over the 256 CUs
    flops = {pk.HSP_MFMA_32X32X16: 32768, pk.HSP_SMFMAC_32X32X32: 65536,
             pk.HSP_MFMA_16X16X32: 16384, pk.HSP_SMFMAC_16X16X64: 32768}
    names = {pk.HSP_MFMA_32X32X16: "v_mfma_f32_32x32x16_bf16",
             pk.HSP_SMFMAC_32X32X32: "v_smfmac_f32_32x32x32_bf16",
             pk.HSP_MFMA_16X16X32: "v_mfma_f32_16x16x32_bf16",
             pk.HSP_SMFMAC_16X16X64: "v_smfmac_f32_16x16x64_bf16"}
    iters = 4096
    f_clk = None
    for kind in names:
        for waves in (4, 8):
            t = timed(lambda: pk.matrix_loop(kind, grid, waves, iters, out, clk))
            f_clk = clock_hz()
            n_ins = grid * waves * iters * 4
            logical = n_ins * flops[kind]
            sparse = kind in (pk.HSP_SMFMAC_32X32X32, pk.HSP_SMFMAC_16X16X64)
            emit({"peak": "matrix_loop", "instruction": names[kind], "waves_per_simd": waves // 4,
                  "ms": round(t * 1e3, 4), "shader_clock_ghz": round(f_clk / 1e9, 3),
                  "tflops_logical": round(logical / t / 1e12, 1),
                  "tflops_executed": round(logical / (2 if sparse else 1) / t / 1e12, 1),
                  "frac_of_2p5pf_executed": round(logical / (2 if sparse else 1) / t / 2.5e15, 4),
                  "cycles_per_instruction_per_simd": round(t * f_clk * n_simd / n_ins, 2)})
    # Dependent chains: each instruction accumulates into the previous one's (or the one before's)
    # result, as a GEMM's k-steps into one output tile do.
    for kind in (pk.HSP_MFMA_32X32X16, pk.HSP_SMFMAC_32X32X32):
        for accs in (1, 2):
            for waves in (4, 8):
                t = timed(lambda: pk.matrix_chain(kind, accs, grid, waves, iters, out, clk))
                f_clk = clock_hz()
                n_ins = grid * waves * iters * 4
                emit({"peak": "matrix_chain", "instruction": names[kind], "accumulators": accs,
                      "waves_per_simd": waves // 4, "ms": round(t * 1e3, 4),
                      "shader_clock_ghz": round(f_clk / 1e9, 3),
                      "cycles_per_instruction_per_simd": round(t * f_clk * n_simd / n_ins, 2)})
    ops = {pk.HSP_VALU_EXP2: "v_exp_f32", pk.HSP_VALU_FMA: "v_fma_f32",
           pk.HSP_VALU_MAX3: "v_max3_f32", pk.HSP_VALU_CVT: "v_cvt_pk_bf16_f32",
           pk.HSP_VALU_SOFTMAX: "softmax_mix", pk.HSP_VALU_DOT2: "v_dot2c_f32_bf16"}
    for op in ops:
        for waves in (4, 8, 16):
            for chains in (8, 16):
                vit = 8192 * 8 // chains
                t = timed(lambda: pk.valu_loop(op, grid, waves, vit, out, clk, chains))
                # softmax mix: per 8 scores 8 FMA + 8 exp + 4 pack + 4 dot2 + 4 max3 = 28 ops
                per_round = chains * 28 // 8 if op == pk.HSP_VALU_SOFTMAX else chains
                n_ins = grid * waves * vit * per_round
                rec = {"peak": "valu_loop", "instruction": ops[op], "chains": chains,
                       "waves_per_simd": waves // 4, "ms": round(t * 1e3, 4),
                       "shader_clock_ghz": round(clock_hz() / 1e9, 3),
                       "cycles_per_wave_instruction_per_simd":
                           round(t * clock_hz() * n_simd / n_ins, 2)}
                if op == pk.HSP_VALU_SOFTMAX:
                    rec["cycles_per_score_per_simd"] = round(
                        t * clock_hz() * n_simd / (grid * waves * vit * chains * 64), 4)
                emit(rec)
    # Matrix core and vector ALU in one wave: 4 MFMAs (32x32x16) plus nops vector ops per round.
    mit = 2048
    for op in (pk.HSP_VALU_EXP2, pk.HSP_VALU_FMA):
        for waves in (4, 8):
            base = None
            for nops in (0, 8, 16, 32, 64):
                t = timed(lambda: pk.mix_wave(op, nops, grid, waves, mit, out, clk))
                rounds = grid * waves * mit / n_simd  # wave-rounds per SIMD
                cyc = t * clock_hz() / rounds
                base = base or cyc
                emit({"peak": "mix_wave", "vector_op": ops[op], "ops_per_4_mfma": nops,
                      "waves_per_simd": waves // 4, "ms": round(t * 1e3, 4),
                      "cycles_per_wave_round_per_simd": round(cyc, 1),
                      "extra_cycles_per_vector_op": round((cyc - base) / max(nops, 1), 2)})
    # Matrix waves and vector waves sharing each SIMD (one of each per SIMD).
    sit = 4096
    for op, vit in ((pk.HSP_VALU_EXP2, 4096), (pk.HSP_VALU_FMA, 8192), (pk.HSP_VALU_MAX3, 8192),
                    (pk.HSP_VALU_CVT, 8192), (pk.HSP_VALU_DOT2, 8192),
                    (pk.HSP_VALU_SOFTMAX, 2048)):
        res = {}
        for tag, m, e in (("mfma_only", sit, 0), ("valu_only", 0, vit), ("both", sit, vit)):
            res[tag] = timed(lambda: pk.mix_split(op, m, e, grid, out, clk))
        emit({"peak": "mix_split", "vector_op": ops[op], "mfma_rounds": sit, "valu_rounds": vit,
              "ms_mfma_only": round(res["mfma_only"] * 1e3, 4),
              "ms_valu_only": round(res["valu_only"] * 1e3, 4),
              "ms_both": round(res["both"] * 1e3, 4),
              "overlap": round((res["mfma_only"] + res["valu_only"] - res["both"])
                               / min(res["mfma_only"], res["valu_only"]), 3)})
    # Matrix phase and dependent vector phase in turn in every wave, one or two waves per SIMD.
    pit = 8192
    for vr in (2, 4, 8):
        for waves in (4, 8):
            res = {tag: timed(lambda: pk.mix_phase(part, waves, pit, vr, grid, out, clk))
                   for tag, part in (("matrix_only", 1), ("vector_only", 2), ("both", 0))}
            emit({"peak": "mix_phase", "vector_rounds": vr, "waves_per_simd": waves // 4,
                  "ms_matrix_only": round(res["matrix_only"] * 1e3, 4),
                  "ms_vector_only": round(res["vector_only"] * 1e3, 4),
                  "ms_both": round(res["both"] * 1e3, 4),
                  "overlap": round((res["matrix_only"] + res["vector_only"] - res["both"])
                                   / min(res["matrix_only"], res["vector_only"]), 3)})
    # LDS read bandwidth per CU (one workgroup per CU, 4 / 8 / 16 waves).
    for waves in (4, 8, 16):
        lit = 4096
        t = timed(lambda: pk.lds_read(grid, waves, lit, out, clk))
        nbytes_l = grid * waves * lit * 8 * 1024
        emit({"peak": "lds_read", "instruction": "ds_read_b128", "waves_per_cu": waves,
              "ms": round(t * 1e3, 4), "shader_clock_ghz": round(clock_hz() / 1e9, 3),
              "bytes_per_clock_per_cu": round(nbytes_l / (t * clock_hz() * 256), 1)})
    # Streaming HBM reads of 2 GiB.
    nbytes = 1 << 31
    src = torch.ones(nbytes // 4, device=dev, dtype=torch.float32)
    rout = torch.empty(4096 * 256, device=dev, dtype=torch.int32)
    if os.environ.get("HSP_SKIP_READ"):
        return 0
    for mode, tag in ((0, "registers_nt"), (1, "direct_to_lds"), (2, "direct_to_lds_nt")):
        for g in (512, 1024, 2048, 4096):
            t = timed(lambda: pk.read(mode, src, g, rout))
            emit({"peak": "read", "path": tag, "workgroups": g, "bytes": nbytes,
                  "ms": round(t * 1e3, 4), "gbs": round(nbytes / t / 1e9, 1),
                  "frac_of_8tbs": round(nbytes / t / 8e12, 4)})
    return 0


def main():
    args = parse()
    if args.cpu_leg:
        return cpu_leg(args.cpu_sample_heads)
    if args.summarize_counters:
        return summarize_counters(*args.summarize_counters)
    if args.peaks:
        return run_peaks()
    if args.suite:
        parts = args.suite.split(",")
        bad = [x for x in parts if x not in SUITE_PARTS]
        if bad:
            print(f"unknown suite part(s) {bad}; choose from {SUITE_PARTS}", file=sys.stderr)
            return 2
        return run_suite(parts)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        return 2

    # The CPU-oracle legs run first, as child processes, before this process initialises the GPU.
    cpu = None if args.no_cpu_baseline else cpu_legs(args.cpu_sample_heads)

    import numpy as np
    import torch
    from sparse_kv_cache_magnitude_amd import hierasparse as hs
    from sparse_kv_cache_magnitude_amd import synth

    w = synth.workload(WORKLOAD)
    G = w.hq // w.hkv
    dev = "cuda"
    stream = torch.cuda.current_stream()
    flags = hs.HS_PREFILL_SMFMAC if args.prefill_path == "smfmac" else hs.HS_PREFILL_DECOMPRESS

    if args.copy_probe:
        src = torch.ones(COPY_BYTES // 4, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    K, V, Q, q = make_inputs(w, torch, dev)
    shp = hs.shape(w.b, w.hq, w.hkv, w.L, w.D, w.B)
    cnt = hs.counts(w.n_p, w.n_sk, w.n_sv)
    cache = hs.alloc_cache(shp, cnt)
    ws_c = hs.alloc_workspace(hs.HS_OP_COMPRESS, shp, cnt)
    ws_d = hs.alloc_workspace(hs.HS_OP_DECODE, shp, cnt)
    O = torch.empty_like(Q)
    lse_p = torch.empty((w.b, w.hq, w.L), device=dev, dtype=torch.float32)
    o = torch.empty_like(q)
    lse_d = torch.empty((w.b, w.hq), device=dev, dtype=torch.float32)

    # The prefill writes a 2 GiB output; the dirty lines it leaves in the last-level cache would be
    # written back to HBM during whatever kernel runs next. A read pass over a buffer larger than
    # that cache, between prefill and decode (inside the step, outside both kernels' windows),
    # settles them, so the decode window measures the decode's own reads.
    settle = torch.ones(SETTLE_BYTES // 4, device=dev, dtype=torch.float32)

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        hs.hs_compress(shp, cnt, K, V, cache, ws_c)
        if ev:
            ev[1].record(stream)
        hs.hs_prefill_attn(shp, cnt, cache, Q, O, lse_p, 0.0, flags)
        if ev:
            ev[2].record(stream)
        settle.sum()
        if ev:
            ev[3].record(stream)
        hs.hs_decode_attn(shp, cnt, cache, q, o, lse_d, 0.0, 0, ws_d)
        if ev:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    comp_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    pre_ms = np.array([e[1].elapsed_time(e[2]) for e in events])
    dec_ms = np.array([e[3].elapsed_time(e[4]) for e in events])
    step_ms = np.array([e[0].elapsed_time(e[4]) for e in events])

    cache_bytes = hs.hs_cache_sizes(shp, cnt)
    map_k = cache["map_k"].cpu().numpy()
    map_v = cache["map_v"].cpu().numpy()
    d_bytes = decode_bytes(w, G)
    dense_eq, executed, full_causal = prefill_flops(w, map_k, map_v, flags == hs.HS_PREFILL_SMFMAC)
    c_bytes = compress_bytes(w, cache_bytes)

    dec_s = float(np.mean(dec_ms)) / 1e3
    pre_s = float(np.mean(pre_ms)) / 1e3
    comp_s = float(np.mean(comp_ms)) / 1e3
    decode_gbs = d_bytes / dec_s / 1e9
    pre_exec_tflops = executed / pre_s / 1e12
    pre_dense_eq_tflops = dense_eq / pre_s / 1e12

    out = {
        "metric": "decode attn µs & HBM GB/s at 32K ctx; prefill attn TFLOP/s; speedup vs dense",
        "value": round(decode_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(float(np.mean(step_ms)), 3),
        "wall_ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16 K/V/Q (4 key channels per KV head x8), no weights",
        "config": {"workload": WORKLOAD, "batch": w.b, "seq_len": w.L, "q_heads": w.hq,
                   "kv_heads": w.hkv, "head_dim": w.D, "block": w.B,
                   "blocks_per_head_dense_2to4_pruned": [w.nb - w.n_p - w.n_sk, w.n_sk, w.n_p],
                   "prefill_2to4_path": args.prefill_path},
        "decode_us": round(dec_s * 1e6, 2),
        "decode_bytes": d_bytes,
        "prefill_ms": round(pre_s * 1e3, 3),
        "prefill_tflops_dense_equivalent": round(pre_dense_eq_tflops, 1),
        "prefill_tflops_executed": round(pre_exec_tflops, 1),
        "prefill_flops": {"dense_equivalent": dense_eq, "executed": executed,
                          "full_causal_dense": full_causal},
        "compress_us": round(comp_s * 1e6, 2),
        "compress_share_of_prefill": round(comp_s / pre_s, 5),
        "roofline": {"bound": "mfma", "kernel": "k_prefill",
                     "achieved": round(pre_exec_tflops, 2), "peak": BF16_DENSE_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(pre_exec_tflops / BF16_DENSE_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("k_prefill", source_digest(
                         "hs_prefill.hip", "hs_device.h"))},
        "roofline_decode": {"bound": "hbm", "kernel": "k_decode_split+k_decode_combine",
                            "achieved": round(decode_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(decode_gbs / HBM_PEAK_GBS, 4),
                            "traffic": measured_traffic("k_decode_split", source_digest(
                                "hs_decode.hip", "hs_device.h"))},
        "roofline_compress": {"bound": "hbm", "kernel": "k_score+k_rank+k_pack",
                              "achieved": round(c_bytes / comp_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                              "unit": "GB/s",
                              "frac": round(c_bytes / comp_s / 1e9 / HBM_PEAK_GBS, 4)},
    }

    if not args.no_dense_baseline:
        # Same kernels, cache compressed with every block dense.
        cnt0 = hs.counts(0, 0, 0)
        cache0 = hs.alloc_cache(shp, cnt0)
        ws_c0 = hs.alloc_workspace(hs.HS_OP_COMPRESS, shp, cnt0)
        ws_d0 = hs.alloc_workspace(hs.HS_OP_DECODE, shp, cnt0)
        hs.hs_compress(shp, cnt0, K, V, cache0, ws_c0)
        del ws_c0
        reps = max(3, args.steps // 2)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
        for r in range(reps + 1):
            e = ev[r - 1] if r else None
            if e:
                e[0].record(stream)
            hs.hs_prefill_attn(shp, cnt0, cache0, Q, O, lse_p, 0.0, flags)
            if e:
                e[1].record(stream)
            settle.sum()
            if e:
                e[2].record(stream)
            hs.hs_decode_attn(shp, cnt0, cache0, q, o, lse_d, 0.0, 0, ws_d0)
            if e:
                e[3].record(stream)
        torch.cuda.synchronize()
        pre0 = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) / 1e3
        dec0 = float(np.mean([e[2].elapsed_time(e[3]) for e in ev])) / 1e3
        # The fastest dense prefill here: the decompress-path kernel on the dense cache (nothing to
        # expand; plain dense MFMA, no GEMM2 lag).
        other = hs.HS_PREFILL_DECOMPRESS if flags == hs.HS_PREFILL_SMFMAC else hs.HS_PREFILL_SMFMAC
        ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for r in range(reps + 1):
            e = ev2[r - 1] if r else None
            if e:
                e[0].record(stream)
            hs.hs_prefill_attn(shp, cnt0, cache0, Q, O, lse_p, 0.0, other)
            if e:
                e[1].record(stream)
        torch.cuda.synchronize()
        pre0_other = float(np.mean([e[0].elapsed_time(e[1]) for e in ev2])) / 1e3
        pre0_best = min(pre0, pre0_other)
        w0 = w.with_counts(0, 0, 0)
        out["dense_baseline"] = {
            "decode_us": round(dec0 * 1e6, 2),
            "decode_gbs": round(decode_bytes(w0, G) / dec0 / 1e9, 1),
            "prefill_ms": round(pre0 * 1e3, 3),
            "prefill_tflops": round(4 * w.D * w.L * (w.L + 1) / 2 * w.hq * w.b / pre0 / 1e12, 1),
            "prefill_ms_other_path": round(pre0_other * 1e3, 3)}
        out["speedup_vs_dense"] = {"decode": round(dec0 / dec_s, 3),
                                   "prefill": round(pre0 / pre_s, 3),
                                   "prefill_vs_fastest_dense": round(pre0_best / pre_s, 3),
                                   "decode_ideal_bytes": round(decode_bytes(w0, G) / d_bytes, 3),
                                   "prefill_ideal_flops": round(
                                       4 * w.D * w.L * (w.L + 1) / 2 * w.hq * w.b / executed, 3)}
        del cache0

    # Config-1 latency: one KV head, 4K tokens, every block 2:4, decode batch 1 (cache-resident,
    # so latency only; median of 21 event windows, no settle pass).
    w1 = synth.workload("decode_1h_4k_all24")
    K1, V1, _, q1 = make_inputs(w1, torch, dev)
    shp1, cnt1 = hs.shape(w1.b, w1.hq, w1.hkv, w1.L, w1.D, w1.B), hs.counts(*w1.counts())
    cache1 = hs.alloc_cache(shp1, cnt1)
    hs.hs_compress(shp1, cnt1, K1, V1, cache1, hs.alloc_workspace(hs.HS_OP_COMPRESS, shp1, cnt1))
    ws1, o1 = hs.alloc_workspace(hs.HS_OP_DECODE, shp1, cnt1), torch.empty_like(q1)
    t1 = []
    for r in range(22):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        hs.hs_decode_attn(shp1, cnt1, cache1, q1, o1, None, 0.0, 0, ws1)
        b.record(stream)
        torch.cuda.synchronize()
        if r:
            t1.append(a.elapsed_time(b) * 1e3)
    out["config1_decode_us"] = {"workload": w1.name, "median_us": round(float(np.median(t1)), 2),
                                "min_us": round(float(np.min(t1)), 2)}

    if cpu is not None:
        all_t, one_t = cpu
        prefill_all = all_t.pop("prefill_16k")
        prefill_one = one_t.pop("prefill_16k")
        out["cpu_baseline"] = all_t
        out["cpu_baseline_1thread"] = one_t
        out["cpu_prefill_16k_extrapolated"] = {
            "all_threads": {**prefill_all, "cores": all_t["cores"]},
            "one_thread": {**prefill_one, "cores": 1}}

    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
