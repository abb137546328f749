"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every entry point the
header declares, computes buffer sizes that match the oracle's closed-form pool sizes, and rejects
every invalid argument before anything is launched.

Only argument combinations that fail host validation are passed with placeholder pointers, so no
call here reaches a HIP launch.
"""
import ctypes
import os
import re

import pytest

import oracle
from oracle import Dims
from sparse_kv_cache_magnitude_amd import hierasparse as hs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hierasparse.h")

FAKE = 1 << 20          # aligned placeholder address, never dereferenced (validation fails first)
MISALIGNED = FAKE + 8


def declared_entry_points():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hs_[a-z_0-9]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared_entry_points() == sorted(hs.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(hs.LIB_PATH)
    for name in declared_entry_points():
        assert hasattr(lib, name), name


def test_peaks_library_exports_every_declared_symbol():
    """The measurement library (include/hs_peaks.h): header, binding and exports agree."""
    from sparse_kv_cache_magnitude_amd import peaks
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "hs_peaks.h")).read(),
                 flags=re.S)
    declared = sorted(set(re.findall(r"\b(hsp_[a-z_0-9]+)\s*\(", src)))
    assert declared == sorted(peaks.EXPORTS)
    lib = ctypes.CDLL(peaks.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


@pytest.mark.parametrize("b,hq,hkv,L,B,counts", [
    (8, 32, 8, 32768, 64, (77, 307, 307)),
    (1, 32, 8, 16384, 128, (0, 90, 90)),
    (4, 32, 8, 131072, 64, (819, 1024, 1024)),
    (3, 6, 2, 9 * 64, 64, (2, 3, 7)),
])
def test_cache_sizes_match_oracle_pools(b, hq, hkv, L, B, counts):
    got = hs.hs_cache_sizes(hs.shape(b, hq, hkv, L, 128, B), hs.counts(*counts))
    want = oracle.pool_bytes(Dims(b, hkv, L, 128, B, *counts))
    assert got == want


def test_workspace_sizes():
    shp, cnt = hs.shape(2, 8, 2, 1024, 128, 64), hs.counts(1, 3, 4)
    assert hs.hs_workspace_size(hs.HS_OP_COMPRESS, shp, cnt) == 2 * 2 * 16 * 3 * 8
    for s in (1, 7, 512):
        # the fp32 partial output (head_dim) and log-sum-exp per (batch, query head, split)
        assert hs.hs_workspace_size(hs.HS_OP_DECODE, shp, cnt, s) == 2 * 8 * s * (128 + 1) * 4
    assert hs.hs_workspace_size(hs.HS_OP_DECODE, shp, cnt, 0) > 0
    # dense K and V bf16 of the whole shape, then the compressor's keys
    assert hs.hs_workspace_size(hs.HS_OP_RECOMPRESS, shp, cnt) == \
        2 * (2 * 2 * 1024 * 128 * 2) + 2 * 2 * 16 * 3 * 8


def _status(call):
    try:
        call()
    except hs.HsError as e:
        return e.status
    return hs.HS_OK


BAD_SHAPES = [
    (hs.shape(1, 4, 1, 1024, 64, 64), hs.HS_ERR_SHAPE),       # head_dim != 128
    (hs.shape(1, 4, 1, 1024, 128, 32), hs.HS_ERR_SHAPE),      # block not 64/128
    (hs.shape(1, 4, 1, 1024, 128, 64, dtype=2), hs.HS_ERR_SHAPE),  # unknown element type
    (hs.shape(1, 4, 1, 1000, 128, 64), hs.HS_ERR_SHAPE),      # seq_len % block
    (hs.shape(1, 6, 4, 1024, 128, 64), hs.HS_ERR_SHAPE),      # q_heads % kv_heads
    (hs.shape(0, 4, 1, 1024, 128, 64), hs.HS_ERR_SHAPE),      # empty batch
    (hs.shape(1, 4, 1, 64 * 4097, 128, 64), hs.HS_ERR_SHAPE),  # too many blocks per head
]


@pytest.mark.parametrize("shp,code", BAD_SHAPES)
def test_bad_shapes_rejected_by_every_entry_point(shp, code):
    cnt = hs.counts(0, 0, 0)
    assert _status(lambda: hs.hs_cache_sizes(shp, cnt)) == code
    assert _status(lambda: hs.hs_workspace_size(hs.HS_OP_DECODE, shp, cnt)) == code
    cache = {f: FAKE for f in hs.CACHE_FIELDS}
    assert _status(lambda: _compress(shp, cnt, FAKE, FAKE, cache, FAKE, 1 << 30)) == code
    assert _status(lambda: _decode(shp, cnt, cache, FAKE, FAKE, None, 0, FAKE, 1 << 30)) == code
    assert _status(lambda: _prefill(shp, cnt, cache, FAKE, FAKE, None, 0)) == code
    assert _status(lambda: _prefill_variant(shp, cnt, cache, FAKE, FAKE, None, 0)) == code
    assert hs.hs_last_error() != ""


@pytest.mark.parametrize("counts", [(-1, 0, 0), (0, 17, 0), (8, 0, 9), (16, 1, 0)])
def test_bad_counts_rejected(counts):
    shp = hs.shape(1, 4, 1, 1024, 128, 64)   # 16 blocks per head
    assert _status(lambda: hs.hs_cache_sizes(shp, hs.counts(*counts))) == hs.HS_ERR_COUNTS


# ---- raw calls with placeholder addresses (validation must fail before any launch) ----------

def _cache_struct(cache):
    return hs.HsCache(*[ctypes.c_void_p(cache[f]) if cache.get(f) else None
                        for f in hs.CACHE_FIELDS])


def _raise(st):
    if st != hs.HS_OK:
        raise hs.HsError(st, hs.hs_last_error())


def _compress(shp, cnt, k, v, cache, ws, ws_bytes):
    _raise(hs.lib().hs_compress(ctypes.byref(shp), ctypes.byref(cnt), k, v,
                                ctypes.byref(_cache_struct(cache)), ws, ws_bytes, None))


def _recompress(shp, cin, cache_in, cout, cache_out, ws, ws_bytes):
    _raise(hs.lib().hs_recompress(ctypes.byref(shp), ctypes.byref(cin),
                                  ctypes.byref(_cache_struct(cache_in)), ctypes.byref(cout),
                                  ctypes.byref(_cache_struct(cache_out)), ws, ws_bytes, None))


def _decode(shp, cnt, cache, q, o, lse, splits, ws, ws_bytes):
    _raise(hs.lib().hs_decode_attn(ctypes.byref(shp), ctypes.byref(cnt),
                                   ctypes.byref(_cache_struct(cache)), q, o, lse, 0.0, splits,
                                   ws, ws_bytes, None))


def _prefill(shp, cnt, cache, q, o, lse, flags):
    _raise(hs.lib().hs_prefill_attn(ctypes.byref(shp), ctypes.byref(cnt),
                                    ctypes.byref(_cache_struct(cache)), q, o, lse, 0.0, flags,
                                    None))


def _prefill_variant(shp, cnt, cache, q, o, lse, variant):
    _raise(hs.lib().hs_prefill_attn_variant(ctypes.byref(shp), ctypes.byref(cnt),
                                            ctypes.byref(_cache_struct(cache)), q, o, lse, 0.0,
                                            variant, None))


SHP, CNT = hs.shape(1, 4, 1, 1024, 128, 64), hs.counts(2, 4, 5)


def test_null_pointers_rejected():
    cache = {f: FAKE for f in hs.CACHE_FIELDS}
    assert _status(lambda: _compress(SHP, CNT, None, FAKE, cache, FAKE, 1 << 30)) == hs.HS_ERR_NULL
    assert _status(lambda: _compress(SHP, CNT, FAKE, None, cache, FAKE, 1 << 30)) == hs.HS_ERR_NULL
    for f in hs.CACHE_FIELDS:
        c = dict(cache, **{f: None})
        assert _status(lambda: _compress(SHP, CNT, FAKE, FAKE, c, FAKE, 1 << 30)) == hs.HS_ERR_NULL
        assert _status(lambda: _decode(SHP, CNT, c, FAKE, FAKE, None, 0, FAKE, 1 << 30)) \
            == hs.HS_ERR_NULL
        assert _status(lambda: _prefill(SHP, CNT, c, FAKE, FAKE, None, 0)) == hs.HS_ERR_NULL
    assert _status(lambda: _decode(SHP, CNT, cache, None, FAKE, None, 0, FAKE, 1 << 30)) \
        == hs.HS_ERR_NULL
    assert _status(lambda: _prefill(SHP, CNT, cache, FAKE, None, None, 0)) == hs.HS_ERR_NULL


def test_misaligned_pointers_rejected():
    cache = {f: FAKE for f in hs.CACHE_FIELDS}
    assert _status(lambda: _compress(SHP, CNT, MISALIGNED, FAKE, cache, FAKE, 1 << 30)) \
        == hs.HS_ERR_ALIGN
    c = dict(cache, v_meta=MISALIGNED)
    assert _status(lambda: _decode(SHP, CNT, c, FAKE, FAKE, None, 0, FAKE, 1 << 30)) \
        == hs.HS_ERR_ALIGN
    assert _status(lambda: _prefill(SHP, CNT, cache, FAKE, FAKE, MISALIGNED, 0)) \
        == hs.HS_ERR_ALIGN


def test_workspace_checks():
    cache = {f: FAKE for f in hs.CACHE_FIELDS}
    need = hs.hs_workspace_size(hs.HS_OP_COMPRESS, SHP, CNT)
    assert _status(lambda: _compress(SHP, CNT, FAKE, FAKE, cache, FAKE, need - 1)) \
        == hs.HS_ERR_WORKSPACE
    assert _status(lambda: _compress(SHP, CNT, FAKE, FAKE, cache, None, need)) \
        == hs.HS_ERR_WORKSPACE
    need = hs.hs_workspace_size(hs.HS_OP_DECODE, SHP, CNT, 3)
    assert _status(lambda: _decode(SHP, CNT, cache, FAKE, FAKE, None, 3, FAKE, need - 4)) \
        == hs.HS_ERR_WORKSPACE
    assert _status(lambda: _decode(SHP, CNT, cache, FAKE, FAKE, None, 513, FAKE, 1 << 30)) \
        == hs.HS_ERR_SHAPE


def test_decode_noalloc_checks():
    """The allocation-free decode rejects, before touching the GPU, every call the plain decode
    rejects, and every call whose workspace would not fit its fixed scratch array."""
    cache = {f: FAKE for f in hs.CACHE_FIELDS}
    call = lambda shp, cnt, c=cache, q=FAKE, splits=0: _status(lambda: _raise(
        hs.lib().hs_decode_attn_noalloc(ctypes.byref(shp), ctypes.byref(cnt),
                                        ctypes.byref(_cache_struct(c)), q, FAKE, None, 0.0,
                                        splits, None)))
    assert call(SHP, CNT, q=None) == hs.HS_ERR_NULL
    assert call(SHP, CNT, q=MISALIGNED) == hs.HS_ERR_ALIGN
    assert call(SHP, CNT, splits=513) == hs.HS_ERR_SHAPE
    assert call(SHP, hs.counts(-1, 0, 0)) == hs.HS_ERR_COUNTS
    # 64 x 32 query heads x 512 splits of 129 floats: far beyond the 16 MiB array
    big = hs.shape(64, 32, 8, 64 * 1024, 128, 64)
    assert hs.hs_workspace_size(hs.HS_OP_DECODE, big, hs.counts(0, 0, 0), 512) > \
        hs.HS_DECODE_NOALLOC_SCRATCH_BYTES
    assert call(big, hs.counts(0, 0, 0), splits=512) == hs.HS_ERR_WORKSPACE
    assert "scratch" in hs.hs_last_error()


def _compress_ex(shp, cnt, pol, k, v, cache, ws, ws_bytes):
    _raise(hs.lib().hs_compress_ex(ctypes.byref(shp), ctypes.byref(cnt),
                                   ctypes.byref(pol) if pol is not None else None, k, v,
                                   ctypes.byref(_cache_struct(cache)), ws, ws_bytes, None))


def test_compress_ex_policy_validation():
    cache = {f: FAKE for f in hs.CACHE_FIELDS}
    shp = hs.shape(1, 4, 1, 1024, 128, 64)                       # 16 blocks
    need = hs.hs_workspace_size(hs.HS_OP_COMPRESS, shp, hs.counts(2, 4, 5))
    call = lambda cnt, pol, n=need, k=FAKE: \
        _status(lambda: _compress_ex(shp, cnt, pol, k, FAKE, cache, FAKE, n))
    # sink 64 + local 256 hold 1 + 4 blocks: 11 are ranked
    assert call(hs.counts(2, 10, 0), hs.policy(64, 256)) == hs.HS_ERR_COUNTS
    assert call(hs.counts(2, 0, 10), hs.policy(64, 256)) == hs.HS_ERR_COUNTS
    assert call(hs.counts(1, 10, 0), hs.policy(65, 256)) == hs.HS_ERR_COUNTS   # sink spills over
    assert call(hs.counts(0, 0, 0), hs.policy(-1, 0)) == hs.HS_ERR_COUNTS
    assert call(hs.counts(0, 0, 0), hs.policy(0, 1025)) == hs.HS_ERR_COUNTS
    # counts that fit pass the policy check and fail on the next invalid argument
    assert call(hs.counts(1, 10, 10), hs.policy(64, 256), k=None) == hs.HS_ERR_NULL
    assert call(hs.counts(0, 0, 0), hs.policy(1024, 1024), k=None) == hs.HS_ERR_NULL
    assert call(hs.counts(2, 4, 5), hs.policy(64, 256), n=need - 8) == hs.HS_ERR_WORKSPACE
    assert call(hs.counts(2, 4, 5), None, n=need - 8) == hs.HS_ERR_WORKSPACE


def _masked(shp, cnt, k, v, mk, mv, cache, status):
    _raise(hs.lib().hs_compress_masked(ctypes.byref(shp), ctypes.byref(cnt), k, v, mk, mv,
                                       ctypes.byref(_cache_struct(cache)), status, None))


def test_compress_masked_validation():
    cache = {f: FAKE for f in hs.CACHE_FIELDS}
    call = lambda shp=SHP, cnt=CNT, k=FAKE, v=FAKE, mk=FAKE, mv=FAKE, c=cache, st=MISALIGNED: \
        _status(lambda: _masked(shp, cnt, k, v, mk, mv, c, st))
    # head_status is optional but, when given, must be aligned: every call below fails before
    # a launch because one argument is invalid
    assert call() == hs.HS_ERR_ALIGN
    for name in ("k", "v", "mk", "mv"):
        assert call(**{name: None}) == hs.HS_ERR_NULL, name
        assert call(**{name: MISALIGNED}) == hs.HS_ERR_ALIGN, name
    for f in hs.CACHE_FIELDS:
        assert call(c=dict(cache, **{f: None}), st=None) == hs.HS_ERR_NULL
    assert call(cnt=hs.counts(9, 8, 0), st=None) == hs.HS_ERR_COUNTS
    assert call(shp=hs.shape(1, 4, 1, 1024, 128, 32), st=None) == hs.HS_ERR_SHAPE


def _disjoint_caches():
    """Placeholder input and output caches whose arrays are far apart, and a workspace address."""
    cin = {f: (1 << 40) + (i << 32) for i, f in enumerate(hs.CACHE_FIELDS)}
    cout = {f: (1 << 41) + (i << 32) for i, f in enumerate(hs.CACHE_FIELDS)}
    return cin, cout, 1 << 42


def test_recompress_validation():
    cin, cout, ws = _disjoint_caches()
    c2 = hs.counts(2, 6, 6)
    need = hs.hs_workspace_size(hs.HS_OP_RECOMPRESS, SHP, c2)
    call = lambda shp=SHP, a=CNT, ca=cin, b=c2, cb=cout, w=ws, n=need: \
        _status(lambda: _recompress(shp, a, ca, b, cb, w, n))
    assert call(n=need - 1) == hs.HS_ERR_WORKSPACE
    assert call(w=None) == hs.HS_ERR_WORKSPACE
    assert call(w=ws + 8) == hs.HS_ERR_ALIGN
    assert call(a=hs.counts(10, 7, 0)) == hs.HS_ERR_COUNTS
    assert call(b=hs.counts(0, 17, 0)) == hs.HS_ERR_COUNTS
    assert call(shp=hs.shape(1, 4, 1, 1000, 128, 64)) == hs.HS_ERR_SHAPE
    for f in hs.CACHE_FIELDS:
        assert call(ca=dict(cin, **{f: None})) == hs.HS_ERR_NULL
        assert call(cb=dict(cout, **{f: None})) == hs.HS_ERR_NULL
        assert call(cb=dict(cout, **{f: cout[f] + 8})) == hs.HS_ERR_ALIGN
    # any shared byte between an input array, an output array and the workspace is refused
    for f in hs.CACHE_FIELDS:
        for g in hs.CACHE_FIELDS:
            assert call(cb=dict(cout, **{g: cin[f] + 16})) == hs.HS_ERR_OVERLAP, (f, g)
        assert call(w=cin[f]) == hs.HS_ERR_OVERLAP
        assert call(w=cout[f] - need + 16) == hs.HS_ERR_OVERLAP
    assert "overlap" in hs.hs_last_error()


def test_unknown_flags_and_ops():
    cache = {f: FAKE for f in hs.CACHE_FIELDS}
    assert _status(lambda: _prefill(SHP, CNT, cache, FAKE, FAKE, None, 7)) == hs.HS_ERR_UNSUPPORTED
    assert _status(lambda: hs.hs_workspace_size(9, SHP, CNT)) == hs.HS_ERR_UNSUPPORTED


def test_prefill_variant_validation():
    cache = {f: FAKE for f in hs.CACHE_FIELDS}
    for v in (3, 5, 32, 0xFFFFFFFF):
        assert _status(lambda: _prefill_variant(SHP, CNT, cache, FAKE, FAKE, None, v)) == \
            hs.HS_ERR_UNSUPPORTED
    # fp16 elements and heads of more than 2048 blocks have no variants
    f16 = hs.shape(1, 4, 1, 1024, 128, 64, dtype=hs.HS_F16)
    assert _status(lambda: _prefill_variant(f16, CNT, cache, FAKE, FAKE, None, 1)) == \
        hs.HS_ERR_UNSUPPORTED
    long_head = hs.shape(1, 4, 1, 64 * 2049, 128, 64)
    assert _status(lambda: _prefill_variant(long_head, hs.counts(0, 0, 0), cache, FAKE, FAKE,
                                            None, 2)) == hs.HS_ERR_UNSUPPORTED
    assert "variant" in hs.hs_last_error()
    mid_head = hs.shape(1, 4, 1, 64 * 1025, 128, 64)
    assert _status(lambda: _prefill_variant(mid_head, hs.counts(0, 0, 0), cache, FAKE, FAKE,
                                            None, 16)) == hs.HS_ERR_UNSUPPORTED
    assert _status(lambda: _prefill_variant(SHP, CNT, cache, None, FAKE, None, 0)) == \
        hs.HS_ERR_NULL


def test_status_strings():
    for code in range(9):
        assert hs.hs_status_string(code) not in ("", "unknown status")
