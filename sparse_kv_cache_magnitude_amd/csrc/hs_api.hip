// hs_api.hip -- the C ABI of libhierasparse.so (declared in include/hierasparse.h).
//
// Host side: validates every argument before anything is enqueued, computes buffer sizes, and
// launches the gfx950 kernels of hs_compress.hip, hs_decode.hip and hs_prefill.hip on the caller's
// stream. The library allocates nothing: scratch comes from the caller, except for
// hs_decode_attn_noalloc, whose scratch is a fixed device array declared here.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "hierasparse.h"
#include "hs_internal.h"

#define HS_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_error[512] = "";

hs_status fail(hs_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof g_error, fmt, ap);
  va_end(ap);
  return s;
}

hs_status ok() {
  g_error[0] = '\0';
  return HS_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Shape and count rules shared by all entry points.
hs_status make_dims(const hs_shape *s, const hs_counts *c, hs::Dims *d) {
  if (!s || !c) return fail(HS_ERR_NULL, "shape or counts is NULL");
  if (s->batch <= 0 || s->q_heads <= 0 || s->kv_heads <= 0 || s->seq_len <= 0)
    return fail(HS_ERR_SHAPE, "batch, q_heads, kv_heads and seq_len must be positive");
  if (s->q_heads % s->kv_heads)
    return fail(HS_ERR_SHAPE, "q_heads (%d) must be a multiple of kv_heads (%d)", s->q_heads,
                s->kv_heads);
  if (s->head_dim != 128) return fail(HS_ERR_SHAPE, "head_dim must be 128 (got %d)", s->head_dim);
  if (s->dtype != HS_BF16 && s->dtype != HS_F16)
    return fail(HS_ERR_SHAPE, "dtype must be HS_BF16 or HS_F16 (got %d)", s->dtype);
  if (s->block != 64 && s->block != 128)
    return fail(HS_ERR_SHAPE, "block must be 64 or 128 (got %d)", s->block);
  if (s->seq_len % s->block)
    return fail(HS_ERR_SHAPE, "seq_len (%d) must be a multiple of block (%d)", s->seq_len,
                s->block);
  const int nb = s->seq_len / s->block;
  if (nb > hs::kMaxBlocks)
    return fail(HS_ERR_SHAPE, "seq_len / block = %d exceeds %d blocks per head", nb,
                hs::kMaxBlocks);
  if ((int64_t)s->batch * s->kv_heads > 65535 || (int64_t)s->batch * s->q_heads > 65535)
    return fail(HS_ERR_SHAPE, "batch * heads exceeds 65535");
  if (c->n_pruned < 0 || c->n_sparse_k < 0 || c->n_sparse_v < 0)
    return fail(HS_ERR_COUNTS, "block counts must be non-negative");
  if (c->n_pruned + c->n_sparse_k > nb || c->n_pruned + c->n_sparse_v > nb)
    return fail(HS_ERR_COUNTS, "n_pruned + n_sparse_{k,v} exceeds the %d blocks per head", nb);
  d->b = s->batch;
  d->hq = s->q_heads;
  d->hkv = s->kv_heads;
  d->G = s->q_heads / s->kv_heads;
  d->L = s->seq_len;
  d->D = s->head_dim;
  d->B = s->block;
  d->nb = nb;
  d->np = c->n_pruned;
  d->nsk = c->n_sparse_k;
  d->nsv = c->n_sparse_v;
  d->ndk = nb - c->n_pruned - c->n_sparse_k;
  d->ndv = nb - c->n_pruned - c->n_sparse_v;
  d->dtype = s->dtype == HS_F16 ? hs::kF16 : hs::kBf16;
  return HS_OK;
}

hs_cache_bytes cache_bytes(const hs::Dims &d) {
  const size_t heads = (size_t)d.b * d.hkv, bd = (size_t)d.B * d.D;
  hs_cache_bytes r;
  r.map_k = r.map_v = heads * d.nb * sizeof(int32_t);
  r.k_dense = heads * d.ndk * bd * 2;
  r.k_nnz = heads * d.nsk * bd;          // bd / 2 values of 2 bytes
  r.k_meta = heads * d.nsk * bd / 8;     // bd / 16 words of 2 bytes
  r.v_dense = heads * d.ndv * bd * 2;
  r.v_nnz = heads * d.nsv * bd;
  r.v_meta = heads * d.nsv * bd / 8;
  return r;
}

// The pointers of a cache: non-NULL and aligned wherever the buffer is non-empty.
hs_status check_cache(const hs_cache *c, const hs::Dims &d, hs::CacheView *v) {
  if (!c) return fail(HS_ERR_NULL, "cache is NULL");
  const hs_cache_bytes n = cache_bytes(d);
  const void *p[8] = {c->map_k, c->map_v, c->k_dense, c->k_nnz,
                      c->k_meta, c->v_dense, c->v_nnz, c->v_meta};
  const size_t sz[8] = {n.map_k, n.map_k, n.k_dense, n.k_nnz, n.k_meta, n.v_dense, n.v_nnz, n.v_meta};
  static const char *names[8] = {"map_k", "map_v", "k_dense", "k_nnz",
                                 "k_meta", "v_dense", "v_nnz", "v_meta"};
  for (int i = 0; i < 8; ++i) {
    if (sz[i] && !p[i]) return fail(HS_ERR_NULL, "cache.%s is NULL", names[i]);
    if (!aligned16(p[i])) return fail(HS_ERR_ALIGN, "cache.%s is not 16-byte aligned", names[i]);
  }
  *v = hs::CacheView{c->map_k, c->map_v, c->k_dense, c->k_nnz,
                     c->k_meta, c->v_dense, c->v_nnz, c->v_meta};
  return HS_OK;
}

hs_status check_ptr(const void *p, const char *name, bool required = true) {
  if (!p) return required ? fail(HS_ERR_NULL, "%s is NULL", name) : HS_OK;
  if (!aligned16(p)) return fail(HS_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return HS_OK;
}

// Split-KV factor of the decode: the split kernel runs one wave per workgroup and two workgroups
// per CU, so aim for 512 workgroups (two per CU on 256 CUs), with at least two visible blocks per
// split.
int auto_splits(const hs::Dims &d) {
  const int units = d.b * d.hkv * ((d.G + 15) / 16);
  const int visible = d.nb - d.np;
  int s = (512 + units - 1) / units;
  const int cap = (visible + 1) / 2;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  if (s > 512) s = 512;
  return s;
}

// Decode workspace: the fp32 partial outputs and log-sum-exps of every split.
size_t decode_ws_bytes(const hs::Dims &d, int splits) {
  const size_t rows = (size_t)d.b * d.hq * splits;
  return rows * d.D * sizeof(float) + rows * sizeof(float);
}

size_t compress_ws_bytes(const hs::Dims &d) { return (size_t)d.b * d.hkv * d.nb * 3 * sizeof(uint64_t); }

// Byte ranges [p, p + n) of a cache's eight arrays (empty arrays have n = 0).
struct Ranges {
  const char *p[8];
  size_t n[8];
};
Ranges cache_ranges(const hs_cache *c, const hs::Dims &d) {
  const hs_cache_bytes b = cache_bytes(d);
  return Ranges{{(const char *)c->map_k, (const char *)c->map_v, (const char *)c->k_dense,
                 (const char *)c->k_nnz, (const char *)c->k_meta, (const char *)c->v_dense,
                 (const char *)c->v_nnz, (const char *)c->v_meta},
                {b.map_k, b.map_k, b.k_dense, b.k_nnz, b.k_meta, b.v_dense, b.v_nnz, b.v_meta}};
}
bool overlap(const char *a, size_t na, const char *b, size_t nb) {
  return na && nb && a < b + nb && b < a + na;
}

// Re-compression workspace: dense K and V of the shape, then the compressor's keys.
size_t dense_bytes(const hs::Dims &d) { return (size_t)d.b * d.hkv * d.L * d.D * sizeof(uint16_t); }
size_t recompress_ws_bytes(const hs::Dims &d) { return 2 * dense_bytes(d) + compress_ws_bytes(d); }

float scale_log2(float softmax_scale, int D) {
  float s = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
  return s * 1.4426950408889634f;
}

}  // namespace

HS_API hs_status hs_cache_sizes(const hs_shape *shape, const hs_counts *counts,
                                hs_cache_bytes *out) {
  hs::Dims d;
  hs_status st = make_dims(shape, counts, &d);
  if (st) return st;
  if (!out) return fail(HS_ERR_NULL, "out is NULL");
  *out = cache_bytes(d);
  return ok();
}

HS_API hs_status hs_workspace_size(int op, const hs_shape *shape, const hs_counts *counts,
                                   int32_t num_splits, size_t *bytes) {
  hs::Dims d;
  hs_status st = make_dims(shape, counts, &d);
  if (st) return st;
  if (!bytes) return fail(HS_ERR_NULL, "bytes is NULL");
  if (op == HS_OP_COMPRESS) {
    *bytes = compress_ws_bytes(d);
  } else if (op == HS_OP_RECOMPRESS) {
    *bytes = recompress_ws_bytes(d);
  } else if (op == HS_OP_DECODE) {
    if (num_splits < 0 || num_splits > 512)
      return fail(HS_ERR_SHAPE, "num_splits must be in 0..512 (got %d)", num_splits);
    *bytes = decode_ws_bytes(d, num_splits ? num_splits : auto_splits(d));
  } else {
    return fail(HS_ERR_UNSUPPORTED, "unknown op %d", op);
  }
  return ok();
}

HS_API hs_status hs_compress_ex(const hs_shape *shape, const hs_counts *counts,
                                const hs_policy *policy, const uint16_t *k, const uint16_t *v,
                                const hs_cache *out, void *ws, size_t ws_bytes, void *stream) {
  hs::Dims d;
  hs::CacheView c;
  hs_status st = make_dims(shape, counts, &d);
  if (st) return st;
  // Blocks [dense_lo, dense_hi) are ranked; the others hold sink or local-window tokens.
  int dense_lo = 0, dense_hi = d.nb;
  if (policy) {
    const int sink = policy->sink_tokens, local = policy->local_tokens;
    if (sink < 0 || local < 0 || sink > d.L || local > d.L)
      return fail(HS_ERR_COUNTS, "sink_tokens (%d) and local_tokens (%d) must be in 0..seq_len",
                  sink, local);
    dense_lo = (sink + d.B - 1) / d.B;
    dense_hi = (d.L - local) / d.B;
    const int ranked = dense_hi > dense_lo ? dense_hi - dense_lo : 0;
    if (d.np + d.nsk > ranked || d.np + d.nsv > ranked)
      return fail(HS_ERR_COUNTS,
                  "n_pruned + n_sparse_{k,v} exceeds the %d blocks outside the dense policy",
                  ranked);
    if (ranked == 0) dense_hi = dense_lo;
  }
  if ((st = check_ptr(k, "k")) || (st = check_ptr(v, "v"))) return st;
  if ((st = check_cache(out, d, &c))) return st;
  if (!ws || ws_bytes < compress_ws_bytes(d))
    return fail(HS_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", compress_ws_bytes(d),
                ws_bytes, ws ? "" : ", NULL");
  if (!aligned16(ws)) return fail(HS_ERR_ALIGN, "workspace is not 16-byte aligned");
  hipError_t e = hs::launch_compress(d, k, v, c, (uint64_t *)ws, (hipStream_t)stream, dense_lo,
                                     dense_hi);
  if (e != hipSuccess) return fail(HS_ERR_HIP, "compress launch: %s", hipGetErrorString(e));
  return ok();
}

HS_API hs_status hs_compress(const hs_shape *shape, const hs_counts *counts, const uint16_t *k,
                             const uint16_t *v, const hs_cache *out, void *ws, size_t ws_bytes,
                             void *stream) {
  return hs_compress_ex(shape, counts, nullptr, k, v, out, ws, ws_bytes, stream);
}

HS_API hs_status hs_compress_masked(const hs_shape *shape, const hs_counts *counts,
                                    const uint16_t *k, const uint16_t *v, const uint8_t *mode_k,
                                    const uint8_t *mode_v, const hs_cache *out,
                                    int32_t *head_status, void *stream) {
  hs::Dims d;
  hs::CacheView c;
  hs_status st = make_dims(shape, counts, &d);
  if (st) return st;
  if ((st = check_ptr(k, "k")) || (st = check_ptr(v, "v"))) return st;
  if ((st = check_ptr(mode_k, "mode_k")) || (st = check_ptr(mode_v, "mode_v"))) return st;
  if ((st = check_ptr(head_status, "head_status", false))) return st;
  if ((st = check_cache(out, d, &c))) return st;
  hipError_t e = hs::launch_modes(d, mode_k, mode_v, c, head_status, (hipStream_t)stream);
  if (e == hipSuccess) e = hs::launch_pack(d, k, v, c, (hipStream_t)stream);
  if (e != hipSuccess) return fail(HS_ERR_HIP, "masked compress launch: %s", hipGetErrorString(e));
  return ok();
}

HS_API hs_status hs_recompress(const hs_shape *shape, const hs_counts *in_counts,
                               const hs_cache *in, const hs_counts *out_counts,
                               const hs_cache *out, void *ws, size_t ws_bytes, void *stream) {
  hs::Dims din, dout;
  hs::CacheView cin, cout;
  hs_status st = make_dims(shape, in_counts, &din);
  if (st) return st;
  if ((st = make_dims(shape, out_counts, &dout))) return st;
  if ((st = check_cache(in, din, &cin))) return st;
  if ((st = check_cache(out, dout, &cout))) return st;
  const size_t need = recompress_ws_bytes(dout);
  if (!ws || ws_bytes < need)
    return fail(HS_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need, ws_bytes,
                ws ? "" : ", NULL");
  if (!aligned16(ws)) return fail(HS_ERR_ALIGN, "workspace is not 16-byte aligned");
  const Ranges ri = cache_ranges(in, din), ro = cache_ranges(out, dout);
  for (int i = 0; i < 8; ++i) {
    if (overlap(ri.p[i], ri.n[i], (const char *)ws, need) ||
        overlap(ro.p[i], ro.n[i], (const char *)ws, need))
      return fail(HS_ERR_OVERLAP, "workspace overlaps a cache array");
    for (int j = 0; j < 8; ++j)
      if (overlap(ri.p[i], ri.n[i], ro.p[j], ro.n[j]))
        return fail(HS_ERR_OVERLAP, "input and output caches overlap");
  }
  uint16_t *kd = (uint16_t *)ws;
  uint16_t *vd = kd + dense_bytes(dout) / sizeof(uint16_t);
  uint64_t *keys = (uint64_t *)(vd + dense_bytes(dout) / sizeof(uint16_t));
  hipError_t e = hs::launch_unpack(din, cin, kd, vd, (hipStream_t)stream);
  if (e == hipSuccess) e = hs::launch_compress(dout, kd, vd, cout, keys, (hipStream_t)stream);
  if (e != hipSuccess) return fail(HS_ERR_HIP, "recompress launch: %s", hipGetErrorString(e));
  return ok();
}

// Arguments of a decode call, checked; the workspace is checked by the caller.
struct DecodeCall {
  hs::Dims d;
  hs::CacheView c;
  int splits;
  size_t need;  // workspace bytes
};
static hs_status check_decode(const hs_shape *shape, const hs_counts *counts,
                              const hs_cache *cache, const uint16_t *q, const uint16_t *o,
                              const float *lse, int32_t num_splits, DecodeCall *dc) {
  hs_status st = make_dims(shape, counts, &dc->d);
  if (st) return st;
  if ((st = check_cache(cache, dc->d, &dc->c))) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(o, "o")) || (st = check_ptr(lse, "lse", false)))
    return st;
  if (num_splits < 0 || num_splits > 512)
    return fail(HS_ERR_SHAPE, "num_splits must be in 0..512 (got %d)", num_splits);
  dc->splits = num_splits ? num_splits : auto_splits(dc->d);
  dc->need = decode_ws_bytes(dc->d, dc->splits);
  return HS_OK;
}
static hs_status run_decode(const DecodeCall &dc, const uint16_t *q, uint16_t *o, float *lse,
                            float softmax_scale, void *ws, void *stream) {
  float *part_o = (float *)ws;
  float *part_lse = part_o + (size_t)dc.d.b * dc.d.hq * dc.splits * dc.d.D;
  hipError_t e = hs::launch_decode(dc.d, dc.c, q, o, lse, scale_log2(softmax_scale, dc.d.D),
                                   dc.splits, part_o, part_lse, (hipStream_t)stream);
  if (e != hipSuccess) return fail(HS_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

HS_API hs_status hs_decode_attn(const hs_shape *shape, const hs_counts *counts,
                                const hs_cache *cache, const uint16_t *q, uint16_t *o, float *lse,
                                float softmax_scale, int32_t num_splits, void *ws,
                                size_t ws_bytes, void *stream) {
  DecodeCall dc;
  hs_status st = check_decode(shape, counts, cache, q, o, lse, num_splits, &dc);
  if (st) return st;
  if (!ws || ws_bytes < dc.need)
    return fail(HS_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", dc.need, ws_bytes,
                ws ? "" : ", NULL");
  if (!aligned16(ws)) return fail(HS_ERR_ALIGN, "workspace is not 16-byte aligned");
  return run_decode(dc, q, o, lse, softmax_scale, ws, stream);
}

// ---- allocation-free decode -------------------------------------------------------------------
// The decode's workspace (the splits' partials) in a file-scope device array. Each GPU holds its
// own copy until the process ends. In host code 'scratch' names a host-side stand-in: its device
// address, per device, comes from hipGetSymbolAddress on the first call on that device and is
// the only form in which the array reaches a kernel.
static __device__ __align__(256) unsigned char scratch[HS_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of 'scratch' on the current device (resolved once per device). Nothing in the
// array needs to start at any value: every call writes the partials it reads.
hs_status scratch_on_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(HS_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(HS_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(HS_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HS_OK;
}
}  // namespace

HS_API hs_status hs_decode_attn_noalloc(const hs_shape *shape, const hs_counts *counts,
                                        const hs_cache *cache, const uint16_t *q, uint16_t *o,
                                        float *lse, float softmax_scale, int32_t num_splits,
                                        void *stream) {
  DecodeCall dc;
  hs_status st = check_decode(shape, counts, cache, q, o, lse, num_splits, &dc);
  if (st) return st;
  if (dc.need > HS_DECODE_NOALLOC_SCRATCH_BYTES)
    return fail(HS_ERR_WORKSPACE,
                "decode needs %zu bytes of scratch, more than the %zu bytes the library holds; "
                "use hs_decode_attn with a workspace (or fewer splits)",
                dc.need, (size_t)HS_DECODE_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  if ((st = scratch_on_device(&ws))) return st;
  return run_decode(dc, q, o, lse, softmax_scale, ws, stream);
}

HS_API hs_status hs_prefill_attn(const hs_shape *shape, const hs_counts *counts,
                                 const hs_cache *cache, const uint16_t *q, uint16_t *o, float *lse,
                                 float softmax_scale, uint32_t flags, void *stream) {
  hs::Dims d;
  hs::CacheView c;
  hs_status st = make_dims(shape, counts, &d);
  if (st) return st;
  if ((st = check_cache(cache, d, &c))) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(o, "o")) || (st = check_ptr(lse, "lse", false)))
    return st;
  if (flags != HS_PREFILL_SMFMAC && flags != HS_PREFILL_DECOMPRESS)
    return fail(HS_ERR_UNSUPPORTED, "unknown prefill flags 0x%x", flags);
  hipError_t e = hs::launch_prefill(d, c, q, o, lse, scale_log2(softmax_scale, d.D),
                                    flags == HS_PREFILL_SMFMAC, (hipStream_t)stream);
  if (e != hipSuccess) return fail(HS_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return ok();
}

HS_API hs_status hs_prefill_attn_variant(const hs_shape *shape, const hs_counts *counts,
                                         const hs_cache *cache, const uint16_t *q, uint16_t *o,
                                         float *lse, float softmax_scale, uint32_t variant,
                                         void *stream) {
  hs::Dims d;
  hs::CacheView c;
  hs_status st = make_dims(shape, counts, &d);
  if (st) return st;
  if ((st = check_cache(cache, d, &c))) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(o, "o")) || (st = check_ptr(lse, "lse", false)))
    return st;
  if (variant != HS_PREFILL_VARIANT_NONE && variant != HS_PREFILL_VARIANT_SYNC_LOADS &&
      variant != HS_PREFILL_VARIANT_NO_ALIAS && variant != HS_PREFILL_VARIANT_GENERIC_WALK &&
      variant != HS_PREFILL_VARIANT_LOCKSTEP && variant != HS_PREFILL_VARIANT_LDS_RELAYOUT)
    return fail(HS_ERR_UNSUPPORTED, "unknown prefill variant %u", variant);
  if (d.dtype != hs::kBf16 || d.nb > (variant == HS_PREFILL_VARIANT_LDS_RELAYOUT ? 1024 : 2048))
    return fail(HS_ERR_UNSUPPORTED,
                "prefill variants take bf16 heads of at most 2048 blocks (1024 for variant 16)");
  static_assert(HS_PREFILL_VARIANT_SYNC_LOADS == hs::kPrefillVariantSyncLoads &&
                    HS_PREFILL_VARIANT_NO_ALIAS == hs::kPrefillVariantNoAlias &&
                    HS_PREFILL_VARIANT_GENERIC_WALK == hs::kPrefillVariantGenericWalk &&
                    HS_PREFILL_VARIANT_LOCKSTEP == hs::kPrefillVariantLockstep &&
                    HS_PREFILL_VARIANT_LDS_RELAYOUT == hs::kPrefillVariantLdsRelayout,
                "variant codes");
  hipError_t e = hs::launch_prefill_variant(d, c, q, o, lse, scale_log2(softmax_scale, d.D),
                                            (int)variant, (hipStream_t)stream);
  if (e != hipSuccess) return fail(HS_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return ok();
}

HS_API const char *hs_status_string(hs_status s) {
  switch (s) {
    case HS_OK: return "ok";
    case HS_ERR_NULL: return "null pointer";
    case HS_ERR_SHAPE: return "unsupported or inconsistent shape";
    case HS_ERR_COUNTS: return "invalid block counts";
    case HS_ERR_ALIGN: return "pointer not 16-byte aligned";
    case HS_ERR_WORKSPACE: return "workspace missing or too small";
    case HS_ERR_UNSUPPORTED: return "unsupported request";
    case HS_ERR_HIP: return "HIP launch error";
    case HS_ERR_OVERLAP: return "overlapping buffers";
  }
  return "unknown status";
}

HS_API const char *hs_last_error(void) { return g_error; }
