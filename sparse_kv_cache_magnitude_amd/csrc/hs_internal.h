// hs_internal.h -- host-side launch interface between the C ABI (hs_api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs {

constexpr int kMaxBlocks = 4096;  // blocks per head handled by the in-LDS ranking
constexpr int kBf16 = 0, kF16 = 1;  // element types (hs_shape.dtype)

// Validated problem description (see hs_api.hip).
struct Dims {
  int b, hq, hkv, G;  // batch, query heads, KV heads, query heads per KV head
  int L, D, B, nb;    // tokens, head_dim, block size, blocks per head
  int np, nsk, nsv;   // per-head pruned / K 2:4 / V 2:4 block counts
  int ndk, ndv;       // per-head dense block counts
  int dtype;          // kBf16 or kF16
};

struct CacheView {
  int32_t *map_k, *map_v;
  uint16_t *k_dense, *k_nnz, *k_meta;
  uint16_t *v_dense, *v_nnz, *v_meta;
};

// Blocks i < dense_lo or i >= dense_hi (dense_hi < 0: nb) stay dense and are not ranked.
hipError_t launch_compress(const Dims &d, const uint16_t *k, const uint16_t *v, const CacheView &c,
                           uint64_t *keys, hipStream_t stream, int dense_lo = 0,
                           int dense_hi = -1);

// The pack step alone: pools written from K, V as c.map_k / c.map_v (already on the device) say.
hipError_t launch_pack(const Dims &d, const uint16_t *k, const uint16_t *v, const CacheView &c,
                       hipStream_t stream);

// Caller-given block modes (uint8 [b][hkv][nb], 0 pruned / 1 dense / 2 2:4) -> index maps, with
// per-head validation (hs_masked.hip). head_status may be null.
hipError_t launch_modes(const Dims &d, const uint8_t *mode_k, const uint8_t *mode_v,
                        const CacheView &c, int32_t *head_status, hipStream_t stream);

// part_o [b][hq][splits][D] and part_lse [b][hq][splits] fp32: the splits' partials (unused with
// one split).
hipError_t launch_decode(const Dims &d, const CacheView &c, const uint16_t *q, uint16_t *o,
                         float *lse, float scale_log2, int splits, float *part_o, float *part_lse,
                         hipStream_t stream);

hipError_t launch_prefill(const Dims &d, const CacheView &c, const uint16_t *q, uint16_t *o,
                          float *lse, float scale_log2, bool smfmac, hipStream_t stream);

// Ablation variants of the SMFMAC prefill (hs_prefill_attn_variant): bf16, heads of at most 2048
// blocks (1024 for the LDS re-layout); hipErrorInvalidValue otherwise.
constexpr int kPrefillVariantSyncLoads = 1, kPrefillVariantNoAlias = 2,
              kPrefillVariantGenericWalk = 4, kPrefillVariantLockstep = 8,
              kPrefillVariantLdsRelayout = 16;
hipError_t launch_prefill_variant(const Dims &d, const CacheView &c, const uint16_t *q,
                                  uint16_t *o, float *lse, float scale_log2, int variant,
                                  hipStream_t stream);

// Dense stand-ins of a compressed cache: K, V [b][hkv][L][D] with kept values in place and zeros
// elsewhere (hs_recompress.hip).
hipError_t launch_unpack(const Dims &d, const CacheView &c, uint16_t *k_out, uint16_t *v_out,
                         hipStream_t stream);

}  // namespace hs
