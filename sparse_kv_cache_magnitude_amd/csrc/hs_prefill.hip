// hs_prefill.hip -- causal tiled prefill attention over the compressed cache (gfx950).
//
// "HieraSparse" (arXiv 2604.16864v2) §III-C1 Algorithm 1 (S^T = K Q^T, online softmax, P^T
// re-layout, O^T += V^T P^T), §III-C2 mixed dense / sparse dispatch through the index map,
// §IV-C1 asynchronous K/V staging, §IV-C2 in-fragment re-layout, §IV-C3 dense and sparse buffers
// aliased in on-chip memory. Made causal; pruned blocks are skipped without any load.
//
// Work decomposition: each wave owns one (query head, 32-query tile) task; a workgroup's tasks
// share one KV head (for GQA group size 4: the four query heads of that KV head at adjacent
// 32-query tiles), so every K/V tile it stages serves 32 queries per wave. Query tiles are issued
// longest-first and the workgroups of one KV head run on one XCD.
//   SMFMAC path (heads of at most 2048 blocks): workgroups of 4 waves (one per SIMD), two
//   workgroups per CU. The two waves on a SIMD then belong to different workgroups whose
//   per-tile barriers are independent, so one wave's staging, barrier and dependency waits
//   overlap the other's matrix and vector work; measured faster than 8-wave workgroups whose two
//   waves per SIMD walk in lockstep.
//   Decompress path (and SMFMAC for longer heads): workgroups of 8 waves (two per SIMD), one per
//   CU.
//
// Per visible 64-token KV tile (matrix-core shapes 32x32: v_mfma_f32_32x32x16_bf16 and
// v_smfmac_f32_32x32x32_bf16; all accumulators in VGPRs):
//   staging   LDS stages filled by direct global->LDS loads (global_load_lds_dwordx4) one tile
//             ahead; one wait for the wave's loads and one barrier per tile. A stage holds the
//             tile's K and V^T in their stored representation (dense copy, or kept values +
//             metadata), rows unit-swizzled so that the operand reads are free of bank conflicts
//             (layout below). The walk reads its tiles from a list of the workgroup's visible
//             blocks built at start, so pruned blocks cost nothing.
//   GEMM1     S^T[64 tok][32 q] = K Q^T (Q stays in registers as the B operand).
//   softmax   causal mask, column-wise running max (exp2 domain, lazy rescale) and
//             P^T = exp2(S^T - max) packed to bf16 in registers.
//   GEMM2     O^T[128 ch][32 q] += V^T P^T: in the same step (4-wave workgroups, two stages), or
//             one tile late beside the exponentials of the next tile (8-wave workgroups, three
//             stages).
// When every visible block of a workgroup has both operands 2:4 (or both dense), the walk runs a
// copy of the tile body compiled for that kind, with no per-tile branches on the operand kinds
// (the specialised fully-2:4 and fully-dense kernels of §IV-C3).
// Token order: GEMM1's A operand rows are the tile's tokens in an order tau chosen so that the
// 32x32 accumulator lands exactly in GEMM2's B operand layout (lane half h holds 16 consecutive
// registers per 32-token half); P^T needs no data movement between lanes. The stage stores the K
// rows already in that order.
// SMFMAC path: 2:4 operands go to v_smfmac; dense V^T is fed to the same instruction as two 2:4
// halves (so the output accumulators see one instruction type). Decompress path: after a tile has
// landed, the whole workgroup expands its 2:4 operands once into a dense scratch tile in LDS (the
// dense stage layout; one more barrier), and GEMM1, the softmax and GEMM2 of that tile then run on
// dense MFMA in the same step.
#include "hs_device.h"
#include "hs_internal.h"

#include <type_traits>

namespace hs {
namespace {

constexpr int kD = 128;
constexpr int kTile = 64;   // KV tokens per tile
constexpr int kQTile = 32;  // queries per wave
constexpr int kWaves = 8;  // decompress path (and the SMFMAC path for heads of > 2048 blocks)

// ---- LDS stage layout (bytes). A stage holds one tile in two 16 KB regions:
//   K region   dense: 64 rows x 256 B; 2:4: 64 rows x 128 B of kept values and the 2:4 K
//              metadata (64 x 16 B) at kMetaOff
//   V^T region dense: 128 rows x 128 B; 2:4: 128 rows x 64 B of kept values in 32-row groups
//              4 KB apart (as for dense, so both kinds address a 32-channel tile alike), and the
//              2:4 V metadata (128 x 8 B) in the free half of the first group, at kVMetaOff
// Rows are not padded: the 16-byte units of row r are stored at unit u ^ f(r), with f chosen so
// that 16 consecutive rows read at one logical unit hit 16 distinct bank groups (f = r & 15 for
// 16-unit rows, (r >> 1) & 7 for 8-unit rows, (r >> 2) & 3 for 4-unit rows). Every region is a
// whole number of 1 KB direct loads per wave: dense 2, 2:4 values 1.
constexpr int kRegion = 16384;
constexpr int kStageBytes = 2 * kRegion;  // 32 KB
constexpr int kMetaOff = 8192;            // K region: 2:4 K metadata
constexpr int kCtStride = 4096;           // V^T region: bytes between 32-channel tiles
constexpr int kVMetaOff = kRegion + 2048;  // stage: 2:4 V metadata
// LDS of a workgroup of W waves, stages first (each 32 KB, 1 KB aligned):
//   stages     kStagesN tiles (SMFMAC path with W = 8: three, GEMM2 of a tile runs one tile late;
//              W = 4: two; decompress path: three)
//   kDenseIdx  SMFMAC path: 1 KB of the index word a dense V^T tile's first SMFMAC uses (0x4444,
//              positions 0 and 1 of every group), laid out like a stage's V^T metadata, so dense
//              and 2:4 tiles read their index words the same way
//   kZero      SMFMAC path: 128 zero bytes. An SMFMAC accumulates in place, so the S^T
//              accumulators of a 2:4 K tile start from zeros read here (LDS broadcast reads)
//              rather than from 16 VALU moves per half
//   kCount     per-wave counts used while building the block list; kKind per-wave operand kinds
//              (bit 0: a visible block has a dense operand, bit 1: a 2:4 one)
//   kListModes the workgroup's visible blocks in order: their modes as local pool slots (int32: K
//              slot code in the high half, V slot code in the low half; +(i+1) dense slot i,
//              -(i+1) 2:4 slot i); kListBlk their block indices (int16); kMaxB entries each
//   kScratch   decompress path: the dense image of the current tile's 2:4 operands (the stage
//              layout, K at 0, V^T at kRegion), expanded once per tile by the whole workgroup
// Ablation variants of the SMFMAC path (measurement only; the library's entry points run A = 0):
constexpr int kAblSyncLoads = 1;    // a tile's loads are issued and waited for in its own step
constexpr int kAblNoAlias = 2;      // a stage holds separate dense and 2:4 buffers (64 KB)
constexpr int kAblGenericWalk = 4;  // no walk specialised on the operand kinds
constexpr int kAblLdsRelayout = 16;  // K rows in token order, P^T re-laid out through LDS
static_assert(kAblSyncLoads == kPrefillVariantSyncLoads && kAblNoAlias == kPrefillVariantNoAlias &&
                  kAblGenericWalk == kPrefillVariantGenericWalk &&
                  kAblLdsRelayout == kPrefillVariantLdsRelayout,
              "variant codes");
template <int W, bool kSmfmac, int A = 0>
struct Lay {
  static constexpr int kStagesN = (kSmfmac && W == 4) ? 2 : 3;
  // (the LDS re-layout variant lists 1024 blocks, to keep its P^T buffers within 80 KB)
  static constexpr int kMaxB = W == 4 ? ((A & kAblLdsRelayout) ? 1024 : 2048) : kMaxBlocks;
  // Without aliasing, the 2:4 representation of a tile sits kSparse bytes above its dense one.
  static constexpr int kSparse = (A & kAblNoAlias) ? kStageBytes : 0;
  static constexpr int kStride = kStageBytes + kSparse;  // bytes between stages
  static constexpr int kDenseIdx = kStagesN * kStride;
  static constexpr int kZero = kDenseIdx + 1024;
  static constexpr int kCount = kZero + 128;
  static constexpr int kKind = kCount + 4 * W;
  static constexpr int kListModes = (kKind + 4 * W + 15) / 16 * 16;
  static constexpr int kListBlk = kListModes + 4 * kMaxB;
  static constexpr int kPBuf = kListBlk + 2 * kMaxB;  // 2 KB per wave (LDS re-layout variant)
  static constexpr int kEnd = kPBuf + ((A & kAblLdsRelayout) ? 2048 * W : 0);
  static constexpr int kScratch = (kEnd + 1023) / 1024 * 1024;
  static constexpr int kBytes = kSmfmac ? kEnd : kScratch + kStageBytes;
  static_assert(kBytes <= ((W == 4 && !(A & kAblNoAlias)) ? 80 : 160) * 1024, "LDS budget");
};
static_assert(kRegion % 1024 == 0 && kMetaOff % 1024 == 0, "whole 1 KB loads per region");

constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)
constexpr float kLazyBound = 256.0f;  // 2^kTau: no probability above it while the max holds


__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }
__device__ __forceinline__ int swap13(int x) { return (x & ~10) | ((x & 2) << 2) | ((x & 8) >> 2); }
// Token held by GEMM1 row r (0..31) of a 32-token half: bits 2,3 of r exchanged when the tile's V
// is consumed in natural order (dense MFMA k-steps, or stored 2:4 groups), bits 1,3 exchanged when
// a dense V tile is split into two 2:4 halves for SMFMAC (see gemm2_smfmac_step).
__device__ __forceinline__ int tau(int r, bool split) { return split ? swap13(r) : swap23(r); }

// ---- matrix-core helpers -----------------------------------------------------------------------
template <class E>
__device__ __forceinline__ f32x16 mfma32(vec8<E> a, vec8<E> b, f32x16 c) {
  return mma32x16(a, b, c);
}
template <class E, int kSet = 0>
__device__ __forceinline__ f32x16 smfmac32(vec8<E> a, vec16<E> b, uint32_t idx, f32x16 c) {
  return smma32x32<kSet>(a, b, c, (int)idx);
}
// Half k of a 32-deep B operand pair: the B operand of one 16-deep dense step.
template <class E>
__device__ __forceinline__ vec8<E> half8(vec16<E> v, int k2) {
  return k2 ? __builtin_shufflevector(v, v, 8, 9, 10, 11, 12, 13, 14, 15)
            : __builtin_shufflevector(v, v, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// LDS reads. A read address is a stage pointer (a multiple of 32 KB from the 1 KB-aligned LDS
// array) plus a lane offset with its k-step unit XORed in, plus a constant row-group offset; as the
// stage pointer has no bits below bit 15, adding it commutes with the XOR.
__device__ __forceinline__ uint4 lds16(const char *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ uint2 lds8(const char *p) { return *reinterpret_cast<const uint2 *>(p); }

// Two packed 2:4 groups (4 kept values as two dwords, 8 metadata bits) -> 8 dense values.
template <class E>
__device__ __forceinline__ vec8<E> expand2(uint2 v, uint32_t bits) {
  const uint2 g0 = expand_group(v.x, bits & 15u), g1 = expand_group(v.y, (bits >> 4) & 15u);
  return as8<E>(make_uint4(g0.x, g0.y, g1.x, g1.y));
}

// Combine a per-lane value of the two wave halves (lanes l and l ^ 32) with max / sum.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct PrefillArgs {
  CacheView c;
  const uint16_t *q;
  uint16_t *o;
  float *lse;
  int L, nb, hkv, hq, G, nqt, wg_per_head, n_wg;
  int ndk, nsk, ndv, nsv;
  float scale_log2;
};

// Per-wave state of the online softmax and the output accumulators (one 32-query tile).
template <class E>
struct WaveState {
  vec16<E> qv[4];  // Q^T as GEMM1 B operand: qv[s] holds channel chunks s and s + 4 (16 channels
                   // each), i.e. the dense k-steps over chunks s and s + 4 back to back
  f32x16 o[4];    // O^T, per 32-channel tile
  f32x16 s[2];    // S^T of the current tile, per 32-token half
  vec16<E> p[2];  // P^T per 32 tokens (two 16-token dense k-steps): previous tile until
                  // overwritten by the current one
  float m_run, l_run, m_use, alpha;
};

// Per-lane LDS byte offsets of the operand reads, relative to a stage, with the lane's part of
// the unit swizzle folded in; a read XORs in the (compile-time) unit of its k-step and adds the
// row-group offset.
struct LaneOffsets {
  int kd, kn, km;       // dense K; 2:4 K values; 2:4 K metadata (16 B each)
  int vd, vdd, vn, vm;  // dense V^T split (SMFMAC) and dense (decompress); 2:4 V^T; metadata
  uint32_t vsel;        // byte selector: the lane half's 16-bit index words of both k-steps
};

// ---- GEMM1: S^T = K Q^T for one staged tile ---------------------------------------------------
// Lane (r, hf) reads row slot 32T + r; the stage holds the K rows in GEMM1 row order. The dense
// k-step over 16-channel chunk cc takes the Q registers half8(qv[cc & 3], cc >> 2). The 2:4 step s
// covers chunks s and s + 4: lane half hf holds the kept values of chunk s + 4hf, whose 16-bit
// metadata word is half s & 1 of dword (s >> 1) + 2hf of the row's metadata. Each lane reads the
// 8 metadata bytes of its half of the row once, and every SMFMAC selects its index set by the
// instruction's key, so no per-lane shift or select of the metadata is needed.
template <bool kSparseK, class E>
__device__ __forceinline__ void gemm1(WaveState<E> &w, const char *st, const LaneOffsets &lo, int hf,
                                      const char *zp) {
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    f32x16 acc = kSparseK ? *reinterpret_cast<const f32x16 *>(zp + 64 * T) : zero16();
    if (!kSparseK) {
      uint4 k[8];  // all reads issued before the first MFMA that needs them
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) k[cc] = lds16(st + (lo.kd ^ (32 * cc)) + T * 8192);
#pragma unroll
      for (int cc = 0; cc < 8; ++cc)
        acc = mfma32(as8<E>(k[cc]), half8<E>(w.qv[cc & 3], cc >> 2), acc);
    } else {
      const uint2 meta = lds8(st + lo.km + T * 512);
      uint4 k[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) k[s] = lds16(st + (lo.kn ^ (16 * s)) + T * 4096);
      acc = smfmac32<E, 0>(as8<E>(k[0]), w.qv[0], meta.x, acc);
      acc = smfmac32<E, 1>(as8<E>(k[1]), w.qv[1], meta.x, acc);
      acc = smfmac32<E, 0>(as8<E>(k[2]), w.qv[2], meta.y, acc);
      acc = smfmac32<E, 1>(as8<E>(k[3]), w.qv[3], meta.y, acc);
    }
    w.s[T] = acc;
  }
}

// ---- GEMM2 on the SMFMAC path, one 32-token k-step u ------------------------------------------
// Dense and 2:4 V^T tiles share one instruction type, so O^T stays in one register set: per
// 32-channel tile, one SMFMAC on the kept values (2:4: stored values and metadata; dense: the
// lane's tokens 0..7 at group positions {0,1}, index 0x4444), and for a dense tile a second one on
// tokens 8..15 at positions {2,3} (index 0xEEEE). For a dense tile P^T arrives in the matching
// token order (tau with bits 1 and 3 exchanged). All operand reads of the k-step are issued before
// its first SMFMAC, so their LDS latency is paid once. The tile-kind test stays next to each second
// SMFMAC: one branch around the whole sequence makes the compiler copy the accumulators at the join.
template <class E>
__device__ __forceinline__ void gemm2_smfmac_step(WaveState<E> &w, const char *st, bool sparse,
                                                  const uint32_t *meta, int u, const LaneOffsets &lo,
                                                  int hf) {
  const int off = sparse ? (lo.vn ^ (32 * u)) : (lo.vd ^ (64 * u));
  uint4 v0[4], v1[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) v0[ct] = lds16(st + off + ct * kCtStride);
  if (!sparse) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) v1[ct] = lds16(st + (off ^ 16) + ct * kCtStride);
  }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    w.o[ct] = u ? smfmac32<E, 1>(as8<E>(v0[ct]), w.p[u], meta[ct], w.o[ct])
                : smfmac32<E, 0>(as8<E>(v0[ct]), w.p[u], meta[ct], w.o[ct]);
    if (!sparse) w.o[ct] = smfmac32(as8<E>(v1[ct]), w.p[u], 0xEEEEu, w.o[ct]);
  }
}
// Index words of GEMM2: a 2:4 tile's metadata, or the dense index words (table at didx). A
// 32-channel tile's 8 bytes hold the 16-bit words of k-step 0 (both lane halves) and then those of
// k-step 1; one byte permute per tile gathers the lane half's two words into one register, low
// half k-step 0 and high half k-step 1, and each SMFMAC picks its half by the instruction's key.
__device__ __forceinline__ void load_vmeta(uint32_t *meta, const char *st, bool sparse,
                                           const LaneOffsets &lo, const char *didx) {
  const char *base = sparse ? st : didx - kVMetaOff;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const uint2 m = lds8(base + lo.vm + ct * 32 * 8);
    meta[ct] = __builtin_amdgcn_perm(m.y, m.x, lo.vsel);
  }
}

// ---- GEMM2 on the decompress path (dense operands), one 16-token k-step ks --------------------
template <class E>
__device__ __forceinline__ void gemm2_dense_step(WaveState<E> &w, const char *st, int ks,
                                                 const LaneOffsets &lo) {
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const vec8<E> v = as8<E>(lds16(st + (lo.vdd ^ (32 * ks)) + ct * kCtStride));
    w.o[ct] = mfma32(v, half8<E>(w.p[ks >> 1], ks & 1), w.o[ct]);
  }
}

// ---- softmax of the current tile: causal mask, running max, decision to rescale ----------------
// 'shift' = (first token of the key tile) - (first query of the wave); a token is masked when
// shift + token > query. kNatural: the K rows are staged in token order (no tau).
template <bool kNatural = false, class E>
__device__ __forceinline__ void softmax_mask(WaveState<E> &w, bool split, int shift, int r, int hf) {
#pragma unroll
  for (int T = 0; T < 2; ++T)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = 8 * (e >> 2) + 4 * hf + (e & 3);
      if (shift + 32 * T + (kNatural ? row : tau(row, split)) > r) w.s[T][e] = -INFINITY;
    }
}

// The tile's row maxima against the running max: returns true if the running max moves (by more
// than kTau; then w.alpha rescales O and l and w.m_use is the new max), else w.m_use = the running
// max.
template <class E>
__device__ __forceinline__ bool softmax_rescale(WaveState<E> &w, float c) {
  float mx = -INFINITY;
#pragma unroll
  for (int T = 0; T < 2; ++T)
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, w.s[T][e]);
  const float mt = max_halves(mx) * c;
  const float m_new = fmaxf(w.m_run, mt);
  const bool need = __builtin_amdgcn_ballot_w64(m_new > w.m_run + kTau) != 0;
  if (need) {
    w.alpha = w.m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(w.m_run - m_new);
    w.m_use = m_new;
  } else {
    w.alpha = 1.f;
    w.m_use = w.m_run;
  }
  return need;
}

template <bool kNatural = false, class E>
__device__ __forceinline__ bool softmax_max(WaveState<E> &w, bool diag, bool split, int shift, int r,
                                            int hf, float c) {
  if (diag) softmax_mask<kNatural>(w, split, shift, r, hf);
  return softmax_rescale(w, c);
}

// P^T of the current tile for GEMM2 k-step ks (16 tokens): the accumulator registers
// 8*(ks&1) .. +7 of half ks>>1, exponentiated and packed to bf16. The fp32 values are also summed
// into the running denominator with plain adds: the packed-pair dot product (v_dot2) would do it in
// half the instructions, but on gfx950 it waits for the matrix core to drain, so every one of them
// stalls the other wave's MFMAs on the same SIMD.
template <class E>
__device__ __forceinline__ void softmax_exp(WaveState<E> &w, int ks, float c, float mc, float &lsum) {
  const f32x16 &s = w.s[ks >> 1];
  const int base = 8 * (ks & 1);
  uint32_t pk[4];
  float p[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    p[2 * e] = __builtin_amdgcn_exp2f(fmaf(s[base + 2 * e], c, -mc));
    p[2 * e + 1] = __builtin_amdgcn_exp2f(fmaf(s[base + 2 * e + 1], c, -mc));
    pk[e] = pack2<E>(p[2 * e], p[2 * e + 1]);
  }
  lsum += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  const vec8<E> nw = as8<E>(make_uint4(pk[0], pk[1], pk[2], pk[3]));
  vec16<E> &pp = w.p[ks >> 1];
  pp = (ks & 1) ? __builtin_shufflevector(half8<E>(pp, 0), nw, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11,
                                          12, 13, 14, 15)
                : __builtin_shufflevector(nw, half8<E>(pp, 1), 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11,
                                          12, 13, 14, 15);
}

template <class E>
__device__ __forceinline__ void softmax_finish(WaveState<E> &w, bool need, float lsum) {
  if (need) {
    w.l_run = w.l_run * w.alpha + lsum;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) w.o[ct] *= w.alpha;
    w.m_run = w.m_use;
  } else {
    w.l_run += lsum;
  }
}

// Exponentials of the current tile interleaved with GEMM2 of the previous tile (if 'gemm'): the
// instructions that read P^T of the previous tile are issued first, then the same registers
// receive P^T of the current tile, 32 tokens at a time.
template <class E>
__device__ __forceinline__ float exp_and_gemm2(WaveState<E> &w, const char *st_prev, bool gemm,
                                               bool sparse, const LaneOffsets &lo, int hf,
                                               float c, const char *didx) {
  float lsum = 0.f;
  const float mc = w.m_use == -INFINITY ? 0.f : w.m_use;  // rows with nothing visible yet
  uint32_t meta[4];
  load_vmeta(meta, st_prev, gemm && sparse, lo, didx);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (gemm) gemm2_smfmac_step(w, st_prev, sparse, meta, u, lo, hf);
    softmax_exp(w, 2 * u, c, mc, lsum);
    softmax_exp(w, 2 * u + 1, c, mc, lsum);
  }
  return lsum;
}

// GEMM2 of one staged tile in two parts: the operand reads of k-step u (and, for u = 0, the
// index words of both), and the SMFMACs of k-step u on them, so that the reads can be issued well
// ahead of the SMFMACs.
struct VOps {
  uint32_t meta[4];
  uint4 v0[4], v1[4];
};
__device__ __forceinline__ void gemm2_read(VOps &v, const char *st, bool sparse, int u,
                                           const LaneOffsets &lo, const char *didx) {
  if (u == 0) load_vmeta(v.meta, st, sparse, lo, didx);
  const int off = sparse ? (lo.vn ^ (32 * u)) : (lo.vd ^ (64 * u));
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) v.v0[ct] = lds16(st + off + ct * kCtStride);
  if (!sparse) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) v.v1[ct] = lds16(st + (off ^ 16) + ct * kCtStride);
  }
}
template <class E>
__device__ __forceinline__ void gemm2_apply(WaveState<E> &w, const VOps &v, bool sparse, int u,
                                            int hf) {
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    w.o[ct] = u ? smfmac32<E, 1>(as8<E>(v.v0[ct]), w.p[u], v.meta[ct], w.o[ct])
                : smfmac32<E, 0>(as8<E>(v.v0[ct]), w.p[u], v.meta[ct], w.o[ct]);
    if (!sparse) w.o[ct] = smfmac32(as8<E>(v.v1[ct]), w.p[u], 0xEEEEu, w.o[ct]);
  }
}

// Measurement variant without the token order tau: the K rows are staged in token order, so the
// accumulator register pair jp of lane half hf (per 32-token half) holds tokens
// nat = 8 (jp >> 1) + 4 hf + 2 (jp & 1), while GEMM2's B operand wants tau(nat) there. P^T is
// moved through this wave's 2 KB of LDS: row q (the lane's query) of 32 tokens, its 16-byte unit
// x stored at x ^ ((q >> 2) & 3); pairs written at their own token, read at tau's.
template <class E>
__device__ __forceinline__ void relayout_through_lds(WaveState<E> &w, int u, char *scr, bool split,
                                                     int q, int hf) {
  auto at = [&](int t) { return scr + 64 * q + 16 * ((t >> 3) ^ ((q >> 2) & 3)) + 2 * (t & 7); };
  {
    const uint4 a = __builtin_bit_cast(uint4, half8<E>(w.p[u], 0)),
                b = __builtin_bit_cast(uint4, half8<E>(w.p[u], 1));
    const uint32_t pr[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int g = 0; g < 4; ++g)  // pairs 2g, 2g + 1: tokens 8 g + 4 hf .. + 3
      *reinterpret_cast<uint2 *>(at(8 * g + 4 * hf)) = make_uint2(pr[2 * g], pr[2 * g + 1]);
    uint4 ra, rb;
    if (!split) {  // tau = swap23: pairs 0..3 are tokens 8 hf .. + 7, pairs 4..7 16 more
      ra = lds16(at(8 * hf));
      rb = lds16(at(16 + 8 * hf));
    } else {
      uint32_t rd[8];
#pragma unroll
      for (int jp = 0; jp < 8; ++jp)
        rd[jp] = *reinterpret_cast<const uint32_t *>(at(swap13(8 * (jp >> 1) + 4 * hf + 2 * (jp & 1))));
      ra = make_uint4(rd[0], rd[1], rd[2], rd[3]);
      rb = make_uint4(rd[4], rd[5], rd[6], rd[7]);
    }
    w.p[u] = __builtin_shufflevector(as8<E>(ra), as8<E>(rb), 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11,
                                     12, 13, 14, 15);
  }
}

// GEMM2 of one staged tile alone.
template <class E>
__device__ __forceinline__ void gemm2_smfmac(WaveState<E> &w, const char *st, bool sparse,
                                             const LaneOffsets &lo, int hf, const char *didx) {
  uint32_t meta[4];
  load_vmeta(meta, st, sparse, lo, didx);
#pragma unroll
  for (int u = 0; u < 2; ++u) gemm2_smfmac_step(w, st, sparse, meta, u, lo, hf);
}

// ---- decompress path: 2:4 operands of a stage expanded into the dense stage layout -------------
// Dense K row slot r holds at 16-byte unit j the channels 8c .. 8c + 7, c = j ^ (r & 15); the 2:4
// K row keeps their eight values (groups 2c, 2c + 1) in half c & 1 of its unit c >> 1, found at
// unit (c >> 1) ^ ((r >> 1) & 7), and their metadata in byte c of the row's 16 metadata bytes.
// Dense V^T channel row ch holds at unit j the tokens 8t .. 8t + 7, t = j ^ ((ch >> 1) & 7); the
// 2:4 V^T row (32-row group ch / 32, row ch % 32) keeps them in half t & 1 of unit t >> 1, found
// at unit (t >> 1) ^ ((ch >> 2) & 3), with metadata byte t of the channel's 8 bytes. Each of the
// workgroup's 512 lanes expands two K units and two V units.
template <class E>
__device__ __forceinline__ void expand_tile(const char *st, char *dst, bool sparse_k, bool sparse_v,
                                            int tid) {
  if (sparse_k) {
#pragma unroll
    for (int i = tid; i < 64 * 16; i += kWaves * 64) {
      const int r = i >> 4, j = i & 15, c = j ^ (r & 15);
      const uint2 kv = lds8(st + r * 128 + 16 * ((c >> 1) ^ ((r >> 1) & 7)) + 8 * (c & 1));
      const uint32_t bits = *reinterpret_cast<const uint8_t *>(st + kMetaOff + r * 16 + c);
      *reinterpret_cast<vec8<E> *>(dst + r * 256 + 16 * j) = expand2<E>(kv, bits);
    }
  }
  if (sparse_v) {
#pragma unroll
    for (int i = tid; i < 128 * 8; i += kWaves * 64) {
      const int ch = i >> 3, j = i & 7, t = j ^ ((ch >> 1) & 7);
      const int row = kRegion + (ch >> 5) * kCtStride + (ch & 31) * 64;
      const uint2 vv = lds8(st + row + 16 * ((t >> 1) ^ ((ch >> 2) & 3)) + 8 * (t & 1));
      const uint32_t bits = *reinterpret_cast<const uint8_t *>(st + kVMetaOff + ch * 8 + t);
      *reinterpret_cast<vec8<E> *>(dst + kRegion + ch * 128 + 16 * j) = expand2<E>(vv, bits);
    }
  }
}

// ---- staging of one tile -----------------------------------------------------------------------
// Each region is a whole number of 1 KB loads (64 lanes x 16 B); load q of a region goes to wave
// q % 8, so a wave issues two loads for a dense region and one for 2:4 values. Metadata: K (1 KB)
// by wave 1; V: one 1 KB load by wave 2 (block 64), or four 256 B dword loads by waves 3-6
// (block 128, where a tile is half of each channel's metadata row).

template <int B, int W, bool kSmfmac, class E, int A = 0>
__global__ __launch_bounds__(64 * W, W == 4 ? 2 : 1) void k_prefill(PrefillArgs a) {
  using L = Lay<W, kSmfmac, A>;
  constexpr int SP = L::kSparse;  // offset of a stage's 2:4 buffers from its dense ones
  static_assert(kSmfmac || W == kWaves, "the decompress path runs eight waves");
  __shared__ __attribute__((aligned(1024))) char lds[L::kBytes];
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int TPB = B / kTile;  // 64-token tiles per block
  constexpr int kVmWave0 = W == 8 ? 3 : 0;  // block 128: first of the four V metadata waves

  // XCD-aware order: consecutive dispatch slots go round-robin over the 8 XCDs, so logical
  // workgroup index i*(N/8)+x runs on XCD x and one KV head's workgroups share an L2.
  const int n = a.n_wg, full = n & ~7, bid = blockIdx.x;
  const int logical = bid < full ? (bid & 7) * (full >> 3) + (bid >> 3) : bid;
  const int head = logical / a.wg_per_head, wgi = logical % a.wg_per_head;
  const int bi = head / a.hkv, h = head % a.hkv;

  // Tasks (query head in group fastest, 32-query tiles last-first); this wave's task and the
  // workgroup's last key tile.
  const int task = wgi * W + wave;
  const bool has_task = task < a.G * a.nqt;
  const int hq_i = h * a.G + (has_task ? task % a.G : 0);
  const int qt = has_task ? a.nqt - 1 - task / a.G : 0;
  const int qt_max = a.nqt - 1 - (wgi * W) / a.G;
  const int kt_max = (kQTile * qt_max + kQTile - 1) / kTile;
  const int nbq = kt_max / TPB + 1;  // blocks touched by this workgroup

  // The visible blocks of this head up to the workgroup's last key tile, compacted in order
  // (ballot per wave, then the counts of the lower waves as the offset).
  int32_t *lmodes = reinterpret_cast<int32_t *>(lds + L::kListModes);
  int16_t *lblk = reinterpret_cast<int16_t *>(lds + L::kListBlk);
  int32_t *wcount = reinterpret_cast<int32_t *>(lds + L::kCount);
  const char *didx = lds + L::kDenseIdx, *zp = lds + L::kZero;
  if (kSmfmac && tid < 256) reinterpret_cast<uint32_t *>(lds + L::kDenseIdx)[tid] = 0x44444444u;
  if (kSmfmac && tid < 32) reinterpret_cast<uint32_t *>(lds + L::kZero)[tid] = 0u;
  int32_t *wkind = reinterpret_cast<int32_t *>(lds + L::kKind);
  int n_vis = 0, kinds = 0;
  {
    const int32_t *mkh = a.c.map_k + (size_t)head * a.nb, *mvh = a.c.map_v + (size_t)head * a.nb;
    for (int base = 0; base < nbq; base += W * 64) {
      const int j = base + tid;
      const int mk = j < nbq ? mkh[j] : 0, mv = j < nbq ? mvh[j] : 0;
      const uint64_t vis = __builtin_amdgcn_ballot_w64(mk != 0);
      const int rank = __builtin_amdgcn_mbcnt_hi(
          (uint32_t)(vis >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)vis, 0u));
      if (lane == 0) wcount[wave] = __builtin_popcountll(vis);
      __syncthreads();
      int off = n_vis;
#pragma unroll
      for (int w2 = 0; w2 < W; ++w2) {
        const int cw = wcount[w2];
        off += w2 < wave ? cw : 0;
        n_vis += cw;
      }
      kinds |= (__builtin_amdgcn_ballot_w64(mk != 0 && (mk > 0 || mv > 0)) != 0 ? 1 : 0) |
               (__builtin_amdgcn_ballot_w64(mk != 0 && (mk < 0 || mv < 0)) != 0 ? 2 : 0);
      if (lane == 0) wkind[wave] = kinds;
      if (mk != 0) {
        const int sk = mk > 0 ? mk - head * a.ndk : mk + head * a.nsk;
        const int sv = mv > 0 ? mv - head * a.ndv : mv + head * a.nsv;
        lmodes[off + rank] = (sk << 16) | (sv & 0xFFFF);
        lblk[off + rank] = (int16_t)j;
      }
      __syncthreads();  // list entries visible; counts free for the next round
    }
  }
  n_vis = __builtin_amdgcn_readfirstlane(n_vis);
  kinds = 0;
#pragma unroll
  for (int w2 = 0; w2 < W; ++w2) kinds |= wkind[w2];
  kinds = __builtin_amdgcn_readfirstlane(kinds);

  WaveState<E> w;
  {
    const uint16_t *qp =
        a.q + (((size_t)bi * a.hq + hq_i) * a.L + (size_t)kQTile * qt + r) * kD + 8 * hf;
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      w.qv[u] = as16<E>(has_task ? *reinterpret_cast<const uint4 *>(qp + 16 * u) : z,
                           has_task ? *reinterpret_cast<const uint4 *>(qp + 16 * u + 64) : z);
  }
  // Retire the Q loads here with a wait the compiler sees, so it never re-waits on them inside
  // the loop (where its vmcnt count would also drain the in-flight K/V prefetch).
  __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) w.o[ct] = zero16();
  w.m_run = -INFINITY;
  w.l_run = 0.f;

  LaneOffsets lo;
  {
    const int f16 = r & 15, f8 = (r >> 1) & 7, f4 = (r >> 2) & 3;
    lo.kd = r * 256 + 32 * (f16 >> 1) + 16 * (hf ^ (f16 & 1));
    lo.kn = r * 128 + 16 * ((4 * hf) ^ f8);
    lo.km = kMetaOff + r * 16 + 8 * hf;
    lo.vd = kRegion + r * 128 + 16 * ((2 * hf) ^ f8);
    lo.vdd = kRegion + r * 128 + 32 * (f8 >> 1) + 16 * (hf ^ (f8 & 1));
    lo.vn = kRegion + r * 64 + 32 * (f4 >> 1) + 16 * (hf ^ (f4 & 1));
    lo.vm = kVMetaOff + r * 8;
    lo.vsel = hf ? 0x07060302u : 0x05040100u;
  }

  const uint32_t lds_base = (uint32_t)(size_t)(__attribute__((address_space(3))) char *)lds;

  // Tile t of the walk: half t % TPB of visible block t / TPB (block modes mk, mv as slot codes).
  auto tile_info = [&](int t, int &kt, int &mk, int &mv) {
    const int i = t / TPB;
    const int e = __builtin_amdgcn_readfirstlane(lmodes[i]);
    kt = __builtin_amdgcn_readfirstlane((int)lblk[i]) * TPB + t % TPB;
    mk = e >> 16;
    mv = (int)(int16_t)(e & 0xFFFF);
  };
  // The last visible block can reach past the last key tile (block 128: its second half).
  const int n_tiles =
      n_vis == 0 ? 0
                 : n_vis * TPB - ((__builtin_amdgcn_readfirstlane((int)lblk[n_vis - 1]) + 1) *
                                          TPB - 1 > kt_max ? 1 : 0);
  // Per-lane global byte offsets of this wave's direct loads: one per region (for K, one per
  // GEMM1 row order, see tau). Load i of a region (LDS bytes 1024 (wave + W i) on) is the same
  // lane pattern 4 W i (dense K), 8 W i (2:4 K, dense V^T) or 16 W i (2:4 V^T) rows further on,
  // a per-load constant: those row steps are multiples of 16, which the unit swizzles and the
  // token order tau leave alone.
  uint32_t oKd[2], oKn[2], oKm[2], oVd, oVn, oVm;
  {
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
      auto token = [&](int slot) {
        return (A & kAblLdsRelayout) ? slot : (slot & ~31) | tau(slot & 31, sp);
      };
      const int rd = 4 * wave + (lane >> 4), cd = lane & 15;   // dense K: 16 units per row
      oKd[sp] = token(rd) * 256 + 16 * (cd ^ (rd & 15));
      const int rn = 8 * wave + (lane >> 3), cn = lane & 7;    // 2:4 K: 8 units per row
      oKn[sp] = token(rn) * 128 + 16 * (cn ^ ((rn >> 1) & 7));
      oKm[sp] = token(lane) * 16;
    }
    const int rd = 8 * wave + (lane >> 3), cd = lane & 7;      // dense V^T: 8 units per row
    oVd = rd * (2 * B) + 16 * (cd ^ ((rd >> 1) & 7));
    const int rn = 16 * wave + (lane >> 2), cn = lane & 3;     // 2:4 V^T: 4 units per row
    oVn = rn * B + 16 * (cn ^ ((rn >> 2) & 3));
    const int d = 64 * (wave - kVmWave0) + lane;  // block 128: dword loads 0..3
    oVm = B == 64 ? 16 * lane : (d >> 1) * (B / 8) + 4 * (d & 1);
  }

  // Direct loads of one tile (block modes mk, mv) into a stage: dense regions 16 / W 1 KB loads
  // per wave, 2:4 values 8 / W, metadata one load by one wave (block 128: four dword loads by
  // waves kVmWave0 .. kVmWave0 + 3).
  const uint16_t *kd_h = a.c.k_dense + (size_t)head * a.ndk * B * kD;
  const uint16_t *kn_h = a.c.k_nnz + (size_t)head * a.nsk * B * (kD / 2);
  const uint16_t *km_h = a.c.k_meta + (size_t)head * a.nsk * B * (kD / 16);
  const uint16_t *vd_h = a.c.v_dense + (size_t)head * a.ndv * B * kD;
  const uint16_t *vn_h = a.c.v_nnz + (size_t)head * a.nsv * B * (kD / 2);
  const uint16_t *vm_h = a.c.v_meta + (size_t)head * a.nsv * B * (kD / 16);
  // Byte address of element e of a per-head array. A head holds at most kMaxBlocks blocks of at
  // most 128 x 128 elements, so 2 e fits 32 unsigned bits: one 32-bit shift, one 64-bit add.
  auto elem_at = [](const uint16_t *base, int e) __attribute__((always_inline)) {
    return reinterpret_cast<const char *>(base) + (uint32_t)e * 2u;
  };
  auto issue = [&](int kt, int mk, int mv, int stage, auto kind_tag) {
    constexpr int KIND = decltype(kind_tag)::value;
    const int half = kt % TPB;
    const uint32_t kl = lds_base + stage * L::kStride, vl = kl + kRegion;
    const uint32_t ksl = kl + SP, vsl = vl + SP;  // 2:4 buffers
    const int sp = (kSmfmac && mv > 0) ? 1 : 0;  // GEMM1 row order of this tile (see tau)
    // The kinds are constants on the specialised walks; on the general one 2:4 tiles are the
    // common case.
    if (KIND == 2 || (KIND == 0 && __builtin_expect(mk > 0, 0))) {
      const char *g = uniform_ptr(elem_at(kd_h, ((mk - 1) * B + kTile * half) * kD));
      const uint32_t o = sp ? oKd[1] : oKd[0];
      const char *gr[16 / W];
#pragma unroll
      for (int i = 0; i < 16 / W; ++i) gr[i] = g + i * (4 * W) * 2 * kD;
      dma16_run<16 / W>(gr, o, kl + 1024 * wave, 1024 * W);
    } else {
      const int row0 = (-mk - 1) * B + kTile * half;
      const char *g = uniform_ptr(elem_at(kn_h, row0 * (kD / 2)));
      const uint32_t o = sp ? oKn[1] : oKn[0];
      const char *gs[8 / W];
#pragma unroll
      for (int i = 0; i < 8 / W; ++i) gs[i] = g + i * (8 * W) * kD;
      dma16_run<8 / W>(gs, o, ksl + 1024 * wave, 1024 * W);
      if (wave == 1)
        dma16(uniform_ptr(elem_at(km_h, row0 * (kD / 16))), sp ? oKm[1] : oKm[0], ksl + kMetaOff);
    }
    if (KIND == 2 || (KIND == 0 && __builtin_expect(mv > 0, 0))) {
      const char *g = uniform_ptr(elem_at(vd_h, (mv - 1) * B * kD + kTile * half));
      const char *gr[16 / W];
#pragma unroll
      for (int i = 0; i < 16 / W; ++i) gr[i] = g + i * (8 * W) * 2 * B;
      dma16_run<16 / W>(gr, oVd, vl + 1024 * wave, 1024 * W);
    } else {
      const int blk = (-mv - 1) * B * kD;
      const char *g = uniform_ptr(elem_at(vn_h, blk / 2 + (kTile / 2) * half));
      // 16 rows per load; load q = wave + W i covers rows 16 q .., and rows 32 ct + .. start at
      // ct * kCtStride: LDS offset (q >> 1) kCtStride + 1024 (q & 1), a step of W / 2 groups per i.
      const char *gs[8 / W];
#pragma unroll
      for (int i = 0; i < 8 / W; ++i) gs[i] = g + i * (16 * W) * B;
      dma16_run<8 / W>(gs, oVn, vsl + (wave >> 1) * kCtStride + 1024 * (wave & 1),
                       (W / 2) * kCtStride);
      const char *gm = uniform_ptr(elem_at(vm_h, blk / 16 + (kTile / 16) * half));
      if (B == 64) {
        if (wave == 2) dma16(gm, oVm, ksl + kVMetaOff);
      } else if (wave >= kVmWave0 && wave < kVmWave0 + 4) {
        dma4(gm, oVm, ksl + kVMetaOff + 256 * (wave - kVmWave0));
      }
    }
  };
  const float c = a.scale_log2;
  constexpr int NS = L::kStagesN;
  // Tile it of the walk is computed from stage it % NS while tile it + 1 lands in the next stage.
  int kt0 = 0, mk0 = 0, mv0 = 0;
  if (n_tiles > 0) {
    tile_info(0, kt0, mk0, mv0);
    issue(kt0, mk0, mv0, 0, std::integral_constant<int, 0>{});
  }

  // Every wave walks every tile the workgroup stages (uniform control flow); tiles beyond a wave's
  // own queries are fully masked by the causal test and contribute nothing.
  if constexpr (!kSmfmac) {
    // Decompress path: each tile's 2:4 operands are expanded once into the dense scratch tile
    // (one more barrier), then GEMM1, the softmax and GEMM2 of the tile run on dense operands.
    char *scratch = lds + L::kScratch;
    int stage = 0;
    for (int it = 0; it < n_tiles; ++it) {
      int kt1 = 0, mk1 = 0, mv1 = 0;
      const bool more = it + 1 < n_tiles;
      if (more) tile_info(it + 1, kt1, mk1, mv1);
      const int next_stage = stage == NS - 1 ? 0 : stage + 1;
      wait_vmem(0);  // this wave's loads of tile it have landed
      barrier();     // ... and every wave's; the scratch tile of tile it - 1 is no longer read
      if (more) issue(kt1, mk1, mv1, next_stage, std::integral_constant<int, 0>{});

      const char *st = lds + stage * L::kStride;
      const bool sparse_k = mk0 < 0, sparse_v = mv0 < 0;
      if (sparse_k || sparse_v) {
        expand_tile<E>(st, scratch, sparse_k, sparse_v, tid);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      }
      gemm1<false>(w, sparse_k ? scratch : st, lo, hf, zp);
      const int shift = kTile * kt0 - kQTile * qt;
      const bool need = softmax_max(w, shift > -kTile, false, shift, r, hf, c);
      const float mc = w.m_use == -INFINITY ? 0.f : w.m_use;
      float lsum = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) softmax_exp(w, ks, c, mc, lsum);
      softmax_finish(w, need, lsum);  // O rescaled before this tile's P V^T is added
      const char *vb = sparse_v ? scratch : st;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) gemm2_dense_step<E>(w, vb, ks, lo);
      stage = next_stage;
      kt0 = kt1;
      mk0 = mk1;
      mv0 = mv1;
    }
  } else {
    // The tile walk, specialised at compile time when every visible block of the workgroup has
    // both operands 2:4 (KIND 1) or both dense (KIND 2): the tile kinds are then constants and
    // the body has no branches on them. KIND 0 tests each tile.
    // Causal mask, running max, exponentials and row sums of the tile in w.s (key tile kt, V of
    // the tile 2:4 or not); P^T lands in w.p and O, l are rescaled if the max moves.
    auto softmax_tile = [&](int kt, bool sparse_v) __attribute__((always_inline)) {
      const int shift = kTile * kt - kQTile * qt;
      constexpr bool kNat = (A & kAblLdsRelayout) != 0;
      if (shift > -kTile) softmax_mask<kNat>(w, !sparse_v, shift, r, hf);
      auto exps = [&]() __attribute__((always_inline)) {
        const float mc = w.m_use == -INFINITY ? 0.f : w.m_use;
        float ls = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          softmax_exp(w, ks, c, mc, ls);
          if constexpr (kNat) {
            if (ks & 1)
              relayout_through_lds(w, ks >> 1, lds + L::kPBuf + 2048 * wave, !sparse_v,
                                   lane & 31, hf);
          }
        }
        return ls;
      };
      // The exponentials are taken against the running max first. The tile's maxima are needed
      // only while a row has no max yet, or when a row's probabilities could exceed 2^kTau,
      // which the sum of a lane's 32 of them reveals; then the max may move and the exponentials
      // are taken again against the new one.
      bool need;
      float lsum;
      // (the LDS re-layout variant always takes the tile max first: its round trip leaves no
      // registers for a second copy of the exponentials)
      if (kNat || __builtin_amdgcn_ballot_w64(w.m_run == -INFINITY) != 0) {
        need = softmax_rescale(w, c);
        lsum = exps();
      } else {
        w.m_use = w.m_run;
        w.alpha = 1.f;
        lsum = exps();
        need = false;
        if (__builtin_amdgcn_ballot_w64(lsum > kLazyBound) != 0) {
          need = softmax_rescale(w, c);
          if (need) lsum = exps();
        }
      }
      softmax_finish(w, need, lsum);
    };
    auto walk = [&](auto kind_tag) {
      constexpr int KIND = decltype(kind_tag)::value;
      auto kinds_of = [&](int mk, int mv, bool &sk, bool &sv) {
        sk = KIND == 0 ? mk < 0 : KIND == 1;
        sv = KIND == 0 ? mv < 0 : KIND == 1;
      };
      if constexpr (W == 4) {
        // Two workgroups per CU, two stages: GEMM2 of a tile follows its softmax in the same
        // step, and the other workgroup's waves on the SIMD fill its dependency waits.
        int stage = 0;
        for (int it = 0; it < n_tiles; ++it) {
          int kt1 = 0, mk1 = 0, mv1 = 0;
          const bool more = it + 1 < n_tiles;
          if (more) tile_info(it + 1, kt1, mk1, mv1);
          if constexpr ((A & kAblSyncLoads) != 0) {
            // ablation: the tile's own loads, waited for at once (no overlap with computing)
            if (it > 0) issue(kt0, mk0, mv0, stage, kind_tag);
            wait_vmem(0);
            barrier();
          } else {
            wait_vmem(0);  // this wave's loads of tile it have landed
            barrier();     // ... and every wave's; the other stage (tile it - 1) is no longer read
            if (more) issue(kt1, mk1, mv1, stage ^ 1, kind_tag);
          }
          const char *st = lds + stage * L::kStride;
          bool sparse_k, sparse_v;
          kinds_of(mk0, mv0, sparse_k, sparse_v);
          if (sparse_k)
            gemm1<true>(w, st + SP, lo, hf, zp);
          else
            gemm1<false>(w, st, lo, hf, zp);
          const char *sv = sparse_v ? st + SP : st;
          // GEMM2's first operand reads go out before the softmax, whose vector work then covers
          // their latency.
          VOps v;
          gemm2_read(v, sv, sparse_v, 0, lo, didx);
          __builtin_amdgcn_sched_barrier(0);
          // The wave runs its matrix phase (GEMM2 of this tile, GEMM1 of the next) at raised
          // priority, so that when both waves of a SIMD can issue, the matrix instruction goes
          // first and the softmax of the other wave fills the matrix core's busy cycles.
          __builtin_amdgcn_s_setprio(0);
          softmax_tile(kt0, sparse_v);  // O rescaled before this tile's P V^T is added
          __builtin_amdgcn_s_setprio(1);
          gemm2_apply(w, v, sparse_v, 0, hf);
          gemm2_read(v, sv, sparse_v, 1, lo, didx);
          gemm2_apply(w, v, sparse_v, 1, hf);
          kt0 = kt1;
          mk0 = mk1;
          stage ^= 1;
          mv0 = mv1;
        }
      } else {
        // One workgroup per CU, three stages: GEMM2 of a tile runs one tile late, beside the
        // exponentials of the next.
        bool prev_sparse_v = KIND == 1;
        const char *st_prev = lds;
        int stage = 0;
        for (int it = 0; it < n_tiles; ++it) {
          int kt1 = 0, mk1 = 0, mv1 = 0;
          const bool more = it + 1 < n_tiles;
          if (more) tile_info(it + 1, kt1, mk1, mv1);
          const int next_stage = stage == NS - 1 ? 0 : stage + 1;
          wait_vmem(0);  // this wave's loads of tile it have landed
          barrier();     // ... and every wave's; stage next_stage (tile it - 2) is no longer read
          if (more) issue(kt1, mk1, mv1, next_stage, kind_tag);
          const char *st = lds + stage * L::kStride;
          bool sparse_k, sparse_v;
          kinds_of(mk0, mv0, sparse_k, sparse_v);
          if (sparse_k)
            gemm1<true>(w, st + SP, lo, hf, zp);
          else
            gemm1<false>(w, st, lo, hf, zp);
          const int shift = kTile * kt0 - kQTile * qt;
          const bool need = softmax_max(w, shift > -kTile, !sparse_v, shift, r, hf, c);
          const char *sv_prev = prev_sparse_v ? st_prev + SP : st_prev;
          const float lsum = exp_and_gemm2(w, sv_prev, it > 0, prev_sparse_v, lo, hf, c, didx);
          softmax_finish(w, need, lsum);
          prev_sparse_v = sparse_v;
          st_prev = st;
          stage = next_stage;
          kt0 = kt1;
          mk0 = mk1;
          mv0 = mv1;
        }
        // GEMM2 of the last tile (its stage is not overwritten after the loop).
        if (n_tiles > 0)
          gemm2_smfmac(w, prev_sparse_v ? st_prev + SP : st_prev, prev_sparse_v, lo, hf, didx);
      }
    };
    if (kinds == 2 && !(A & kAblGenericWalk))
      walk(std::integral_constant<int, 1>{});
    else if (kinds == 1 && !(A & kAblGenericWalk))
      walk(std::integral_constant<int, 2>{});
    else
      walk(std::integral_constant<int, 0>{});
  }

  if (!has_task) return;
  // ---- O = O^T / l, log-sum-exp ----
  const float l = sum_halves(w.l_run);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const size_t qrow = ((size_t)bi * a.hq + hq_i) * a.L + (size_t)kQTile * qt + r;
  uint16_t *op = a.o + qrow * kD + 4 * hf;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x16 &acc = w.o[ct];
      const uint2 v = make_uint2(pack2<E>(acc[4 * j] * inv, acc[4 * j + 1] * inv),
                                 pack2<E>(acc[4 * j + 2] * inv, acc[4 * j + 3] * inv));
      *reinterpret_cast<uint2 *>(op + 32 * ct + 8 * j) = v;
    }
  if (a.lse && hf == 0) a.lse[qrow] = l > 0.f ? (w.m_run + log2f(l)) * kLn2 : -INFINITY;
}

// Workgroups of W waves: each takes W (query head, 32-query tile) tasks of one KV head.
template <int W>
void set_grid(PrefillArgs &a, int b) {
  a.wg_per_head = (a.G * a.nqt + W - 1) / W;
  a.n_wg = b * a.hkv * a.wg_per_head;
}
template <int B, class E>
hipError_t launch_b(PrefillArgs a, int b, bool smfmac, hipStream_t stream) {
  if (smfmac && a.nb <= Lay<4, true>::kMaxB) {
    set_grid<4>(a, b);
    k_prefill<B, 4, true, E><<<a.n_wg, 4 * 64, 0, stream>>>(a);
  } else if (smfmac) {
    set_grid<kWaves>(a, b);
    k_prefill<B, kWaves, true, E><<<a.n_wg, kWaves * 64, 0, stream>>>(a);
  } else {
    set_grid<kWaves>(a, b);
    k_prefill<B, kWaves, false, E><<<a.n_wg, kWaves * 64, 0, stream>>>(a);
  }
  return hipGetLastError();
}
// Ablation variants of the SMFMAC path, bf16 (measurement only).
template <int B>
hipError_t launch_variant_b(PrefillArgs a, int b, int variant, hipStream_t stream) {
  if (variant == kPrefillVariantLockstep) {
    set_grid<kWaves>(a, b);
    k_prefill<B, kWaves, true, __bf16><<<a.n_wg, kWaves * 64, 0, stream>>>(a);
    return hipGetLastError();
  }
  set_grid<4>(a, b);
  switch (variant) {
    case 0: k_prefill<B, 4, true, __bf16><<<a.n_wg, 256, 0, stream>>>(a); break;
    case kAblSyncLoads:
      k_prefill<B, 4, true, __bf16, kAblSyncLoads><<<a.n_wg, 256, 0, stream>>>(a);
      break;
    case kAblNoAlias:
      k_prefill<B, 4, true, __bf16, kAblNoAlias><<<a.n_wg, 256, 0, stream>>>(a);
      break;
    case kAblGenericWalk:
      k_prefill<B, 4, true, __bf16, kAblGenericWalk><<<a.n_wg, 256, 0, stream>>>(a);
      break;
    case kAblLdsRelayout:
      if (a.nb > Lay<4, true, kAblLdsRelayout>::kMaxB) return hipErrorInvalidValue;
      k_prefill<B, 4, true, __bf16, kAblLdsRelayout><<<a.n_wg, 256, 0, stream>>>(a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class E>
hipError_t launch_e(const PrefillArgs &a, int b, int block, bool smfmac, hipStream_t stream) {
  return block == 64 ? launch_b<64, E>(a, b, smfmac, stream)
                     : launch_b<128, E>(a, b, smfmac, stream);
}

}  // namespace

namespace {
PrefillArgs prefill_args(const Dims &d, const CacheView &c, const uint16_t *q, uint16_t *o,
                         float *lse, float scale_log2) {
  PrefillArgs a;
  a.c = c;
  a.q = q;
  a.o = o;
  a.lse = lse;
  a.L = d.L;
  a.nb = d.nb;
  a.hkv = d.hkv;
  a.hq = d.hq;
  a.G = d.G;
  a.nqt = d.L / kQTile;
  a.ndk = d.ndk;
  a.nsk = d.nsk;
  a.ndv = d.ndv;
  a.nsv = d.nsv;
  a.scale_log2 = scale_log2;
  return a;
}
}  // namespace

hipError_t launch_prefill(const Dims &d, const CacheView &c, const uint16_t *q, uint16_t *o,
                          float *lse, float scale_log2, bool smfmac, hipStream_t stream) {
  const PrefillArgs a = prefill_args(d, c, q, o, lse, scale_log2);
  return d.dtype == kF16 ? launch_e<_Float16>(a, d.b, d.B, smfmac, stream)
                         : launch_e<__bf16>(a, d.b, d.B, smfmac, stream);
}

hipError_t launch_prefill_variant(const Dims &d, const CacheView &c, const uint16_t *q,
                                  uint16_t *o, float *lse, float scale_log2, int variant,
                                  hipStream_t stream) {
  if (d.dtype != kBf16 || d.nb > Lay<4, true>::kMaxB) return hipErrorInvalidValue;
  const PrefillArgs a = prefill_args(d, c, q, o, lse, scale_log2);
  return d.B == 64 ? launch_variant_b<64>(a, d.b, variant, stream)
                   : launch_variant_b<128>(a, d.b, variant, stream);
}

}  // namespace hs
