/*
 * hierasparse.h -- C ABI of libhierasparse.so: hierarchical semi-structured sparse KV attention
 * on MI355X (gfx950).
 *
 * The operations follow "HieraSparse: Hierarchical Semi-Structured Sparse KV Attention"
 * (arXiv 2604.16864v2, cited as [HS]):
 *   hs_compress      [HS] §III-A Eq. (2a)-(2d) magnitude pruner + §III-B memory pools and signed
 *                    block index map + §IV-B fused magnitude compression kernel.
 *   hs_decode_attn   [HS] Eq. (1) over the compressed cache, §IV-C split-KV decode with a
 *                    log-sum-exp combine step and GQA packing.
 *   hs_prefill_attn  [HS] §III-C Algorithm 1 with the mixed dense/sparse dispatch of §III-C2,
 *                    made causal, skipping pruned blocks.
 *   hs_prefill_attn_variant  the prefill with one optimisation of [HS] §IV-C left out (Fig. 4).
 *   hs_recompress    [HS] §III, Fig. 3: the cache compressed again with other block counts (e.g.
 *                    K dense and V 2:4 for prefill, then both 2:4 for decode).
 *   hs_compress_masked  [HS] §III-A cache pruner fed by any pruning algorithm's block-level and
 *                    element-level masks + §IV-B generic compression kernel.
 *   hs_compress_ex   hs_compress with the sink / local-window dense policy of the quality runs
 *                    ([HS] §V-A).
 *
 * Conventions shared by every entry point
 *   - bf16 or fp16 tensors (hs_shape.dtype) are passed as uint16_t bit patterns; all tensors are
 *     dense row-major.
 *   - Every pointer except the size-query outputs is a DEVICE pointer owned by the caller. The
 *     library allocates no memory and keeps no state besides a thread-local error string.
 *   - Work is enqueued asynchronously on 'stream' (a hipStream_t; NULL = the default stream).
 *     Calls on different streams may run concurrently if their buffers do not overlap.
 *   - All arguments are validated on the host before anything is launched. On any error the
 *     call returns a non-zero hs_status, enqueues nothing, and hs_last_error() describes it.
 *     Faults inside a launched kernel surface at the caller's next synchronisation.
 *   - Inputs must be finite with |x| < 2^24 (the compressor's integer loss keys rely on it; every
 *     finite fp16 value is); this is documented, not checked.
 *   - GPU limits: head_dim = 128, block in {64, 128}, seq_len % block = 0,
 *     seq_len / block <= 4096, q_heads % kv_heads = 0. Every pointer must be 16-byte aligned.
 *
 * Block modes and the compressed cache (per batch entry b and KV head h, independently)
 *   The sequence is cut into nb = seq_len / block blocks. Each block is pruned (its tokens are
 *   dropped from attention for K and V together), dense, or 2:4 (two of every four elements kept,
 *   [HS] §III-A); K and V choose dense or 2:4 independently. K is 2:4 along head_dim (groups of four
 *   consecutive channels of one token), V along tokens (four consecutive tokens of one channel):
 *   each tensor is sparse along the reduction axis of the product that consumes it ([HS] §III-C1,
 *   Table II, "Trans-Both").
 *   Selection: the n_pruned blocks with the smallest sum of |x| over K and V are pruned; among the
 *   rest, the n_sparse_k blocks with the smallest K 2:4 loss (sum of |x| of the dropped elements,
 *   [HS] Eq. (2c)) become K 2:4, and likewise for V. Losses are compared as integer sums of
 *   floor(|x| * 2^24); equal losses go to the lower block index. Within a group, the two largest
 *   |x| are kept; equal magnitudes go to the lower position.
 *
 *   map_k, map_v   int32 [batch][kv_heads][nb]: 0 = pruned, +(i + 1) = dense slot i,
 *                  -(i + 1) = 2:4 slot i. The slots of head (b, h) are the contiguous range
 *                  (b * kv_heads + h) * count .. + count - 1, assigned in block order.
 *   k_dense        [Nd_k][block][head_dim]      token-major copy of a K block
 *   k_nnz          [Ns_k][block][head_dim / 2]  kept K values, two per group, in position order
 *   k_meta         [Ns_k][block][head_dim / 16] 2-bit positions: group g of a token uses bits
 *                                               4*(g%4)..4*(g%4)+3 of word g/4, first kept
 *                                               position in the low two bits
 *   v_dense        [Nd_v][head_dim][block]      channel-major copy of a V block
 *   v_nnz          [Ns_v][head_dim][block / 2]  kept V values of each channel, two per group
 *   v_meta         [Ns_v][head_dim][block / 16] positions, same packing over token groups
 *   with Nd_x = batch * kv_heads * (nb - n_pruned - n_sparse_x), Ns_x = batch * kv_heads *
 *   n_sparse_x. A 2:4 block costs (1/2 + 1/16) of a dense one, matching [HS] Eq. (5c)-(5d).
 *
 * GQA: query head hq reads KV head hq / (q_heads / kv_heads).
 * A query with no visible token gets output 0 and log-sum-exp -inf.
 */
#ifndef HIERASPARSE_H
#define HIERASPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HS_OK = 0,
  HS_ERR_NULL = 1,        /* a required pointer is NULL */
  HS_ERR_SHAPE = 2,       /* shape outside the supported set (see limits above) */
  HS_ERR_COUNTS = 3,      /* negative counts or n_pruned + n_sparse_x > nb */
  HS_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  HS_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than hs_workspace_size() */
  HS_ERR_UNSUPPORTED = 6, /* valid request the library does not implement (e.g. flags) */
  HS_ERR_HIP = 7,         /* a HIP launch failed; hs_last_error() has the HIP message */
  HS_ERR_OVERLAP = 8      /* hs_recompress: input, output and workspace memory overlap */
} hs_status;

typedef struct {
  int32_t batch, q_heads, kv_heads;
  int32_t seq_len;  /* tokens in the cache (decode) or in the prompt (prefill) */
  int32_t head_dim; /* D */
  int32_t block;    /* B, tokens per block */
  int32_t dtype;    /* element type of K, V, Q and O: HS_BF16 (0) or HS_F16 (1) */
} hs_shape;

/* Element types. bf16 is the default; fp16 is the precision of [HS] §IV-A. The packed format,
   the metadata and the block modes are the same for both (the 2:4 selection compares the 16-bit
   magnitudes, which order both formats alike); loss keys are floor(|x| * 2^24) of the value. */
enum { HS_BF16 = 0, HS_F16 = 1 };

/* Block counts per (batch entry, KV head); the same for every head. */
typedef struct {
  int32_t n_pruned, n_sparse_k, n_sparse_v;
} hs_counts;

typedef struct {
  int32_t *map_k, *map_v;
  uint16_t *k_dense, *k_nnz, *k_meta;
  uint16_t *v_dense, *v_nnz, *v_meta;
} hs_cache;

typedef struct {
  size_t map_k, map_v, k_dense, k_nnz, k_meta, v_dense, v_nnz, v_meta;
} hs_cache_bytes;

/* Tokens kept dense by hs_compress_ex: the first sink_tokens and the last local_tokens of the
   sequence ([HS] §V-A keeps 64 and 256). */
typedef struct {
  int32_t sink_tokens, local_tokens;
} hs_policy;

enum { HS_OP_COMPRESS = 1, HS_OP_DECODE = 2, HS_OP_RECOMPRESS = 3 };

/* Prefill flags: how 2:4 blocks reach the matrix cores. */
enum {
  HS_PREFILL_SMFMAC = 0,    /* sparse MFMA (v_smfmac) on the packed values, the default */
  HS_PREFILL_DECOMPRESS = 1 /* expand 2:4 blocks to dense in LDS, then dense MFMA */
};

/* Bytes of every buffer of the compressed cache for this shape and these counts (host call, no
   GPU needed). A buffer of size 0 may be passed as NULL. */
hs_status hs_cache_sizes(const hs_shape *shape, const hs_counts *counts, hs_cache_bytes *out);

/* Workspace bytes needed by hs_compress (op = HS_OP_COMPRESS: three 8-byte loss keys per block),
   hs_decode_attn (op = HS_OP_DECODE: the fp32 partial outputs and log-sum-exps of every split;
   num_splits = 0 selects the same automatic split count hs_decode_attn uses) or
   hs_recompress (op = HS_OP_RECOMPRESS: dense K and V [batch][kv_heads][seq_len][head_dim] bf16,
   then the compressor's keys; the counts only need to be valid). Host call. */
hs_status hs_workspace_size(int op, const hs_shape *shape, const hs_counts *counts,
                            int32_t num_splits, size_t *bytes);

/* Compress K, V [batch][kv_heads][seq_len][head_dim] into 'out' (all eight buffers, sized by
   hs_cache_sizes). 'ws' is device scratch of hs_workspace_size(HS_OP_COMPRESS) bytes. Deterministic:
   the same input gives the same bytes. */
hs_status hs_compress(const hs_shape *shape, const hs_counts *counts, const uint16_t *k,
                      const uint16_t *v, const hs_cache *out, void *ws, size_t ws_bytes,
                      void *stream);

/* hs_compress with a dense policy: every block holding one of the first policy->sink_tokens or
   the last policy->local_tokens tokens is dense for K and V and takes no part in the ranking;
   the counts select among the other blocks, so n_pruned + n_sparse_k and n_pruned + n_sparse_v
   must not exceed their number (HS_ERR_COUNTS, also for a negative token count or one above
   seq_len). policy = NULL or {0, 0} is hs_compress. Same workspace as hs_compress
   (HS_OP_COMPRESS). Deterministic. */
hs_status hs_compress_ex(const hs_shape *shape, const hs_counts *counts, const hs_policy *policy,
                         const uint16_t *k, const uint16_t *v, const hs_cache *out, void *ws,
                         size_t ws_bytes, void *stream);

/* Compress with the caller's masks instead of the magnitude ranking. mode_k, mode_v: uint8
   [batch][kv_heads][nb] device arrays, one per block: 0 = pruned, 1 = dense, 2 = 2:4. The element
   mask must already be applied to k and v: in every group of four of a 2:4 block at most two
   values are non-zero (bf16 +0 and -0 count as zero). Such a group is stored as its non-zero
   values and their positions, padded with the lowest-position zeros to exactly two; a group with
   more non-zeros keeps its two largest |x| (lower position on ties), as hs_compress does.
   Per (batch entry, KV head) the modes must match 'counts': n_pruned blocks pruned for both K and
   V, n_sparse_k K blocks and n_sparse_v V blocks 2:4, no byte above 2. A head that does not is
   rejected: its maps are written as all pruned and its pool slots are left as they were.
   head_status (optional, int32 [batch][kv_heads] device array, NULL = not wanted) receives 0 for
   an accepted head, else the OR of 1 (a mode byte above 2), 2 (K and V disagree on a pruned
   block) and 4 (the numbers of K bytes equal to 0, K bytes equal to 2 and V bytes equal to 2
   are not n_pruned, n_sparse_k and n_sparse_v). Pool layout and slot order are those of
   hs_compress. No workspace. Deterministic. */
hs_status hs_compress_masked(const hs_shape *shape, const hs_counts *counts, const uint16_t *k,
                             const uint16_t *v, const uint8_t *mode_k, const uint8_t *mode_v,
                             const hs_cache *out, int32_t *head_status, void *stream);

/* Re-compress: 'out' becomes exactly what hs_compress with 'out_counts' produces from the dense
   K, V that 'in' (compressed with 'in_counts' by hs_compress or hs_recompress) stands for: kept
   values in place, zeros where a 2:4 group dropped an element and over pruned blocks. A block that
   is 2:4 or pruned in 'in' has zero loss for that mode, so it is chosen for it first again; dropped
   values are not recovered. No array of 'in', of 'out' and the workspace may overlap
   (HS_ERR_OVERLAP). 'ws' is device scratch of hs_workspace_size(HS_OP_RECOMPRESS) bytes.
   Deterministic. */
hs_status hs_recompress(const hs_shape *shape, const hs_counts *in_counts, const hs_cache *in,
                        const hs_counts *out_counts, const hs_cache *out, void *ws,
                        size_t ws_bytes, void *stream);

/* Decode attention of one new query per (batch entry, query head) over all seq_len cached
   tokens: q [batch][q_heads][head_dim] -> o [batch][q_heads][head_dim] (bf16), and if lse is not
   NULL, lse [batch][q_heads] (fp32, natural log). softmax_scale <= 0 selects 1/sqrt(head_dim).
   num_splits = 0 picks the split-KV factor automatically (1..512 otherwise). 'ws' is device
   scratch of hs_workspace_size(HS_OP_DECODE, ..., num_splits) bytes, with no required contents
   (every call writes the partials it reads); it serves any later call whose size it covers. The
   call launches the split kernel and, with more than one split, a combine kernel, both on
   'stream'. Two calls that run at the same time must not share a workspace. */
hs_status hs_decode_attn(const hs_shape *shape, const hs_counts *counts, const hs_cache *cache,
                         const uint16_t *q, uint16_t *o, float *lse, float softmax_scale,
                         int32_t num_splits, void *ws, size_t ws_bytes, void *stream);

/* Bytes of the device array hs_decode_attn_noalloc uses instead of a workspace (16 MiB). */
#define HS_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* hs_decode_attn without a workspace, for callers that cannot allocate device memory (code under
   HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the splits' partials
   live in a device array of HS_DECODE_NOALLOC_SCRATCH_BYTES that the library holds on
   each GPU until the process ends. Arguments, outputs and results are those of hs_decode_attn
   (same kernels, same split count). A call whose hs_workspace_size(HS_OP_DECODE, ..., num_splits)
   exceeds the array returns HS_ERR_WORKSPACE and launches nothing. The call allocates nothing
   and launches only the decode's own kernels. Every call on a GPU shares that GPU's array: two
   calls that overlap in time on one GPU (different streams, or different threads) race and give
   wrong results; calls ordered on one stream are safe. */
hs_status hs_decode_attn_noalloc(const hs_shape *shape, const hs_counts *counts,
                                 const hs_cache *cache, const uint16_t *q, uint16_t *o, float *lse,
                                 float softmax_scale, int32_t num_splits, void *stream);

/* Causal prefill attention: q [batch][q_heads][seq_len][head_dim] -> o (same shape, bf16) and,
   if lse is not NULL, lse [batch][q_heads][seq_len]. Query position i attends the visible tokens
   t <= i of the compressed cache of the same sequence. flags: HS_PREFILL_SMFMAC or
   HS_PREFILL_DECOMPRESS. No workspace. */
hs_status hs_prefill_attn(const hs_shape *shape, const hs_counts *counts, const hs_cache *cache,
                          const uint16_t *q, uint16_t *o, float *lse, float softmax_scale,
                          uint32_t flags, void *stream);

/* Variants of the SMFMAC prefill that each leave out one of its optimisations, for measuring
   what every optimisation is worth (the ablation of [HS] §IV-C, Fig. 4). Same arguments, outputs
   and results (up to the order of fp32 sums for LOCKSTEP and LDS_RELAYOUT) as hs_prefill_attn
   with HS_PREFILL_SMFMAC, for bf16 heads of at most 2048 blocks, 1024 for LDS_RELAYOUT
   (HS_ERR_UNSUPPORTED otherwise, or for another variant code). */
enum {
  HS_PREFILL_VARIANT_NONE = 0,         /* the SMFMAC kernel hs_prefill_attn runs */
  HS_PREFILL_VARIANT_SYNC_LOADS = 1,   /* no pipelining: a tile's loads are issued and waited for
                                          in the step that computes on it (§IV-C1) */
  HS_PREFILL_VARIANT_NO_ALIAS = 2,     /* dense and 2:4 forms of a stage in separate LDS buffers,
                                          so one workgroup per CU (§IV-C3) */
  HS_PREFILL_VARIANT_GENERIC_WALK = 4, /* no walk specialised for all-2:4 or all-dense workgroups
                                          (§IV-C3) */
  HS_PREFILL_VARIANT_LOCKSTEP = 8,     /* one eight-wave workgroup per CU, GEMM2 one tile late */
  HS_PREFILL_VARIANT_LDS_RELAYOUT = 16 /* K staged in token order, so P^T reaches GEMM2's operand
                                          layout through a round trip in LDS instead of being
                                          produced in place (§IV-C2, Fig. 5) */
};
hs_status hs_prefill_attn_variant(const hs_shape *shape, const hs_counts *counts,
                                  const hs_cache *cache, const uint16_t *q, uint16_t *o,
                                  float *lse, float softmax_scale, uint32_t variant, void *stream);

/* Static description of a status code. */
const char *hs_status_string(hs_status status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char *hs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HIERASPARSE_H */
