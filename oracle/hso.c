/*
 * hso.c -- plain fp64 CPU oracle for hierarchical semi-structured sparse KV attention.
 *
 * TEST INFRASTRUCTURE ONLY. The GPU library never links, includes or calls this file, and it
 * shares no header, helper or table with it. Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark use it.
 *
 * What it follows ("HieraSparse: Hierarchical Semi-Structured Sparse KV Attention",
 * arXiv 2604.16864v2, cited below as [HS]):
 *   - [HS] §II, Eq. (1): softmax attention with scale 1/sqrt(d).
 *   - [HS] §III-A, Eq. (2a)-(2d): magnitude pruner. Sequence blocks of B tokens; top-N:M element
 *     mask (N=2, M=4); block loss = L1 norm of what the element mask drops; the S_X fraction of
 *     blocks with the lowest loss becomes 2:4, the rest stays dense.
 *   - [HS] §III-B: dense / non-zero / metadata memory pools and the signed block index map, filled
 *     by sequential dense and sparse counters.
 *   - [HS] §III-C1, Table II ("Trans-Both"): K is 2:4 along head_dim, V is 2:4 along tokens.
 *   - [HS] §IV-A: 2-bit position metadata, eight entries per 16-bit word.
 *   - [HS] §IV-B: fused magnitude compression keeps the top-2 |x| of each 2:4 group.
 *
 * Readings where [HS] is silent, ambiguous or garbled (each is also repeated where it is used):
 *   R1 ties in the top-2 selection: exactly two are kept; of equal magnitudes the lower position
 *      in the group is kept.
 *   R2 block losses are compared as the integer sum of floor(|x| * 2^24) (exact for |x| >= 2^-17),
 *      ties between blocks broken by the lower block index; inputs must satisfy |x| < 2^24.
 *   R3 a third block state, "pruned", drops a block's tokens from attention for K and V together;
 *      the n_p blocks with the smallest total magnitude of K and V are pruned first, then K and V
 *      rank the surviving blocks independently. Ranking is per (batch, KV head).
 *   R4 index map: int32, pruned = 0, dense = +(offset + 1), 2:4 = -(offset + 1).
 *   R5 pool layouts (bf16 kept as raw little-endian uint16 bits):
 *        K dense [Nd][B][D] token-major copy;   K nnz [Ns][B][D/2];  K meta [Ns][B][D/16]
 *        V dense [Nd][D][B] channel-major copy; V nnz [Ns][D][B/2];  V meta [Ns][D][B/16]
 *      group g of a row keeps (i0 < i1) at nnz[2g], nnz[2g+1]; its metadata nibble sits at bits
 *      4*(g%4) .. 4*(g%4)+3 of word g/4 with i0 in the low two bits and i1 in the high two bits.
 *   R6 a query row whose visible set is empty gets output 0 and log-sum-exp -inf.
 *   R7 decode: the single query attends every visible cached token; prefill: query position i
 *      attends visible tokens t <= i (causal).
 *   R8 GQA: query head hq reads KV head hq / (Hq / Hkv).
 *   R9 re-compression ([HS] §III, Fig. 3) compresses what the cache holds: kept values in place,
 *      zeros for dropped elements and pruned blocks (oracle/__init__.py: recompress).
 *   R10 generic compression with caller masks ([HS] §III-A cache pruner, §IV-B generic kernel):
 *      a 2:4 group of the pre-masked input is stored as its non-zero elements (+0 and -0 are
 *      zero) in position order, padded with the lowest-position zeros to exactly two; a group
 *      with more than two non-zeros violates the mask and falls back to R1's top-2. A (batch,
 *      KV head) whose block modes do not match the pool counts is rejected: all-pruned map, no
 *      pool writes, a status bit.
 *   R11 dense policy ([HS] §V-A quality runs): a block holding any of the first 'sink' or the last
 *      'local' tokens stays dense for K and V and is not ranked; the counts select among the
 *      others.
 *   R12 element type: K, V, Q are bf16 or IEEE binary16 ([HS] §IV-A computes in fp16) bit
 *      patterns; the selection, the keys and the attention use the values they encode.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define HSO_OK 0
#define HSO_ERR_SHAPE 1
#define HSO_ERR_COUNTS 2
#define HSO_ERR_VALUE 3
#define HSO_ERR_MAP 4

/* ------------------------------------------------------------------------------------------ */
/* Element values (R12): bf16 (dtype 0) or IEEE binary16 (dtype 1), as 16-bit patterns.        */

static double bf16_value(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

/* binary16: sign, 5-bit exponent (bias 15), 10-bit fraction; exponent 0 is subnormal. */
static double f16_value(uint16_t bits) {
  int e = (bits >> 10) & 31, m = bits & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp(1024.0 + m, e - 25);
  return (bits & 0x8000u) ? -v : v;
}

static double value(uint16_t bits, int dtype) { return dtype ? f16_value(bits) : bf16_value(bits); }

/* R2: finite and |x| < 2^24 (bf16: exponent field at most 127 + 23; every finite fp16 value). */
static int in_range(uint16_t bits, int dtype) {
  if (dtype) return ((bits >> 10) & 31) != 31;
  return ((bits & 0x7FFFu) >> 7) <= 150u;
}
static int is_finite(uint16_t bits, int dtype) {
  return dtype ? (bits & 0x7C00u) != 0x7C00u : (bits & 0x7F80u) != 0x7F80u;
}

/* R2: the fixed-point magnitude floor(|x| * 2^24). |x| < 2^24 makes the product < 2^48, which a
   double holds exactly, so floor() of it is exact. */
static uint64_t fixed_magnitude(uint16_t bits, int dtype) {
  return (uint64_t)floor(fabs(value(bits, dtype)) * 16777216.0);
}

/* ------------------------------------------------------------------------------------------ */
/* Shapes                                                                                      */

typedef struct {
  int b, hkv, L, D, B;        /* batch, KV heads, tokens, head_dim, block size */
  int n_p, n_sk, n_sv;        /* per (batch, KV head): pruned, K 2:4, V 2:4 block counts */
  int dtype;                  /* R12: 0 bf16, 1 fp16 */
} hso_dims;

static int dims_check(const hso_dims *d) {
  if (d->b <= 0 || d->hkv <= 0 || d->L <= 0 || d->D <= 0 || d->B <= 0) return HSO_ERR_SHAPE;
  if (d->D % 16 || d->B % 16 || d->L % d->B) return HSO_ERR_SHAPE;
  if ((int64_t)2 * d->B * d->D > 32768) return HSO_ERR_SHAPE; /* keeps the loss keys < 2^63 */
  int nb = d->L / d->B;
  if (d->n_p < 0 || d->n_sk < 0 || d->n_sv < 0) return HSO_ERR_COUNTS;
  if (d->n_p + d->n_sk > nb || d->n_p + d->n_sv > nb) return HSO_ERR_COUNTS;
  return HSO_OK;
}

/* Element counts (uint16 elements for pools, int32 for maps) of every buffer of the compressed
   cache, in the order map_k, map_v, k_dense, k_nnz, k_meta, v_dense, v_nnz, v_meta. */
int hso_pool_elems(const hso_dims *d, int64_t out[8]) {
  int rc = dims_check(d);
  if (rc) return rc;
  int64_t heads = (int64_t)d->b * d->hkv, nb = d->L / d->B, BD = (int64_t)d->B * d->D;
  int64_t ndk = nb - d->n_p - d->n_sk, ndv = nb - d->n_p - d->n_sv;
  out[0] = heads * nb;
  out[1] = heads * nb;
  out[2] = heads * ndk * BD;
  out[3] = heads * d->n_sk * BD / 2;
  out[4] = heads * d->n_sk * BD / 16;
  out[5] = heads * ndv * BD;
  out[6] = heads * d->n_sv * BD / 2;
  out[7] = heads * d->n_sv * BD / 16;
  return HSO_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* Element level: [HS] Eq. (2a)-(2b) and the fused top-2 selection of §IV-B.                   */

/* Keep the two largest |x| of a group of four; R1 for ties. Returns the kept positions with
   *i0 < *i1. A stable insertion sort by |x|, descending, leaves equal magnitudes in position
   order, so the first two entries are the kept pair. */
static void keep_two(const uint16_t x[4], int dtype, int *i0, int *i1) {
  int order[4] = {0, 1, 2, 3};
  for (int p = 1; p < 4; ++p) {
    int j = order[p];
    double mj = fabs(value(x[j], dtype));
    int q = p - 1;
    while (q >= 0 && fabs(value(x[order[q]], dtype)) < mj) {
      order[q + 1] = order[q];
      --q;
    }
    order[q + 1] = j;
  }
  *i0 = order[0] < order[1] ? order[0] : order[1];
  *i1 = order[0] < order[1] ? order[1] : order[0];
}

/* R10: the generic kernel's selection for a group the caller's element mask already thinned. */
static void keep_nonzero(const uint16_t x[4], int dtype, int *i0, int *i1) {
  int pos[4], n = 0;
  for (int j = 0; j < 4; ++j)
    if (x[j] & 0x7FFFu) pos[n++] = j;
  if (n > 2) {
    keep_two(x, dtype, i0, i1);
    return;
  }
  for (int j = 0; j < 4 && n < 2; ++j)
    if (!(x[j] & 0x7FFFu)) pos[n++] = j;
  *i0 = pos[0] < pos[1] ? pos[0] : pos[1];
  *i1 = pos[0] < pos[1] ? pos[1] : pos[0];
}

typedef void (*select_fn)(const uint16_t x[4], int dtype, int *i0, int *i1);

/* The four elements of group g of block i, for K (4 consecutive channels of one token, row = the
   token within the block) or V (4 consecutive tokens of one channel, row = the channel). */
static void gather_group(const uint16_t *X, int is_v, int L, int D, int B, int i, int row, int g,
                         uint16_t x[4]) {
  (void)L;
  for (int j = 0; j < 4; ++j) {
    if (!is_v)
      x[j] = X[(int64_t)(i * B + row) * D + 4 * g + j];
    else
      x[j] = X[(int64_t)(i * B + 4 * g + j) * D + row];
  }
}

/* ------------------------------------------------------------------------------------------ */
/* Block level: [HS] Eq. (2c)-(2d) with R2 and R3.                                             */

typedef struct {
  uint64_t key;
  int idx;
} ranked;

static int ranked_cmp(const void *a, const void *b) {
  const ranked *x = (const ranked *)a, *y = (const ranked *)b;
  if (x->key != y->key) return x->key < y->key ? -1 : 1;
  return (x->idx > y->idx) - (x->idx < y->idx);
}

/*
 * hso_block_keys: per block of one (batch, KV head), the three losses of R2/R3:
 *   keys[3*i + 0] = K 2:4 loss (Eq. 2c on K), keys[3*i + 1] = V 2:4 loss (Eq. 2c on V),
 *   keys[3*i + 2] = loss of pruning the whole block = sum over all K and V elements,
 * as integers (R2) and, if loss != NULL, as fp64 L1 sums in the same order.
 * Kh, Vh point at one head's [L][D] tokens.
 */
static void block_keys(const hso_dims *d, const uint16_t *Kh, const uint16_t *Vh, uint64_t *keys,
                       double *loss) {
  int nb = d->L / d->B;
  for (int i = 0; i < nb; ++i) {
    uint64_t kk = 0, kv = 0, kp = 0;
    double fk = 0, fv = 0, fp = 0;
    for (int is_v = 0; is_v < 2; ++is_v) {
      const uint16_t *X = is_v ? Vh : Kh;
      int rows = is_v ? d->D : d->B, groups = is_v ? d->B / 4 : d->D / 4;
      for (int r = 0; r < rows; ++r)
        for (int g = 0; g < groups; ++g) {
          uint16_t x[4];
          int i0, i1;
          gather_group(X, is_v, d->L, d->D, d->B, i, r, g, x);
          keep_two(x, d->dtype, &i0, &i1);
          for (int j = 0; j < 4; ++j) {
            uint64_t q = fixed_magnitude(x[j], d->dtype);
            double a = fabs(value(x[j], d->dtype));
            kp += q;
            fp += a;
            if (j != i0 && j != i1) {
              if (is_v) { kv += q; fv += a; } else { kk += q; fk += a; }
            }
          }
        }
    }
    keys[3 * i + 0] = kk;
    keys[3 * i + 1] = kv;
    keys[3 * i + 2] = kp;
    if (loss) {
      loss[3 * i + 0] = fk;
      loss[3 * i + 1] = fv;
      loss[3 * i + 2] = fp;
    }
  }
}

/* Block modes of one head: mode_k[i], mode_v[i] in {0 = pruned, 1 = dense, 2 = 2:4}. Blocks with
   held[i] set stay dense and are not ranked (R11). */
static void block_modes(const hso_dims *d, const uint64_t *keys, const char *held, int *mode_k,
                        int *mode_v, ranked *scratch) {
  int nb = d->L / d->B, n = 0;
  /* R3 step 1: the n_p blocks with the smallest whole-block loss are pruned. */
  for (int i = 0; i < nb; ++i)
    if (!held[i]) { scratch[n].key = keys[3 * i + 2]; scratch[n].idx = i; ++n; }
  qsort(scratch, n, sizeof(ranked), ranked_cmp);
  for (int i = 0; i < nb; ++i) { mode_k[i] = 1; mode_v[i] = 1; }
  for (int r = 0; r < d->n_p; ++r) { mode_k[scratch[r].idx] = 0; mode_v[scratch[r].idx] = 0; }
  /* Eq. (2d) per tensor among the survivors: the n_sX smallest 2:4 losses become 2:4. */
  for (int t = 0; t < 2; ++t) {
    int *mode = t ? mode_v : mode_k;
    int want = t ? d->n_sv : d->n_sk;
    n = 0;
    for (int i = 0; i < nb; ++i)
      if (!held[i] && mode[i] != 0) { scratch[n].key = keys[3 * i + t]; scratch[n].idx = i; ++n; }
    qsort(scratch, n, sizeof(ranked), ranked_cmp);
    for (int r = 0; r < want; ++r) mode[scratch[r].idx] = 2;
  }
}

/* ------------------------------------------------------------------------------------------ */
/* Compressor: [HS] §III-B memory pools and index map, §IV-A/B packing.                        */

/* One 2:4 row: 'groups' groups gathered by gather_group -> nnz (2 per group), meta (1 per 4);
   'select' picks the two stored positions of a group. */
static void pack_row(const uint16_t *X, int is_v, const hso_dims *d, int i, int row, int groups,
                     select_fn select, uint16_t *nnz, uint16_t *meta) {
  for (int w = 0; w < groups / 4; ++w) meta[w] = 0;
  for (int g = 0; g < groups; ++g) {
    uint16_t x[4];
    int i0, i1;
    gather_group(X, is_v, d->L, d->D, d->B, i, row, g, x);
    select(x, d->dtype, &i0, &i1);
    nnz[2 * g] = x[i0];
    nnz[2 * g + 1] = x[i1];
    meta[g / 4] |= (uint16_t)((i0 | (i1 << 2)) << (4 * (g % 4)));
  }
}

/* [HS] §III-B: the pools and map entries of one (batch, KV head) from its block modes; walks the
   blocks in order with one dense and one sparse counter per tensor. Each head owns a contiguous
   range of each pool, so the counters start at head * count. */
static void write_head(const hso_dims *d, int64_t hd, const uint16_t *Kh, const uint16_t *Vh,
                       const int *mode_k, const int *mode_v, select_fn select, int32_t *map_k,
                       int32_t *map_v, uint16_t *k_dense, uint16_t *k_nnz, uint16_t *k_meta,
                       uint16_t *v_dense, uint16_t *v_nnz, uint16_t *v_meta) {
  const int nb = d->L / d->B, B = d->B, D = d->D;
  const int ndk = nb - d->n_p - d->n_sk, ndv = nb - d->n_p - d->n_sv;
  const int64_t BD = (int64_t)B * D;
  int64_t dk = hd * ndk, sk = hd * d->n_sk, dv = hd * ndv, sv = hd * d->n_sv;
  for (int i = 0; i < nb; ++i) {
    int32_t *mk = &map_k[hd * nb + i], *mv = &map_v[hd * nb + i];
    /* K: 2:4 along head_dim, one row per token. */
    if (mode_k[i] == 0) {
      *mk = 0;
    } else if (mode_k[i] == 1) {
      memcpy(k_dense + dk * BD, Kh + (int64_t)i * BD, sizeof(uint16_t) * BD);
      *mk = (int32_t)(dk + 1);
      ++dk;
    } else {
      for (int t = 0; t < B; ++t)
        pack_row(Kh, 0, d, i, t, D / 4, select, k_nnz + sk * BD / 2 + (int64_t)t * D / 2,
                 k_meta + sk * BD / 16 + (int64_t)t * D / 16);
      *mk = (int32_t)-(sk + 1);
      ++sk;
    }
    /* V: 2:4 along tokens, one row per channel; the dense copy is stored channel-major. */
    if (mode_v[i] == 0) {
      *mv = 0;
    } else if (mode_v[i] == 1) {
      for (int c = 0; c < D; ++c)
        for (int t = 0; t < B; ++t)
          v_dense[dv * BD + (int64_t)c * B + t] = Vh[(int64_t)(i * B + t) * D + c];
      *mv = (int32_t)(dv + 1);
      ++dv;
    } else {
      for (int c = 0; c < D; ++c)
        pack_row(Vh, 1, d, i, c, B / 4, select, v_nnz + sv * BD / 2 + (int64_t)c * B / 2,
                 v_meta + sv * BD / 16 + (int64_t)c * B / 16);
      *mv = (int32_t)-(sv + 1);
      ++sv;
    }
  }
}

/*
 * hso_compress: the whole compressor (R1-R5). K, V: [b][hkv][L][D] bf16 bits. Outputs are sized
 * by hso_pool_elems. keys (optional, [b][hkv][nb][3] uint64) and loss (optional, same shape,
 * fp64) receive the block losses. Returns HSO_ERR_VALUE if an input is non-finite or |x| >= 2^24.
 */
int hso_compress_ex(const hso_dims *d, int sink, int local, const uint16_t *K, const uint16_t *V,
                    int32_t *map_k, int32_t *map_v, uint16_t *k_dense, uint16_t *k_nnz,
                    uint16_t *k_meta, uint16_t *v_dense, uint16_t *v_nnz, uint16_t *v_meta,
                    uint64_t *keys_out, double *loss_out) {
  int rc = dims_check(d);
  if (rc) return rc;
  /* R11: a block holding any of the first 'sink' or the last 'local' tokens is not ranked. */
  if (sink < 0 || local < 0 || sink > d->L || local > d->L) return HSO_ERR_COUNTS;
  const int nblk = d->L / d->B;
  char *held = (char *)malloc(nblk);
  int n_ranked = 0;
  for (int i = 0; i < nblk; ++i) {
    held[i] = 0;
    for (int t = i * d->B; t < (i + 1) * d->B; ++t)
      if (t < sink || t >= d->L - local) held[i] = 1;
    n_ranked += !held[i];
  }
  if (d->n_p + d->n_sk > n_ranked || d->n_p + d->n_sv > n_ranked) {
    free(held);
    return HSO_ERR_COUNTS;
  }
  const int64_t heads = (int64_t)d->b * d->hkv, per_head = (int64_t)d->L * d->D;
  for (int64_t e = 0; e < heads * per_head; ++e)
    if (!in_range(K[e], d->dtype) || !in_range(V[e], d->dtype)) {
      free(held);
      return HSO_ERR_VALUE;
    }

  const int nb = d->L / d->B;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t hd = 0; hd < heads; ++hd) {
    const uint16_t *Kh = K + hd * per_head, *Vh = V + hd * per_head;
    uint64_t *keys = (uint64_t *)malloc(sizeof(uint64_t) * 3 * nb);
    double *loss = loss_out ? loss_out + hd * 3 * nb : NULL;
    int *mode_k = (int *)malloc(sizeof(int) * nb), *mode_v = (int *)malloc(sizeof(int) * nb);
    ranked *scratch = (ranked *)malloc(sizeof(ranked) * nb);
    block_keys(d, Kh, Vh, keys, loss);
    if (keys_out) memcpy(keys_out + hd * 3 * nb, keys, sizeof(uint64_t) * 3 * nb);
    block_modes(d, keys, held, mode_k, mode_v, scratch);
    write_head(d, hd, Kh, Vh, mode_k, mode_v, keep_two, map_k, map_v, k_dense, k_nnz, k_meta,
               v_dense, v_nnz, v_meta);
    free(keys);
    free(mode_k);
    free(mode_v);
    free(scratch);
  }
  free(held);
  return HSO_OK;
}

int hso_compress(const hso_dims *d, const uint16_t *K, const uint16_t *V, int32_t *map_k,
                 int32_t *map_v, uint16_t *k_dense, uint16_t *k_nnz, uint16_t *k_meta,
                 uint16_t *v_dense, uint16_t *v_nnz, uint16_t *v_meta, uint64_t *keys_out,
                 double *loss_out) {
  return hso_compress_ex(d, 0, 0, K, V, map_k, map_v, k_dense, k_nnz, k_meta, v_dense, v_nnz,
                         v_meta, keys_out, loss_out);
}

/*
 * hso_compress_masked: compression with the caller's masks ([HS] §III-A cache pruner, §IV-B
 * generic kernel; R10). mode_k, mode_v: [b][hkv][nb] bytes, 0 pruned / 1 dense / 2 2:4. K, V
 * carry the element mask already. head_status [b][hkv] receives 0, or the OR of 1 (a mode above
 * 2), 2 (K and V disagree on a pruned block), 4 (counts differ from d's); a rejected head gets an
 * all-pruned map and no pool writes. Returns HSO_ERR_VALUE if an input is not finite.
 */
int hso_compress_masked(const hso_dims *d, const uint16_t *K, const uint16_t *V,
                        const uint8_t *mode_k, const uint8_t *mode_v, int32_t *map_k,
                        int32_t *map_v, uint16_t *k_dense, uint16_t *k_nnz, uint16_t *k_meta,
                        uint16_t *v_dense, uint16_t *v_nnz, uint16_t *v_meta,
                        int32_t *head_status) {
  int rc = dims_check(d);
  if (rc) return rc;
  const int64_t heads = (int64_t)d->b * d->hkv, per_head = (int64_t)d->L * d->D;
  for (int64_t e = 0; e < heads * per_head; ++e)
    if (!is_finite(K[e], d->dtype) || !is_finite(V[e], d->dtype)) return HSO_ERR_VALUE;

  const int nb = d->L / d->B;
  for (int64_t hd = 0; hd < heads; ++hd) {
    const uint8_t *mk = mode_k + hd * nb, *mv = mode_v + hd * nb;
    int status = 0, n_p = 0, n_sk = 0, n_sv = 0;
    for (int i = 0; i < nb; ++i) {
      if (mk[i] > 2 || mv[i] > 2) status |= 1;
      if ((mk[i] == 0) != (mv[i] == 0)) status |= 2;
      n_p += mk[i] == 0;
      n_sk += mk[i] == 2;
      n_sv += mv[i] == 2;
    }
    if (n_p != d->n_p || n_sk != d->n_sk || n_sv != d->n_sv) status |= 4;
    head_status[hd] = status;
    if (status) {
      for (int i = 0; i < nb; ++i) map_k[hd * nb + i] = map_v[hd * nb + i] = 0;
      continue;
    }
    int *ik = (int *)malloc(sizeof(int) * nb), *iv = (int *)malloc(sizeof(int) * nb);
    for (int i = 0; i < nb; ++i) { ik[i] = mk[i]; iv[i] = mv[i]; }
    write_head(d, hd, K + hd * per_head, V + hd * per_head, ik, iv, keep_nonzero, map_k, map_v,
               k_dense, k_nnz, k_meta, v_dense, v_nnz, v_meta);
    free(ik);
    free(iv);
  }
  return HSO_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* Decompression: the dense tensors the compressed cache stands for.                           */

/*
 * hso_unpack: Kt, Vt [b][hkv][L][D] bf16 bits with the kept values in place and zeros elsewhere
 * (dense blocks copied back, pruned blocks zero); visible [b][hkv][nb] = 1 unless pruned.
 * Returns HSO_ERR_MAP if the two maps disagree on which blocks are pruned or an offset is out of
 * its pool.
 */
int hso_unpack(const hso_dims *d, const int32_t *map_k, const int32_t *map_v,
               const uint16_t *k_dense, const uint16_t *k_nnz, const uint16_t *k_meta,
               const uint16_t *v_dense, const uint16_t *v_nnz, const uint16_t *v_meta,
               uint16_t *Kt, uint16_t *Vt, uint8_t *visible) {
  int rc = dims_check(d);
  if (rc) return rc;
  const int nb = d->L / d->B, B = d->B, D = d->D;
  const int64_t heads = (int64_t)d->b * d->hkv, BD = (int64_t)B * D;
  const int64_t ndk = heads * (nb - d->n_p - d->n_sk), ndv = heads * (nb - d->n_p - d->n_sv);
  const int64_t nsk = heads * d->n_sk, nsv = heads * d->n_sv;
  int bad = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t hd = 0; hd < heads; ++hd) {
    for (int i = 0; i < nb; ++i) {
      int32_t mk = map_k[hd * nb + i], mv = map_v[hd * nb + i];
      uint16_t *Kb = Kt + hd * (int64_t)d->L * D + (int64_t)i * BD;
      uint16_t *Vb = Vt + hd * (int64_t)d->L * D + (int64_t)i * BD;
      memset(Kb, 0, sizeof(uint16_t) * BD);
      memset(Vb, 0, sizeof(uint16_t) * BD);
      visible[hd * nb + i] = (uint8_t)(mk != 0);
      if ((mk == 0) != (mv == 0)) { bad = 1; continue; }
      if (mk > 0) {
        if (mk > ndk) { bad = 1; continue; }
        memcpy(Kb, k_dense + (int64_t)(mk - 1) * BD, sizeof(uint16_t) * BD);
      } else if (mk < 0) {
        int64_t s = -(int64_t)mk - 1;
        if (s >= nsk) { bad = 1; continue; }
        for (int t = 0; t < B; ++t)
          for (int g = 0; g < D / 4; ++g) {
            uint16_t w = k_meta[s * BD / 16 + (int64_t)t * D / 16 + g / 4];
            int nib = (w >> (4 * (g % 4))) & 0xF;
            Kb[(int64_t)t * D + 4 * g + (nib & 3)] = k_nnz[s * BD / 2 + (int64_t)t * D / 2 + 2 * g];
            Kb[(int64_t)t * D + 4 * g + (nib >> 2)] =
                k_nnz[s * BD / 2 + (int64_t)t * D / 2 + 2 * g + 1];
          }
      }
      if (mv > 0) {
        if (mv > ndv) { bad = 1; continue; }
        for (int c = 0; c < D; ++c)
          for (int t = 0; t < B; ++t)
            Vb[(int64_t)t * D + c] = v_dense[(int64_t)(mv - 1) * BD + (int64_t)c * B + t];
      } else if (mv < 0) {
        int64_t s = -(int64_t)mv - 1;
        if (s >= nsv) { bad = 1; continue; }
        for (int c = 0; c < D; ++c)
          for (int g = 0; g < B / 4; ++g) {
            uint16_t w = v_meta[s * BD / 16 + (int64_t)c * B / 16 + g / 4];
            int nib = (w >> (4 * (g % 4))) & 0xF;
            Vb[(int64_t)(4 * g + (nib & 3)) * D + c] = v_nnz[s * BD / 2 + (int64_t)c * B / 2 + 2 * g];
            Vb[(int64_t)(4 * g + (nib >> 2)) * D + c] =
                v_nnz[s * BD / 2 + (int64_t)c * B / 2 + 2 * g + 1];
          }
      }
    }
  }
  return bad ? HSO_ERR_MAP : HSO_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* Attention: [HS] Eq. (1) over the visible tokens (R6-R8).                                    */

/*
 * hso_attention: o = softmax(q K^T * scale) V over the visible tokens of one query row, in fp64
 * from the exact bf16 values, for the rows listed in 'rows' (flat indices into [b][hq][Lq]; all
 * rows when rows == NULL). causal = 0: every visible token t < L (decode, Lq = 1 in practice);
 * causal = 1: visible t <= query position (prefill, Lq must equal L).
 * Q [b][hq][Lq][D]; Kt, Vt [b][hkv][L][D] bf16 bits; visible [b][hkv][L/B].
 * O [nrows][D] fp64; lse [nrows] = max + ln(sum of exp(s - max)), -inf for an empty row.
 * scale <= 0 selects 1/sqrt(D).
 */
int hso_attention(int b, int hq, int hkv, int L, int D, int B, int Lq, int causal, int dtype,
                  const uint16_t *Q, const uint16_t *Kt, const uint16_t *Vt,
                  const uint8_t *visible, double scale, int64_t nrows, const int64_t *rows,
                  double *O, double *lse) {
  if (b <= 0 || hq <= 0 || hkv <= 0 || L <= 0 || D <= 0 || B <= 0 || Lq <= 0) return HSO_ERR_SHAPE;
  if (hq % hkv || L % B || (causal && Lq != L)) return HSO_ERR_SHAPE;
  const int G = hq / hkv, nb = L / B;
  const int64_t total = (int64_t)b * hq * Lq;
  if (!rows) nrows = total;
  if (scale <= 0) scale = 1.0 / sqrt((double)D);
  for (int64_t r = 0; r < nrows; ++r)
    if (rows && (rows[r] < 0 || rows[r] >= total)) return HSO_ERR_SHAPE;

#pragma omp parallel
  {
    double *s = (double *)malloc(sizeof(double) * L);
    double *q = (double *)malloc(sizeof(double) * D);
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < nrows; ++r) {
      int64_t id = rows ? rows[r] : r;
      int bi = (int)(id / ((int64_t)hq * Lq)), hi = (int)((id / Lq) % hq), qi = (int)(id % Lq);
      int64_t kvh = (int64_t)bi * hkv + hi / G;
      const uint16_t *Kh = Kt + kvh * (int64_t)L * D, *Vh = Vt + kvh * (int64_t)L * D;
      const uint8_t *vis = visible + kvh * nb;
      for (int c = 0; c < D; ++c) q[c] = value(Q[id * D + c], dtype);
      int last = causal ? qi : L - 1;
      double m = -INFINITY;
      for (int t = 0; t <= last; ++t) {
        if (!vis[t / B]) continue;
        double acc = 0;
        for (int c = 0; c < D; ++c) acc += q[c] * value(Kh[(int64_t)t * D + c], dtype);
        s[t] = acc * scale;
        if (s[t] > m) m = s[t];
      }
      double *o = O + r * D;
      for (int c = 0; c < D; ++c) o[c] = 0;
      if (m == -INFINITY) { lse[r] = -INFINITY; continue; }
      double l = 0;
      for (int t = 0; t <= last; ++t) {
        if (!vis[t / B]) continue;
        double w = exp(s[t] - m);
        l += w;
        for (int c = 0; c < D; ++c) o[c] += w * value(Vh[(int64_t)t * D + c], dtype);
      }
      for (int c = 0; c < D; ++c) o[c] /= l;
      lse[r] = m + log(l);
    }
    free(s);
    free(q);
  }
  return HSO_OK;
}
