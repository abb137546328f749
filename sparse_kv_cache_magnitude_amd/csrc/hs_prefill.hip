// hs_prefill.hip -- causal tiled prefill attention over the compressed cache (gfx950).
//
// "HieraSparse" (arXiv 2604.16864v2) §III-C1 Algorithm 1 (S^T = K Q^T, online softmax, P^T
// re-layout, O^T += V^T P^T), §III-C2 mixed dense / sparse dispatch through the index map,
// §IV-C1 double-buffered K/V staging, §IV-C2 in-fragment re-layout, §IV-C3 dense and sparse
// buffers aliased in on-chip memory. Made causal; pruned blocks are skipped without any load.
//
// Work decomposition (one workgroup = 4 waves = 256 threads, one wave per SIMD):
//   Each wave owns one (query head, 64-query tile) "task". A workgroup's four tasks share one KV
//   head: for GQA group size G the tasks are consecutive (head-in-group, query tile) pairs with
//   the head index fastest, so with G = 4 the four query heads of a KV head share every K/V tile
//   the workgroup stages (the paper's GQA packing applied to prefill). Query tiles are handed out
//   last-first (the longest causal rows start first), and workgroups of one KV head are mapped to
//   one XCD so its K/V stream stays in that XCD's L2.
//   Per 64-token KV tile: the workgroup stages the tile's K and V^T into LDS (dense copy, or the
//   2:4 values + metadata, or -- in the decompress variant -- the 2:4 tile expanded to dense), then
//   every wave runs
//     S^T[64 tok][64 q]  = K Q^T     16 dense MFMA per 16x16 output block column, or 8 SMFMAC
//     causal mask on the diagonal tile, online softmax per query column (exp2 domain)
//     O^T[128 ch][64 q] += V^T P^T   with P^T taken straight from the GEMM1 accumulators
//   while the next tile's global loads are in flight.
// Operand layouts: hs_device.h. Q stays in registers for the whole KV loop.
#include "hs_device.h"
#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kD = 128;
constexpr int kTile = 64;               // tokens per KV tile and queries per task
constexpr int kBufBytes = 32 * 1024;    // one stage: K region 16 KB + V region 16 KB
constexpr int kVOff = 16 * 1024;
constexpr float kTau = 8.0f;            // lazy-rescale threshold (log2 units)

__device__ __forceinline__ bf16x8 lo8(bf16x16 v) {
  return __builtin_shufflevector(v, v, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 hi8(bf16x16 v) {
  return __builtin_shufflevector(v, v, 8, 9, 10, 11, 12, 13, 14, 15);
}
__device__ __forceinline__ f32x4 mfma16v(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// kHalf selects the index half word (abid): 0 = bits 15:0, 1 = bits 31:16.
template <int kHalf>
__device__ __forceinline__ f32x4 smfmac16v(bf16x8 a, bf16x16 b, uint32_t idx, f32x4 c) {
  return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a, b, c, (int)idx, 0, kHalf);
}

struct PrefillArgs {
  CacheView c;
  const uint16_t *q;
  uint16_t *o;
  float *lse;
  int L, nb, hkv, hq, G, nqt, wg_per_head, n_wg;
  float scale_log2;
};

// ---- LDS addressing (byte offsets inside one stage) ----------------------------------------
// Each 16-lane group of an MFMA operand read touches 16 rows at one 16-byte chunk column; the
// XOR swizzles below spread those rows over distinct bank groups. rho(row) is the row's index
// inside such a 16-lane group: tokens of a K tile are read in tile_token() order, channels of a
// V tile in natural order.
__device__ __forceinline__ int rho_tok(int tok) { return (tok & 3) | (((tok >> 3) & 3) << 2); }
__device__ __forceinline__ int rho_ch(int ch) { return ch & 15; }

// K dense: [64 tok][256 B], 16 chunks per row.
__device__ __forceinline__ int k_dense_off(int tok, int chunk) {
  return tok * 256 + ((chunk ^ rho_tok(tok)) << 4);
}
// 128-byte rows with 8 chunks: K 2:4 values [64 tok][128 B] and V^T dense [128 ch][128 B].
__device__ __forceinline__ int row128_off(int row, int rho, int chunk) {
  const int f = (rho >> 1) ^ ((rho & 1) << 2);
  return row * 128 + (((chunk ^ f) & 7) << 4);
}
// V 2:4 values: [128 ch][64 B], 4 chunks per row.
__device__ __forceinline__ int v_nnz_off(int ch, int chunk) {
  const int rho = rho_ch(ch);
  const int f = ((rho >> 1) ^ (rho >> 2)) & 3;
  return ch * 64 + ((chunk ^ f) << 4);
}
constexpr int kKMetaOff = 8 * 1024;   // K 2:4 metadata: [64 tok][4] dwords (words kc | 4+kc << 16)
constexpr int kVMetaOff = 8 * 1024;   // V 2:4 metadata: [128 ch][4] words, after the V values

__device__ __forceinline__ uint4 lds_read16(const char *base, int off) {
  return *reinterpret_cast<const uint4 *>(base + off);
}
__device__ __forceinline__ void lds_write16(char *base, int off, uint4 v) {
  *reinterpret_cast<uint4 *>(base + off) = v;
}

// Expand four packed groups (8 kept values + one metadata word) to 16 dense slots.
__device__ __forceinline__ void expand4(uint4 v, uint32_t word, uint4 &lo, uint4 &hi) {
  const uint2 g0 = expand_group(v.x, word & 15u), g1 = expand_group(v.y, (word >> 4) & 15u);
  const uint2 g2 = expand_group(v.z, (word >> 8) & 15u), g3 = expand_group(v.w, (word >> 12) & 15u);
  lo = make_uint4(g0.x, g0.y, g1.x, g1.y);
  hi = make_uint4(g2.x, g2.y, g3.x, g3.y);
}

// Global -> register staging of one KV tile (all 256 threads).
struct Stage {
  uint4 k[4], v[4];
  uint32_t km[2], vm[2];
};

template <int B, bool kSmfmac>
__device__ __forceinline__ void stage_load(Stage &st, const CacheView &c, int mk, int mv, int half,
                                           int tid) {
  if (mk > 0) {
    const uint16_t *src = c.k_dense + ((size_t)(mk - 1) * B + kTile * half) * kD;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tid + 256 * j;
      st.k[j] = *reinterpret_cast<const uint4 *>(src + (e >> 4) * kD + 8 * (e & 15));
    }
  } else {
    const size_t row0 = (size_t)(-mk - 1) * B + kTile * half;
    const uint16_t *nnz = c.k_nnz + row0 * (kD / 2), *meta = c.k_meta + row0 * (kD / 16);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = tid + 256 * j;
      st.k[j] = *reinterpret_cast<const uint4 *>(nnz + (e >> 3) * (kD / 2) + 8 * (e & 7));
      if (!kSmfmac) st.km[j] = meta[(e >> 3) * (kD / 16) + (e & 7)];
    }
    if (kSmfmac) {  // item (token, kc): metadata words kc and 4 + kc
      const int tok = tid >> 2, kc = tid & 3;
      st.km[0] = meta[tok * (kD / 16) + kc] | ((uint32_t)meta[tok * (kD / 16) + 4 + kc] << 16);
    }
  }
  if (mv > 0) {
    const uint16_t *src = c.v_dense + (size_t)(mv - 1) * B * kD + kTile * half;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tid + 256 * j;
      st.v[j] = *reinterpret_cast<const uint4 *>(src + (e >> 3) * B + 8 * (e & 7));
    }
  } else {
    const size_t blk = (size_t)(-mv - 1) * B * kD;
    const uint16_t *nnz = c.v_nnz + blk / 2 + (kTile / 2) * half;
    const uint16_t *meta = c.v_meta + blk / 16 + (kTile / 16) * half;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = tid + 256 * j;  // (channel e >> 2, chunk / word e & 3)
      st.v[j] = *reinterpret_cast<const uint4 *>(nnz + (e >> 2) * (B / 2) + 8 * (e & 3));
      st.vm[j] = meta[(e >> 2) * (B / 16) + (e & 3)];
    }
  }
}

template <bool kSmfmac>
__device__ __forceinline__ void stage_store(const Stage &st, char *buf, int mk, int mv, int tid) {
  char *kl = buf, *vl = buf + kVOff;
  if (mk > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tid + 256 * j;
      lds_write16(kl, k_dense_off(e >> 4, e & 15), st.k[j]);
    }
  } else if (kSmfmac) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = tid + 256 * j, tok = e >> 3;
      lds_write16(kl, row128_off(tok, rho_tok(tok), e & 7), st.k[j]);
    }
    *reinterpret_cast<uint32_t *>(kl + kKMetaOff + 4 * tid) = st.km[0];
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = tid + 256 * j, tok = e >> 3, w = e & 7;
      uint4 lo, hi;
      expand4(st.k[j], st.km[j], lo, hi);
      lds_write16(kl, k_dense_off(tok, 2 * w), lo);
      lds_write16(kl, k_dense_off(tok, 2 * w + 1), hi);
    }
  }
  if (mv > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tid + 256 * j, ch = e >> 3;
      lds_write16(vl, row128_off(ch, rho_ch(ch), e & 7), st.v[j]);
    }
  } else if (kSmfmac) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = tid + 256 * j;
      lds_write16(vl, v_nnz_off(e >> 2, e & 3), st.v[j]);
      *reinterpret_cast<uint16_t *>(vl + kVMetaOff + 2 * e) = (uint16_t)st.vm[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = tid + 256 * j, ch = e >> 2, w = e & 3;
      uint4 lo, hi;
      expand4(st.v[j], st.vm[j], lo, hi);
      lds_write16(vl, row128_off(ch, rho_ch(ch), 2 * w), lo);
      lds_write16(vl, row128_off(ch, rho_ch(ch), 2 * w + 1), hi);
    }
  }
}

template <int B, bool kSmfmac>
__global__ __launch_bounds__(256, 1) void k_prefill(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kBufBytes];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, col = lane & 15, kc = lane >> 4;

  // XCD-aware order: consecutive dispatch slots go round-robin over the 8 XCDs, so logical
  // workgroup index i*(N/8)+x runs on XCD x and one KV head's workgroups share an L2.
  const int n = a.n_wg, full = n & ~7, bid = blockIdx.x;
  const int logical = bid < full ? (bid & 7) * (full >> 3) + (bid >> 3) : bid;
  const int head = logical / a.wg_per_head, wgi = logical % a.wg_per_head;
  const int bi = head / a.hkv, h = head % a.hkv;

  const int task = wgi * 4 + wave;
  const bool has_task = task < a.G * a.nqt;
  const int hq_i = h * a.G + (has_task ? task % a.G : 0);
  const int qt = has_task ? a.nqt - 1 - task / a.G : -1;
  const int qt_max = a.nqt - 1 - (wgi * 4) / a.G;

  // Q registers: B operand of GEMM1 for 4 column blocks n (queries 16n + col) and 4 k-steps.
  // qv[n][c]: channels 64c + 8kc .. +7 (slots 0..7) and 64c + 32 + 8kc .. +7 (slots 8..15); the
  // halves are the dense k-steps 2c and 2c + 1.
  bf16x16 qv[4][2];
  {
    const uint16_t *qp =
        a.q + (((size_t)bi * a.hq + hq_i) * a.L + (size_t)kTile * (qt < 0 ? 0 : qt) + col) * kD +
        8 * kc;
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int nn = 0; nn < 4; ++nn)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint16_t *p = qp + (size_t)16 * nn * kD + 64 * c;
        qv[nn][c] = as_bf16x16(has_task ? *reinterpret_cast<const uint4 *>(p) : z,
                               has_task ? *reinterpret_cast<const uint4 *>(p + 32) : z);
      }
  }

  f32x4 oacc[8][4];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int nn = 0; nn < 4; ++nn) oacc[ct][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int nn = 0; nn < 4; ++nn) {
    m_run[nn] = -INFINITY;
    l_run[nn] = 0.f;
  }

  const int32_t *mkh = a.c.map_k + (size_t)head * a.nb;
  const int32_t *mvh = a.c.map_v + (size_t)head * a.nb;
  constexpr int kTilesPerBlock = B / kTile;
  auto next_visible = [&](int kt) {
    while (kt <= qt_max && mkh[kt / kTilesPerBlock] == 0) ++kt;
    return kt;
  };

  Stage st;
  int kt = next_visible(0);
  if (kt <= qt_max)
    stage_load<B, kSmfmac>(st, a.c, mkh[kt / kTilesPerBlock], mvh[kt / kTilesPerBlock],
                           kt % kTilesPerBlock, tid);
  int buf = 0;
  while (kt <= qt_max) {
    const int mk = mkh[kt / kTilesPerBlock], mv = mvh[kt / kTilesPerBlock];
    char *sb = lds + buf * kBufBytes;
    stage_store<kSmfmac>(st, sb, mk, mv, tid);
    __syncthreads();
    const int kn = next_visible(kt + 1);
    if (kn <= qt_max)
      stage_load<B, kSmfmac>(st, a.c, mkh[kn / kTilesPerBlock], mvh[kn / kTilesPerBlock],
                             kn % kTilesPerBlock, tid);

    if (kt <= qt) {
      const char *kl = sb, *vl = sb + kVOff;
      const bool diag = kt == qt;
      bf16x16 pv[4];  // P^T of the whole tile per query block: slots 0..7 = half 0, 8..15 = half 1
      // Two 32-token halves: accumulator tiles t = 2*hh, 2*hh + 1 hold tokens 32*hh + 8*kc + 0..7
      // of each lane, i.e. exactly the B slots 8*hh .. 8*hh + 7 of GEMM2.
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        // ---- S^T = K Q^T for this half ----
        f32x4 sacc[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int nn = 0; nn < 4; ++nn) sacc[t][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (mk > 0 || !kSmfmac) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int tok = tile_token(2 * hh + t, col);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const bf16x8 ka = as_bf16x8(lds_read16(kl, k_dense_off(tok, 4 * s + kc)));
#pragma unroll
              for (int nn = 0; nn < 4; ++nn)
                sacc[t][nn] = mfma16v(ka, (s & 1) ? hi8(qv[nn][s >> 1]) : lo8(qv[nn][s >> 1]),
                                      sacc[t][nn]);
            }
          }
        } else {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int tok = tile_token(2 * hh + t, col);
            const uint32_t idx =
                *reinterpret_cast<const uint32_t *>(kl + kKMetaOff + 4 * (4 * tok + kc));
            const bf16x8 k0 = as_bf16x8(lds_read16(kl, row128_off(tok, rho_tok(tok), kc)));
            const bf16x8 k1 = as_bf16x8(lds_read16(kl, row128_off(tok, rho_tok(tok), 4 + kc)));
#pragma unroll
            for (int nn = 0; nn < 4; ++nn) {
              sacc[t][nn] = smfmac16v<0>(k0, qv[nn][0], idx, sacc[t][nn]);
              sacc[t][nn] = smfmac16v<1>(k1, qv[nn][1], idx, sacc[t][nn]);
            }
          }
        }

        // ---- causal mask, online softmax per query column, P^T in registers ----
#pragma unroll
        for (int nn = 0; nn < 4; ++nn) {
          float mt = -INFINITY;
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float x = sacc[t][nn][i] * a.scale_log2;
              if (diag && tile_token(2 * hh + t, 4 * kc + i) > 16 * nn + col) x = -INFINITY;
              sacc[t][nn][i] = x;
              mt = fmaxf(mt, x);
            }
          mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
          mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
          // Lazy rescale: keep the running max while new scores exceed it by at most 2^kTau
          // (probabilities then stay <= 2^kTau, harmless in fp32 sums and bf16 operands); the
          // final normalisation uses the same max, so the result is unchanged.
          const float m_new = fmaxf(m_run[nn], mt);
          if (__builtin_expect(__any(m_new > m_run[nn] + kTau), 0)) {
            const float alpha = m_run[nn] == -INFINITY ? 0.f : exp2f(m_run[nn] - m_new);
            l_run[nn] *= alpha;
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) oacc[ct][nn] *= alpha;
            m_run[nn] = m_new;
          }
          const float m_use = m_run[nn] == -INFINITY ? 0.f : m_run[nn];
          float psum = 0.f;
          uint32_t pp[4];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const float p0 = exp2f(sacc[t][nn][0] - m_use), p1 = exp2f(sacc[t][nn][1] - m_use);
            const float p2 = exp2f(sacc[t][nn][2] - m_use), p3 = exp2f(sacc[t][nn][3] - m_use);
            psum += (p0 + p1) + (p2 + p3);
            pp[2 * t] = pack_bf16x2(p0, p1);
            pp[2 * t + 1] = pack_bf16x2(p2, p3);
          }
          l_run[nn] += psum;
          const bf16x8 ph = as_bf16x8(make_uint4(pp[0], pp[1], pp[2], pp[3]));
          pv[nn] = hh == 0 ? __builtin_shufflevector(ph, ph, 0, 1, 2, 3, 4, 5, 6, 7, 0, 1, 2, 3, 4,
                                                     5, 6, 7)
                           : __builtin_shufflevector(lo8(pv[nn]), ph, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9,
                                                     10, 11, 12, 13, 14, 15);
        }

        // ---- O^T += V^T P^T: dense V per half, 2:4 V once both halves are in ----
        if (mv > 0 || !kSmfmac) {
#pragma unroll
          for (int ct = 0; ct < 8; ++ct) {
            const int ch = 16 * ct + col;
            const bf16x8 v = as_bf16x8(lds_read16(vl, row128_off(ch, rho_ch(ch), 4 * hh + kc)));
#pragma unroll
            for (int nn = 0; nn < 4; ++nn)
              oacc[ct][nn] = mfma16v(v, hh ? hi8(pv[nn]) : lo8(pv[nn]), oacc[ct][nn]);
          }
        } else if (hh == 1) {
#pragma unroll
          for (int ct = 0; ct < 8; ++ct) {
            const int ch = 16 * ct + col;
            const bf16x8 v = as_bf16x8(lds_read16(vl, v_nnz_off(ch, kc)));
            const uint32_t idx =
                *reinterpret_cast<const uint16_t *>(vl + kVMetaOff + 2 * (4 * ch + kc));
#pragma unroll
            for (int nn = 0; nn < 4; ++nn) oacc[ct][nn] = smfmac16v<0>(v, pv[nn], idx, oacc[ct][nn]);
          }
        }
      }
    }
    buf ^= 1;
    kt = kn;
  }

  if (!has_task) return;
  // ---- O = O^T / l, log-sum-exp ----
#pragma unroll
  for (int nn = 0; nn < 4; ++nn) {
    float l = l_run[nn];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const size_t qrow = ((size_t)bi * a.hq + hq_i) * a.L + (size_t)kTile * qt + 16 * nn + col;
    uint16_t *op = a.o + qrow * kD + 4 * kc;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const uint2 w = make_uint2(pack_bf16x2(oacc[ct][nn][0] * inv, oacc[ct][nn][1] * inv),
                                 pack_bf16x2(oacc[ct][nn][2] * inv, oacc[ct][nn][3] * inv));
      *reinterpret_cast<uint2 *>(op + 16 * ct) = w;
    }
    if (a.lse && kc == 0) a.lse[qrow] = l > 0.f ? (m_run[nn] + log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int B>
hipError_t launch_b(const PrefillArgs &a, bool smfmac, hipStream_t stream) {
  if (smfmac)
    k_prefill<B, true><<<a.n_wg, 256, 0, stream>>>(a);
  else
    k_prefill<B, false><<<a.n_wg, 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const Dims &d, const CacheView &c, const uint16_t *q, uint16_t *o,
                          float *lse, float scale_log2, bool smfmac, hipStream_t stream) {
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
  a.nqt = d.L / kTile;
  a.wg_per_head = (d.G * a.nqt + 3) / 4;
  a.n_wg = d.b * d.hkv * a.wg_per_head;
  a.scale_log2 = scale_log2;
  return d.B == 64 ? launch_b<64>(a, smfmac, stream) : launch_b<128>(a, smfmac, stream);
}

}  // namespace hs
