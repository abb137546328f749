// hs_decode.hip -- split-KV GQA decode attention over the compressed cache (gfx950).
//
// "HieraSparse" (arXiv 2604.16864v2) §II Eq. (1), §III-C1 Table II "Trans-Both", §III-C2 mixed
// dense / sparse dispatch, §IV-C split-KV decode + log-sum-exp combine + GQA packing.
//
// k_decode_split: one wave per (split, KV head, column group, batch entry). The query heads that
//   share the KV head form the 16 columns of the matrix-core tiles ("a short duplicated sequence";
//   unused columns are zero). The split walks its share of the head's visible blocks in 64-token
//   tiles, streaming only the bytes of each block's representation straight into registers:
//     S^T = K Q^T   dense block: 16 v_mfma_f32_16x16x32_bf16; 2:4 block: 8 v_smfmac_f32_16x16x64_bf16
//     online softmax per query column (exp2 domain), P^T packed to bf16 in place
//     O^T += V^T P^T dense block: 16 MFMA over the channel-major copy; 2:4 block: 8 SMFMAC
//   Pruned blocks are never touched. Splits are balanced by visible blocks, not raw block ranges.
//   Output: per split, normalised partial o (fp32) and its log-sum-exp.
// k_decode_combine: one workgroup per (batch entry, query head) merges the splits by their
//   log-sum-exp and writes o (bf16) and lse.
#include "hs_device.h"
#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kD = 128;

struct DecodeArgs {
  CacheView c;
  const uint16_t *q;
  float *part_o, *part_lse;
  int nb, nvis, hkv, hq, G, splits;
  float scale_log2;
};

template <int B>
__global__ __launch_bounds__(64) void k_decode_split(DecodeArgs a) {
  const int lane = threadIdx.x, col = lane & 15, g = lane >> 4;
  const int split = blockIdx.x, hkv = a.hkv;
  const int h = blockIdx.y % hkv, cg = blockIdx.y / hkv, bi = blockIdx.z;
  const int head = bi * hkv + h;
  const int hq0 = h * a.G + 16 * cg, ncol = min(16, a.G - 16 * cg);
  const bool live = col < ncol;

  // Query registers: B operand of GEMM1, k-step s covers channels 32s .. 32s+31.
  uint4 qr[4];
  {
    const uint16_t *qp = a.q + ((size_t)bi * a.hq + hq0 + (live ? col : 0)) * kD + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qr[s] = live ? *reinterpret_cast<const uint4 *>(qp + 32 * s) : make_uint4(0, 0, 0, 0);
  }

  // This split's visible blocks: ranks [lo, hi) among the head's non-pruned blocks.
  const int lo = (int)((int64_t)split * a.nvis / a.splits);
  const int hi = (int)((int64_t)(split + 1) * a.nvis / a.splits);
  const int32_t *mkh = a.c.map_k + (size_t)head * a.nb;
  const int32_t *mvh = a.c.map_v + (size_t)head * a.nb;
  int j = a.nb;
  {
    int seen = 0;
    for (int base = 0; base < a.nb && hi > lo; base += 64) {
      const int jj = base + lane;
      const bool vis = jj < a.nb && mkh[jj] != 0;
      const uint64_t bal = __ballot(vis);
      const int cnt = __popcll(bal);
      if (seen + cnt > lo) {
        const int pre = __popcll(bal & ((1ull << lane) - 1ull));
        const uint64_t hit = __ballot(vis && pre == lo - seen);
        j = base + __ffsll((unsigned long long)hit) - 1;
        break;
      }
      seen += cnt;
    }
  }

  f32x4 oacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int todo = hi - lo; todo > 0 && j < a.nb; ++j) {
    const int mk = mkh[j];
    if (mk == 0) continue;
    --todo;
    const int mv = mvh[j];
#pragma unroll
    for (int tile = 0; tile < B / 64; ++tile) {
      // ---- issue this tile's K and V loads ----
      uint4 ka[16], va[16];
      uint32_t kix[8], vix[8];
      if (mk > 0) {
        const uint16_t *kb = a.c.k_dense + ((size_t)(mk - 1) * B + 64 * tile) * kD + 8 * g;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int s = 0; s < 4; ++s)
            ka[4 * t + s] =
                *reinterpret_cast<const uint4 *>(kb + (size_t)tile_token(t, col) * kD + 32 * s);
      } else {
        const size_t sb = (size_t)(-mk - 1) * B + 64 * tile;
        const uint16_t *nb_ = a.c.k_nnz + sb * (kD / 2) + 8 * g;
        const uint16_t *mb = a.c.k_meta + sb * (kD / 16) + g;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int tok = tile_token(t, col);
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            ka[2 * t + c] = *reinterpret_cast<const uint4 *>(nb_ + (size_t)tok * (kD / 2) + 32 * c);
            kix[2 * t + c] = mb[(size_t)tok * (kD / 16) + 4 * c];
          }
        }
      }
      if (mv > 0) {
        const uint16_t *vb = a.c.v_dense + (size_t)(mv - 1) * B * kD + 64 * tile + 8 * g;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
          for (int m = 0; m < 2; ++m)
            va[2 * ct + m] =
                *reinterpret_cast<const uint4 *>(vb + (size_t)(16 * ct + col) * B + 32 * m);
      } else {
        const size_t sb = (size_t)(-mv - 1) * B * kD;
        const uint16_t *nb_ = a.c.v_nnz + sb / 2 + 32 * tile + 8 * g;
        const uint16_t *mb = a.c.v_meta + sb / 16 + 4 * tile + g;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          va[ct] = *reinterpret_cast<const uint4 *>(nb_ + (size_t)(16 * ct + col) * (B / 2));
          vix[ct] = mb[(size_t)(16 * ct + col) * (B / 16)];
        }
      }

      // ---- S^T = K Q^T ----
      f32x4 sacc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (mk > 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int s = 0; s < 4; ++s) sacc[t] = mfma16(ka[4 * t + s], qr[s], sacc[t]);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int c = 0; c < 2; ++c)
            sacc[t] = smfmac16(ka[2 * t + c], qr[2 * c], qr[2 * c + 1], kix[2 * t + c], sacc[t]);
      }

      // ---- online softmax over this tile's 64 tokens, per query column ----
      float mt = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sacc[t][i] *= a.scale_log2;
          mt = fmaxf(mt, sacc[t][i]);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float m_new = fmaxf(m_run, mt);
      const float alpha = exp2f(m_run - m_new);
      m_run = m_new;
      float psum = 0.f;
      uint32_t pp[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float p0 = exp2f(sacc[t][0] - m_new), p1 = exp2f(sacc[t][1] - m_new);
        float p2 = exp2f(sacc[t][2] - m_new), p3 = exp2f(sacc[t][3] - m_new);
        psum += (p0 + p1) + (p2 + p3);
        pp[2 * t] = pack_bf16x2(p0, p1);
        pp[2 * t + 1] = pack_bf16x2(p2, p3);
      }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) oacc[ct] *= alpha;
      const uint4 plo = make_uint4(pp[0], pp[1], pp[2], pp[3]);  // tokens 8g .. 8g+7
      const uint4 phi = make_uint4(pp[4], pp[5], pp[6], pp[7]);  // tokens 32+8g .. 32+8g+7

      // ---- O^T += V^T P^T ----
      if (mv > 0) {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          oacc[ct] = mfma16(va[2 * ct], plo, oacc[ct]);
          oacc[ct] = mfma16(va[2 * ct + 1], phi, oacc[ct]);
        }
      } else {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) oacc[ct] = smfmac16(va[ct], plo, phi, vix[ct], oacc[ct]);
      }
    }
  }

  // ---- normalised partial output and log-sum-exp of this split ----
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (!live) return;
  const size_t row = ((size_t)bi * a.hq + hq0 + col) * a.splits + split;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  float *po = a.part_o + row * kD + 4 * g;
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
    *reinterpret_cast<float4 *>(po + 16 * ct) =
        make_float4(oacc[ct][0] * inv, oacc[ct][1] * inv, oacc[ct][2] * inv, oacc[ct][3] * inv);
  if (g == 0) a.part_lse[row] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
}

__global__ __launch_bounds__(128) void k_decode_combine(const float *__restrict__ part_o,
                                                        const float *__restrict__ part_lse,
                                                        int splits, uint16_t *__restrict__ o,
                                                        float *__restrict__ lse) {
  const size_t row = blockIdx.x;
  const int d = threadIdx.x;
  const float *pl = part_lse + row * splits;
  float mx = -INFINITY;
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, pl[s]);
  float acc = 0.f, wsum = 0.f;
  if (mx != -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      const float w = pl[s] == -INFINITY ? 0.f : __expf(pl[s] - mx);
      wsum += w;
      acc += w * part_o[(row * splits + s) * kD + d];
    }
  }
  const float out = wsum > 0.f ? acc / wsum : 0.f;
  o[row * kD + d] = __builtin_bit_cast(uint16_t, (__bf16)out);
  if (lse && d == 0) lse[row] = wsum > 0.f ? mx + __logf(wsum) : -INFINITY;
}

}  // namespace

hipError_t launch_decode(const Dims &d, const CacheView &c, const uint16_t *q, uint16_t *o,
                         float *lse, float scale_log2, int splits, float *part_o, float *part_lse,
                         hipStream_t stream) {
  DecodeArgs a{c, q, part_o, part_lse, d.nb, d.nb - d.np, d.hkv, d.hq, d.G, splits, scale_log2};
  const int col_groups = (d.G + 15) / 16;
  const dim3 grid(splits, d.hkv * col_groups, d.b);
  if (d.B == 64)
    k_decode_split<64><<<grid, 64, 0, stream>>>(a);
  else
    k_decode_split<128><<<grid, 64, 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_decode_combine<<<d.b * d.hq, 128, 0, stream>>>(part_o, part_lse, splits, o, lse);
  return hipGetLastError();
}

}  // namespace hs
