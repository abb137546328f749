// hs_prefill.hip -- causal tiled prefill attention over the compressed cache (gfx950).
//
// "HieraSparse" (arXiv 2604.16864v2) §III-C1 Algorithm 1 (S^T = K Q^T, online softmax, P^T
// re-layout, O^T += V^T P^T), §III-C2 mixed dense / sparse dispatch through the index map,
// §IV-C1 asynchronous K/V staging, §IV-C2 in-fragment re-layout, §IV-C3 dense and sparse buffers
// aliased in on-chip memory. Made causal; pruned blocks are skipped without any load.
//
// Work decomposition: one workgroup = 8 waves (two per SIMD, one workgroup per CU). Each wave
// owns one (query head, 32-query tile) task; a workgroup's eight tasks share one KV head (for GQA
// group size 4: the four query heads of that KV head at two adjacent 32-query tiles), so every K/V
// tile the workgroup stages serves 256 queries. Query tiles are issued longest-first and the
// workgroups of one KV head run on one XCD. Two waves per SIMD let one wave's matrix-core work
// overlap the other's softmax.
//
// Per visible 64-token KV tile n (matrix-core shapes 32x32: v_mfma_f32_32x32x16_bf16 for dense,
// v_smfmac_f32_32x32x32_bf16 for 2:4 operands; all accumulators in VGPRs):
//   staging   four 32 KB LDS stages filled by direct global->LDS loads (global_load_lds_dwordx4)
//             two tiles ahead; one barrier per tile. A stage holds the tile's K and V^T exactly in
//             their stored representation (dense copy, or kept values + metadata).
//   GEMM1     S^T[64 tok][32 q] = K Q^T (Q stays in registers as the B operand).
//   softmax   causal mask, column-wise running max (exp2 domain, lazy rescale) and
//             P^T = exp2(S^T - max) packed to bf16 in registers.
//   GEMM2     O^T[128 ch][32 q] += V^T P^T, for tile n-1, interleaved with the softmax of tile n.
// Token order: GEMM1's A operand rows are the tile's tokens in the order tau (bits 2 and 3 of the
// row index exchanged). The 32x32 accumulator then holds, in lane half h, tokens 8h..8h+7 and
// 16+8h..16+8h+7 of each 32-token half in consecutive registers, which is exactly GEMM2's B operand
// layout (lane half h, k = 8h + e): P^T needs no data movement between lanes.
// 2:4 tiles go to SMFMAC, or (decompress variant) are expanded in registers from the same LDS
// stage into dense MFMA operands.
#include "hs_device.h"
#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kD = 128;
constexpr int kTile = 64;                                 // KV tokens per tile
constexpr int kQTile = 32;                                // queries per wave
constexpr int kWaves = 8;
constexpr int kStages = 4;
constexpr int kStageBytes = 32 * 1024;                    // K region 16 KB + V region 16 KB
constexpr int kVRegion = 16 * 1024;
constexpr int kMetaOff = 8 * 1024;                        // metadata of a 2:4 K or V tile
constexpr int kMapOff = kStages * kStageBytes;            // per-block local slots, int16
constexpr int kLdsBytes = kMapOff + 2 * kMaxBlocks * 2;   // 144 KB
constexpr float kTau = 8.0f;                              // lazy-rescale threshold (log2 units)

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---- LDS swizzles (16-byte chunk index XOR a function of the row) ------------------------------
// Every 16-lane group of an operand read touches 16 rows at one logical chunk; the functions below
// make the physical chunks distinct within every 8 and every 16 consecutive lanes.
__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }
__device__ __forceinline__ int fv(int x) { return (x & 7) ^ ((x >> 3) & 1); }   // 128-byte rows
__device__ __forceinline__ int gv(int x) { return ((x >> 1) ^ (x >> 2)) & 3; }  // 64-byte rows

// ---- direct global -> LDS loads -----------------------------------------------------------------
// Lane i of the wave writes LDS[lds_addr + size * i]; the global address is gbase + voff (per lane).
// Issued through inline assembly so the compiler does not serialise them with its own wait
// insertion; completion is tracked with explicit vmcnt waits before the per-tile barrier.
__device__ __forceinline__ void dma16(const void *gbase, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(gbase), "s"(lds_addr)
      : "memory");
}
__device__ __forceinline__ void dma4(const void *gbase, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(gbase), "s"(lds_addr)
      : "memory");
}
// Wait until at most n of this wave's vector-memory operations are outstanding (n in 0..4).
__device__ __forceinline__ void wait_vmem(int n) {
  switch (n) {
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ const char *uniform_ptr(const void *p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char *)(((uint64_t)hi << 32) | lo);
}

// ---- matrix-core helpers -----------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 smfmac32(bf16x8 a, bf16x16 b, uint32_t idx, f32x16 c) {
  return __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a, b, c, (int)idx, 0, 0);
}
// Half k of a 32-deep B operand pair: the B operand of one 16-deep dense step.
__device__ __forceinline__ bf16x8 half8(bf16x16 v, int k2) {
  return k2 ? __builtin_shufflevector(v, v, 8, 9, 10, 11, 12, 13, 14, 15)
            : __builtin_shufflevector(v, v, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ uint4 lds16(const char *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ uint2 lds8(const char *p) { return *reinterpret_cast<const uint2 *>(p); }

// Two packed 2:4 groups (4 kept values as two dwords, 8 metadata bits) -> 8 dense values.
__device__ __forceinline__ bf16x8 expand2(uint2 v, uint32_t bits) {
  const uint2 g0 = expand_group(v.x, bits & 15u), g1 = expand_group(v.y, (bits >> 4) & 15u);
  return as_bf16x8(make_uint4(g0.x, g0.y, g1.x, g1.y));
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
struct WaveState {
  bf16x16 qv[4];    // Q^T as GEMM1 B operand, per 32 channels (two 16-channel dense k-steps)
  f32x16 o[4];      // O^T, per 32-channel tile
  f32x16 s[2];      // S^T of the current tile, per 32-token half
  bf16x16 p[2];     // P^T per 32 tokens (two 16-token dense k-steps): previous tile until
                    // overwritten by the current one
  float m_run, l_run, m_use, alpha;
};

// ---- GEMM1: S^T = K Q^T for one staged tile ---------------------------------------------------
template <bool kSparseK, bool kSmfmac>
__device__ __forceinline__ void gemm1(WaveState &w, const char *kl, int r, int hf) {
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    f32x16 acc = zero16();
    const int row = 32 * T + swap23(r);
    if (!kSparseK) {
      const char *rp = kl + row * 256;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 k = as_bf16x8(lds16(rp + (((2 * ks + hf) ^ (r & 15)) << 4)));
        acc = mfma32(k, half8(w.qv[ks >> 1], ks & 1), acc);
      }
    } else {
      const char *rp = kl + row * 128;
      const uint4 meta = lds16(kl + kMetaOff + (32 * T + r) * 16);
      const uint32_t mw[4] = {meta.x, meta.y, meta.z, meta.w};
      const int f = fv(r & 15);
      if (kSmfmac) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bf16x8 k = as_bf16x8(lds16(rp + (((2 * u + hf) ^ f) << 4)));
          acc = smfmac32(k, w.qv[u], mw[u] >> (16 * hf), acc);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const uint2 v = lds8(rp + ((ks ^ f) << 4) + 8 * hf);
          const uint32_t bits = (mw[ks >> 1] >> (16 * (ks & 1) + 8 * hf)) & 0xFFu;
          acc = mfma32(expand2(v, bits), half8(w.qv[ks >> 1], ks & 1), acc);
        }
      }
    }
    w.s[T] = acc;
  }
}

// ---- GEMM2: O^T += V^T P^T for one staged tile, P^T of that tile in w.p ------------------------
template <bool kSparseV, bool kSmfmac>
__device__ __forceinline__ void gemm2(WaveState &w, const char *vl, int r, int hf) {
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int ch = 32 * ct + r;
    if (!kSparseV) {
      const char *rp = vl + ch * 128;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 v = as_bf16x8(lds16(rp + (((2 * ks + hf) ^ fv(r & 15)) << 4)));
        w.o[ct] = mfma32(v, half8(w.p[ks >> 1], ks & 1), w.o[ct]);
      }
    } else {
      const char *rp = vl + ch * 64;
      const uint2 meta = lds8(vl + kMetaOff + ch * 8);
      const int g = gv(r);
      if (kSmfmac) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bf16x8 v = as_bf16x8(lds16(rp + (((2 * u + hf) ^ g) << 4)));
          w.o[ct] = smfmac32(v, w.p[u], (u ? meta.y : meta.x) >> (16 * hf), w.o[ct]);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const uint2 v = lds8(rp + ((ks ^ g) << 4) + 8 * hf);
          const uint32_t bits = (((ks >> 1) ? meta.y : meta.x) >> (16 * (ks & 1) + 8 * hf)) & 0xFFu;
          w.o[ct] = mfma32(expand2(v, bits), half8(w.p[ks >> 1], ks & 1), w.o[ct]);
        }
      }
    }
  }
}

// ---- softmax of the current tile: causal mask, running max, decision to rescale ----------------
// 'shift' = (first token of the key tile) - (first query of the wave); a token is masked when
// shift + token > query. Returns true if the running max moves (then w.alpha rescales O and l).
__device__ __forceinline__ bool softmax_max(WaveState &w, bool diag, int shift, int r, int hf,
                                            float c) {
  float mx = -INFINITY;
#pragma unroll
  for (int T = 0; T < 2; ++T)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float x = w.s[T][e];
      if (diag && shift + 32 * T + 16 * (e >> 3) + 8 * hf + (e & 7) > r) x = -INFINITY;
      w.s[T][e] = x;
      mx = fmaxf(mx, x);
    }
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

// P^T of the current tile for GEMM2 k-step ks (tokens 16ks .. 16ks+15): the accumulator
// registers 8*(ks&1) .. +7 of half ks>>1, exponentiated and packed to bf16. The bf16 values are
// also summed (dot product with ones) into the running denominator.
__device__ __forceinline__ void softmax_exp(WaveState &w, int ks, float c, float mc, float &lsum) {
  const f32x16 &s = w.s[ks >> 1];
  const int base = 8 * (ks & 1);
  uint32_t pk[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[base + 2 * e], c, -mc));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[base + 2 * e + 1], c, -mc));
    pk[e] = pack_bf16x2(p0, p1);
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[e]), one, lsum, false);
  }
  const bf16x8 nw = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
  bf16x16 &pp = w.p[ks >> 1];
  pp = (ks & 1) ? __builtin_shufflevector(half8(pp, 0), nw, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11,
                                          12, 13, 14, 15)
                : __builtin_shufflevector(nw, half8(pp, 1), 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11,
                                          12, 13, 14, 15);
}

__device__ __forceinline__ void softmax_finish(WaveState &w, bool need, float lsum) {
  if (need) {
    w.l_run = w.l_run * w.alpha + lsum;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) w.o[ct] *= w.alpha;
    w.m_run = w.m_use;
  } else {
    w.l_run += lsum;
  }
}

// Exponentials of the current tile interleaved with GEMM2 of the previous tile, one 16-token
// k-step at a time (two for SMFMAC): the MFMAs that read P^T[ks] of the previous tile are issued,
// then the same registers receive P^T[ks] of the current tile. Only the V operands of one k-step
// are live at a time.
template <bool kGemm2, bool kSparseV, bool kSmfmac>
__device__ __forceinline__ float exp_and_gemm2(WaveState &w, const char *vl, int r, int hf,
                                               float c) {
  float lsum = 0.f;
  const float mc = w.m_use == -INFINITY ? 0.f : w.m_use;  // rows with nothing visible yet
  if (!kGemm2) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) softmax_exp(w, ks, c, mc, lsum);
  } else if (!kSparseV) {
    const int f = fv(r & 15);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const bf16x8 v = as_bf16x8(lds16(vl + (32 * ct + r) * 128 + (((2 * ks + hf) ^ f) << 4)));
        w.o[ct] = mfma32(v, half8(w.p[ks >> 1], ks & 1), w.o[ct]);
      }
      softmax_exp(w, ks, c, mc, lsum);
    }
  } else {
    uint2 meta[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) meta[ct] = lds8(vl + kMetaOff + (32 * ct + r) * 8);
    const int g = gv(r);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const char *rp = vl + (32 * ct + r) * 64;
        const uint32_t mw = u ? meta[ct].y : meta[ct].x;
        if (kSmfmac) {
          const bf16x8 v = as_bf16x8(lds16(rp + (((2 * u + hf) ^ g) << 4)));
          w.o[ct] = smfmac32(v, w.p[u], mw >> (16 * hf), w.o[ct]);
        } else {
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const int ks = 2 * u + k2;
            const uint2 v = lds8(rp + ((ks ^ g) << 4) + 8 * hf);
            w.o[ct] = mfma32(expand2(v, (mw >> (16 * k2 + 8 * hf)) & 0xFFu), half8(w.p[u], k2),
                             w.o[ct]);
          }
        }
      }
      softmax_exp(w, 2 * u, c, mc, lsum);
      softmax_exp(w, 2 * u + 1, c, mc, lsum);
    }
  }
  return lsum;
}

template <int B, bool kSmfmac>
__global__ __launch_bounds__(512, 1) void k_prefill(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int TPB = B / kTile;  // 64-token tiles per block

  // XCD-aware order: consecutive dispatch slots go round-robin over the 8 XCDs, so logical
  // workgroup index i*(N/8)+x runs on XCD x and one KV head's workgroups share an L2.
  const int n = a.n_wg, full = n & ~7, bid = blockIdx.x;
  const int logical = bid < full ? (bid & 7) * (full >> 3) + (bid >> 3) : bid;
  const int head = logical / a.wg_per_head, wgi = logical % a.wg_per_head;
  const int bi = head / a.hkv, h = head % a.hkv;

  // Tasks (query head in group fastest, 32-query tiles last-first); this wave's task and the
  // workgroup's last key tile.
  const int task = wgi * kWaves + wave;
  const bool has_task = task < a.G * a.nqt;
  const int hq_i = h * a.G + (has_task ? task % a.G : 0);
  const int qt = has_task ? a.nqt - 1 - task / a.G : 0;
  const int qt_max = a.nqt - 1 - (wgi * kWaves) / a.G;
  const int kt_max = (kQTile * qt_max + kQTile - 1) / kTile;
  const int nbq = kt_max / TPB + 1;  // blocks touched by this workgroup

  // Block modes of this head as local pool slots: +(i+1) dense slot i, -(i+1) 2:4 slot i, 0 pruned.
  int16_t *mk16 = reinterpret_cast<int16_t *>(lds + kMapOff);
  int16_t *mv16 = mk16 + kMaxBlocks;
  {
    const int32_t *mkh = a.c.map_k + (size_t)head * a.nb, *mvh = a.c.map_v + (size_t)head * a.nb;
    for (int i = tid; i < nbq; i += kWaves * 64) {
      const int mk = mkh[i], mv = mvh[i];
      mk16[i] = (int16_t)(mk > 0 ? mk - head * a.ndk : (mk < 0 ? mk + head * a.nsk : 0));
      mv16[i] = (int16_t)(mv > 0 ? mv - head * a.ndv : (mv < 0 ? mv + head * a.nsv : 0));
    }
  }

  WaveState w;
  {
    const uint16_t *qp =
        a.q + (((size_t)bi * a.hq + hq_i) * a.L + (size_t)kQTile * qt + r) * kD + 8 * hf;
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      w.qv[u] = as_bf16x16(has_task ? *reinterpret_cast<const uint4 *>(qp + 32 * u) : z,
                           has_task ? *reinterpret_cast<const uint4 *>(qp + 32 * u + 16) : z);
  }
  // Retire the Q loads here with a wait the compiler sees, so it never re-waits on them inside
  // the loop (where its vmcnt count would also drain the in-flight K/V prefetch).
  __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) w.o[ct] = zero16();
  w.m_run = -INFINITY;
  w.l_run = 0.f;

  const uint32_t lds_base = (uint32_t)(size_t)(__attribute__((address_space(3))) char *)lds;

  __syncthreads();  // block modes visible

  auto next_visible = [&](int kt) {
    while (kt <= kt_max && mk16[kt / TPB] == 0) ++kt;
    return kt;
  };
  auto dma_count = [&](int kt) {
    const int blk = kt / TPB;
    return (mk16[blk] > 0 ? 2 : 1 + (wave < 4)) + (mv16[blk] > 0 ? 2 : 1 + (wave >= 4));
  };
  // Direct loads of one tile into a stage. Instruction q of a region writes LDS bytes
  // 1024*q .. +1023 (lane i: bytes 16*i .. +15); metadata goes as 256-byte dword loads (lane i:
  // bytes 4*i .. +3), K metadata by waves 0-3 and V metadata by waves 4-7. The per-lane global
  // byte offsets implement the LDS swizzles; they are recomputed here rather than kept live.
  auto issue = [&](int kt, int stage) {
    const int blk = kt / TPB, half = kt % TPB;
    const int mk = __builtin_amdgcn_readfirstlane(mk16[blk]);
    const int mv = __builtin_amdgcn_readfirstlane(mv16[blk]);
    const uint32_t kl = lds_base + stage * kStageBytes, vl = kl + kVRegion;
    int ln = lane;
    asm volatile("" : "+v"(ln));  // keep the offset arithmetic here instead of hoisted and spilled
    const int p1 = 64 * wave + ln;     // slot of a single-instruction region
    const int dm = 64 * (wave & 3) + ln;  // dword slot of a metadata region
    if (mk > 0) {
      const char *g = uniform_ptr(
          a.c.k_dense + ((size_t)(head * a.ndk + mk - 1) * B + kTile * half) * kD);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int p = 64 * (2 * wave + m) + ln, row = p >> 4;
        dma16(g, row * 256 + (((p & 15) ^ swap23(row & 15)) << 4), kl + 1024 * (2 * wave + m));
      }
    } else {
      const size_t row0 = (size_t)(head * a.nsk - mk - 1) * B + kTile * half;
      const int t = p1 >> 3;
      dma16(uniform_ptr(a.c.k_nnz + row0 * (kD / 2)),
            t * 128 + (((p1 & 7) ^ fv(swap23(t & 15))) << 4), kl + 1024 * wave);
      if (wave < 4) {
        const int sl = dm >> 2, tok = (sl & ~15) | swap23(sl & 15);
        dma4(uniform_ptr(a.c.k_meta + row0 * (kD / 16)), tok * 16 + (dm & 3) * 4,
             kl + kMetaOff + 256 * wave);
      }
    }
    if (mv > 0) {
      const char *g = uniform_ptr(a.c.v_dense + (size_t)(head * a.ndv + mv - 1) * B * kD +
                                  kTile * half);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int p = 64 * (2 * wave + m) + ln, ch = p >> 3;
        dma16(g, ch * (2 * B) + (((p & 7) ^ fv(ch & 15)) << 4), vl + 1024 * (2 * wave + m));
      }
    } else {
      const size_t blk0 = (size_t)(head * a.nsv - mv - 1) * B * kD;
      const int ch = p1 >> 2;
      dma16(uniform_ptr(a.c.v_nnz + blk0 / 2 + (kTile / 2) * half),
            ch * B + (((p1 & 3) ^ gv(ch)) << 4), vl + 1024 * wave);
      if (wave >= 4)
        dma4(uniform_ptr(a.c.v_meta + blk0 / 16 + (kTile / 16) * half),
             (dm >> 1) * (B / 8) + (dm & 1) * 4, vl + kMetaOff + 256 * (wave - 4));
    }
  };

  const float c = a.scale_log2;
  int kt0 = next_visible(0);
  int kt1 = kt0 <= kt_max ? next_visible(kt0 + 1) : kt_max + 1;
  if (kt0 <= kt_max) issue(kt0, 0);
  if (kt1 <= kt_max) issue(kt1, 1);

  // Every wave walks every tile the workgroup stages (uniform control flow); tiles beyond a wave's
  // own queries are fully masked by the causal test and contribute nothing.
  bool prev_sparse_v = false;
  const char *vl_prev = lds;
  int it = 0;
  while (kt0 <= kt_max) {
    const int kt2 = kt1 <= kt_max ? next_visible(kt1 + 1) : kt_max + 1;
    wait_vmem(kt1 <= kt_max ? dma_count(kt1) : 0);
    barrier();  // tile kt0 staged by every wave; stage (it + 2) % 4 no longer read
    if (kt2 <= kt_max) issue(kt2, (it + 2) & 3);

    const char *kl = lds + (it & 3) * kStageBytes, *vl = kl + kVRegion;
    const int blk = kt0 / TPB;
    const bool sparse_k = mk16[blk] < 0, sparse_v = mv16[blk] < 0;
    if (sparse_k)
      gemm1<true, kSmfmac>(w, kl, r, hf);
    else
      gemm1<false, kSmfmac>(w, kl, r, hf);
    const int shift = kTile * kt0 - kQTile * qt;
    const bool need = softmax_max(w, shift > -kTile, shift, r, hf, c);
    float lsum;
    if (it == 0)
      lsum = exp_and_gemm2<false, false, kSmfmac>(w, vl_prev, r, hf, c);
    else if (prev_sparse_v)
      lsum = exp_and_gemm2<true, true, kSmfmac>(w, vl_prev, r, hf, c);
    else
      lsum = exp_and_gemm2<true, false, kSmfmac>(w, vl_prev, r, hf, c);
    softmax_finish(w, need, lsum);
    prev_sparse_v = sparse_v;
    vl_prev = vl;
    kt0 = kt1;
    kt1 = kt2;
    ++it;
  }
  if (it > 0) {  // GEMM2 of the last tile (its stage is not overwritten after the loop)
    if (prev_sparse_v)
      gemm2<true, kSmfmac>(w, vl_prev, r, hf);
    else
      gemm2<false, kSmfmac>(w, vl_prev, r, hf);
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
      const uint2 v = make_uint2(pack_bf16x2(acc[4 * j] * inv, acc[4 * j + 1] * inv),
                                 pack_bf16x2(acc[4 * j + 2] * inv, acc[4 * j + 3] * inv));
      *reinterpret_cast<uint2 *>(op + 32 * ct + 8 * j) = v;
    }
  if (a.lse && hf == 0) a.lse[qrow] = l > 0.f ? (w.m_run + log2f(l)) * kLn2 : -INFINITY;
}

template <int B>
hipError_t launch_b(const PrefillArgs &a, bool smfmac, hipStream_t stream) {
  if (smfmac)
    k_prefill<B, true><<<a.n_wg, kWaves * 64, 0, stream>>>(a);
  else
    k_prefill<B, false><<<a.n_wg, kWaves * 64, 0, stream>>>(a);
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
  a.nqt = d.L / kQTile;
  a.wg_per_head = (d.G * a.nqt + kWaves - 1) / kWaves;
  a.n_wg = d.b * d.hkv * a.wg_per_head;
  a.ndk = d.ndk;
  a.nsk = d.nsk;
  a.ndv = d.ndv;
  a.nsv = d.nsv;
  a.scale_log2 = scale_log2;
  return d.B == 64 ? launch_b<64>(a, smfmac, stream) : launch_b<128>(a, smfmac, stream);
}

}  // namespace hs
