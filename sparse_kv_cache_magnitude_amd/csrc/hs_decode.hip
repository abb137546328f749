// hs_decode.hip -- split-KV GQA decode attention over the compressed cache (gfx950).
//
// "HieraSparse" (arXiv 2604.16864v2) §II Eq. (1), §III-C1 Table II "Trans-Both", §III-C2 mixed
// dense / sparse dispatch, §IV-C split-KV decode + log-sum-exp combine + GQA packing.
//
// k_decode_split: one wave per workgroup, one workgroup per (split, KV head, column group, batch
//   entry); two workgroups share a CU. The query heads that share the KV head form the 16 columns
//   of the matrix-core tiles ("a short duplicated sequence"; unused columns are zero). A split owns
//   a run of the head's visible blocks, balanced by bytes (pruned blocks cost nothing).
//   The blocks' representations stream through two LDS stages by direct global->LDS loads
//   (global_load_lds_dwordx4: whole 1 KB requests, no register staging), one 64-token tile ahead of
//   the tile being computed. Every byte is read once, so the loads carry the nontemporal cache
//   policy (measured about 10% faster than the default policy on the 32K and 128K workloads):
//     S^T = K Q^T   dense block: 16 v_mfma_f32_16x16x32_bf16; 2:4 block: 8 v_smfmac_f32_16x16x64_bf16
//     online softmax per query column (exp2 domain), P^T packed to bf16 in place
//     O^T += V^T P^T dense block: 16 MFMA over the channel-major copy; 2:4 block: 8 SMFMAC
//   Every split writes its normalised partial o (fp32) and log-sum-exp to the workspace.
// k_decode_combine: a second launch on the same stream, one wave per (batch entry, query head);
//   merges that head's splits by their log-sum-exp and writes o (bf16) and lse. With one split
//   the split kernel writes o and lse itself and nothing else is launched.
//
// LDS tile layout (unpadded, 32 KB per stage): K rows are stored in the MFMA row order
// (tile_token), V^T rows in channel order. The 16-byte units of every row are XOR-swizzled by a
// function of the row, so that the 16 rows one operand read touches at one k-step land in distinct
// bank groups. The swizzle of a row is the XOR of a per-lane part (the lane's position inside a
// 1 KB load) and a per-load constant, so a load costs one precomputed lane offset plus uniform
// arithmetic, and an operand read one precomputed lane offset plus an immediate.
#include "hs_device.h"
#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kD = 128;
constexpr int kTile = 64;
constexpr int kKMeta = 8 * 1024;             // 2:4 K metadata inside the K region
constexpr int kVReg = 16 * 1024;             // V region of a stage
constexpr int kVMeta = 8 * 1024;             // 2:4 V metadata inside the V region
constexpr int kStage = 32 * 1024;            // one tile: K 16 KB + V 16 KB (dense)
constexpr int kListCap = 1024;               // visible blocks listed per pass
constexpr int kScanChunks = 8;               // 64-block map chunks loaded per scan round
constexpr int kListOff = 2 * kStage;         // map entries of the listed blocks (K, then V)
constexpr int kLdsDec = kListOff + 2 * kListCap * 4;

struct DecodeArgs {
  CacheView c;
  const uint16_t *q;
  uint16_t *o;
  float *lse;
  float *part_o, *part_lse;
  int nb, total_w, hkv, hq, G, splits;
  float scale_log2;
};

// Row swizzles: 128-byte rows (8 units, 16 rows per operand read) and 64-byte rows (4 units).
__device__ __forceinline__ int f8(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int f4(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

// Direct loads one tile issues, by block modes (see issue() below).
template <int B>
__device__ __forceinline__ int tile_loads(int mk, int mv) {
  return (mk > 0 ? 16 : 9) + (mv > 0 ? 16 : (B == 64 ? 9 : 12));
}
// Inclusive prefix sum of x over the 64 lanes of the wave, on DPP lane moves (no LDS round trips):
// Hillis-Steele steps of 1, 2, 4, 8 lanes inside each 16-lane row (a lane whose source lies before
// its row adds 0), then each row adds the totals of the rows before it: lane 15's sum goes to row
// 1 (and lane 47's to row 3), then lane 31's to rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
  constexpr int kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143;
  x += __builtin_amdgcn_update_dpp(0, x, kRowShr | 1, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, kRowShr | 2, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, kRowShr | 4, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, kRowShr | 8, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, kRowBcast15, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, kRowBcast31, 0xC, 0xF, false);
  return x;
}

// Wait until at most n vector-memory operations are outstanding (n = a tile_loads value).
__device__ __forceinline__ void wait_tile(int n) {
  switch (n) {
    case 32: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
    case 28: asm volatile("s_waitcnt vmcnt(28)" ::: "memory"); break;
    case 25: asm volatile("s_waitcnt vmcnt(25)" ::: "memory"); break;
    case 21: asm volatile("s_waitcnt vmcnt(21)" ::: "memory"); break;
    case 18: asm volatile("s_waitcnt vmcnt(18)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

// Merge the splits of one query head's row (partial rows row * splits + s) by their log-sum-exps:
// o = sum_s e^(lse_s - m) o_s / sum_s e^(lse_s - m), lse = m + log(sum). Lane l owns channels
// 2 l, 2 l + 1. Each round of up to 64 splits keeps split s's weight in lane s, and its partial
// rows are loaded eight at a time, all before any is used; loads past the last split read the last
// split's row with weight 0, so every load is unconditional.
template <class E>
__device__ __forceinline__ void combine_row(const DecodeArgs &a, size_t row, int lane) {
  const int S = a.splits;
  const float *pl = a.part_lse + row * S;
  const float *po = a.part_o + row * S * kD + 2 * lane;
  const float ls0 = pl[min(lane, S - 1)];  // log-sum-exps of splits 0 .. 63
  float mx = lane < S ? ls0 : -INFINITY;
  for (int s0 = 64; s0 < S; s0 += 64)
    if (s0 + lane < S) mx = fmaxf(mx, pl[s0 + lane]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  float wsum = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int s0 = 0; s0 < S; s0 += 64) {
    const int ns = min(64, S - s0);
    const float ls = s0 == 0 ? ls0 : pl[s0 + min(lane, ns - 1)];
    // an empty split (no visible token) has lse -inf and weight 0
    const float wl = lane < ns && ls != -INFINITY ? __expf(ls - mx) : 0.f;
    for (int k0 = 0; k0 < ns; k0 += 8) {
      float2 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        v[k] = *reinterpret_cast<const float2 *>(po + (size_t)(s0 + min(k0 + k, ns - 1)) * kD);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float w = k0 + k < ns ? __builtin_bit_cast(
                                          float, __builtin_amdgcn_readlane(
                                                     __builtin_bit_cast(int, wl), k0 + k))
                                    : 0.f;
        wsum += w;
        acc0 += w * v[k].x;
        acc1 += w * v[k].y;
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  *reinterpret_cast<uint32_t *>(a.o + row * kD + 2 * lane) = pack2<E>(acc0 * inv, acc1 * inv);
  if (a.lse && lane == 0) a.lse[row] = wsum > 0.f ? mx + __logf(wsum) : -INFINITY;
}

template <int B, class E>
__global__ __launch_bounds__(64) void k_decode_split(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsDec];
  const int lane = threadIdx.x, col = lane & 15, g = lane >> 4;
  const int split = blockIdx.x, hkv = a.hkv;
  const int h = blockIdx.y % hkv, cg = blockIdx.y / hkv, bi = blockIdx.z;
  const int head = bi * hkv + h;
  const int hq0 = h * a.G + 16 * cg, ncol = min(16, a.G - 16 * cg);
  const bool live = col < ncol;
  constexpr int TPB = B / kTile;

  // Query registers: B operand of GEMM1, k-step s covers channels 32s .. 32s+31.
  uint4 qr[4];
  {
    const uint16_t *qp = a.q + ((size_t)bi * a.hq + hq0 + (live ? col : 0)) * kD + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qr[s] = live ? *reinterpret_cast<const uint4 *>(qp + 32 * s) : make_uint4(0, 0, 0, 0);
  }

  // ---- lane constants ----
  // Operand reads (byte offsets inside a stage). GEMM1 reads row slot 16t + col (token
  // tile_token(t, col)), GEMM2 reads channel 16ct + col.
  int rk[4], rkn[2], rvd[2];
#pragma unroll
  for (int s = 0; s < 4; ++s) rk[s] = col * 256 + (((4 * s + g) ^ col) << 4);
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
    rkn[c2] = col * 128 + (((4 * c2 + g) ^ f8(col)) << 4);
    rvd[c2] = kVReg + col * 128 + (((4 * c2 + g) ^ f8(col)) << 4);
  }
  const int rkm = kKMeta + col * 16 + 2 * g;
  const int rvn = kVReg + col * 64 + ((g ^ f4(col)) << 4);
  const int rvm = kVReg + kVMeta + col * 8 + 2 * g;
  // Direct loads (byte offsets from the global base of a load, before its uniform XOR part).
  const int rr4 = lane >> 4, rr8 = lane >> 3, rr16 = lane >> 2;
  const uint32_t dkd = rr4 * 256 + 16 * ((lane & 15) ^ rr4);
  const uint32_t dkn = ((rr8 & 3) | ((rr8 & 4) << 1)) * 128 + 16 * ((lane & 7) ^ rr8);
  const uint32_t dkm = (uint32_t)tile_token(lane >> 4, lane & 15) * 16;
  const uint32_t dvd = rr8 * (2 * B) + 16 * ((lane & 7) ^ rr8);
  const uint32_t dvn = rr16 * B + 16 * ((lane & 3) ^ f4(rr16));
  const uint32_t dvm = B == 64 ? 16 * lane : (lane >> 1) * 16 + 4 * (lane & 1);

  const uint32_t lds_base = (uint32_t)(size_t)(__attribute__((address_space(3))) char *)lds;
  int32_t *lk = reinterpret_cast<int32_t *>(lds + kListOff), *lv = lk + kListCap;

  // Direct loads of tile 'half' of a block (map entries mk, mv) into stage 'st'.
  auto issue = [&](int mk, int mv, int half, int st) {
    // Earlier reads of this stage are done, and at most 31 loads of the previous tile are still
    // outstanding, so with this tile's (at most 32) the 6-bit load counter cannot overflow.
    asm volatile("s_waitcnt vmcnt(31) lgkmcnt(0)" ::: "memory");
    const uint32_t kl = lds_base + st * kStage, vl = kl + kVReg;
    if (mk > 0) {
      const char *gb = uniform_ptr(a.c.k_dense + ((size_t)(mk - 1) * B + kTile * half) * kD);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        // rows 4q .. 4q+3 of the MFMA row order are four consecutive tokens (one 1 KB chunk)
        const int pq = ((q >> 2) & 1) | ((q & 3) << 1) | ((q >> 3) << 3);
        dma16_nt(gb + 1024 * pq, dkd ^ (64 * (q & 3)), kl + 1024 * q);
      }
    } else {
      const size_t row0 = (size_t)(-mk - 1) * B + kTile * half;
      const char *gb = uniform_ptr(a.c.k_nnz + row0 * (kD / 2));
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        // rows 8q .. 8q+7 are tokens tq + {0, 1, 2, 3, 8, 9, 10, 11}
        const int tq = (((q >> 1) & 1) << 2) | ((q & 1) << 4) | ((q >> 2) << 5);
        dma16_nt(gb + 128 * tq, dkn ^ (16 * (q & 1)), kl + 1024 * q);
      }
      dma16_nt(uniform_ptr(a.c.k_meta + row0 * (kD / 16)), dkm, kl + kKMeta);
    }
    if (mv > 0) {
      const char *gb = uniform_ptr(a.c.v_dense + (size_t)(mv - 1) * B * kD + kTile * half);
#pragma unroll
      for (int q = 0; q < 16; ++q) dma16_nt(gb + 16 * B * q, dvd ^ (16 * (q & 1)), vl + 1024 * q);
    } else {
      const size_t blk0 = (size_t)(-mv - 1) * B * kD;
      const char *gb = uniform_ptr(a.c.v_nnz + blk0 / 2 + (kTile / 2) * half);
#pragma unroll
      for (int q = 0; q < 8; ++q) dma16_nt(gb + 16 * B * q, dvn, vl + 1024 * q);
      const char *gm = uniform_ptr(a.c.v_meta + blk0 / 16 + (kTile / 16) * half);
      if (B == 64) {
        dma16_nt(gm, dvm, vl + kVMeta);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) dma4(gm + 512 * i, dvm, vl + kVMeta + 256 * i);
      }
    }
  };

  f32x4 oacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // This split's blocks. Splits are balanced by the loads their blocks issue (i.e. by bytes): with
  // w_j the load count of visible block j, p_j the sum of w over the blocks before it and W the sum
  // over the head, block j belongs to the split whose share of W holds the block's midpoint
  // (2 p_j + w_j) / 2W (clamped to the last split). Split s's share is the fraction
  // [C(s), C(s + 1)) / C(S) of a prefix sum C of split weights: 1 each, or, when the split count is
  // a multiple of 8 (split s then runs on XCD s mod 8: consecutive workgroups go to the 8 XCDs in
  // turn), 16 on even and 15 on odd XCDs, whose HBM reads were measured 7-9% slower. The blocks
  // are listed in LDS a batch of kScanChunks 64-block chunks at a time, in passes of at most
  // kListCap entries.
  const int32_t *mkh = a.c.map_k + (size_t)head * a.nb;
  const int32_t *mvh = a.c.map_v + (size_t)head * a.nb;
  const bool xcd_weighted = a.splits % 8 == 0;
  auto cum = [&](int sp) -> uint64_t {  // C(sp)
    return xcd_weighted ? (uint64_t)(sp >> 3) * 124 + 16 * (((sp & 7) + 1) >> 1) + 15 * ((sp & 7) >> 1)
                        : (uint64_t)sp;
  };
  const uint64_t c_total = cum(a.splits);
  const uint64_t two_w = 2 * (uint64_t)a.total_w;
  const uint64_t lo_key = two_w * cum(split), hi_key = two_w * cum(split + 1);
  const bool last_split = split == a.splits - 1;
  int scan = 0;       // first block of the next chunk
  int base = 0;       // sum of w over the blocks before 'scan'
  bool finished = a.total_w <= 0;
  while (!finished) {
    int got = 0;  // blocks listed in this pass
    while (!finished && got <= kListCap - 64 * kScanChunks) {
      int mkv[kScanChunks], mvv[kScanChunks];
#pragma unroll
      for (int i = 0; i < kScanChunks; ++i) {
        const int j = scan + 64 * i + lane;
        mkv[i] = j < a.nb ? mkh[j] : 0;
        mvv[i] = j < a.nb ? mvh[j] : 0;
      }
#pragma unroll
      for (int i = 0; i < kScanChunks; ++i) {
        if (finished) break;
        const int w = mkv[i] != 0 ? TPB * tile_loads<B>(mkv[i], mvv[i]) : 0;
        const int incl = wave_incl_scan(w);
        const uint64_t key = (uint64_t)(2 * (base + incl - w) + w) * c_total;
        const bool mine = w > 0 && key >= lo_key && (key < hi_key || last_split);
        const uint64_t bal = __ballot(mine);
        if (mine) {
          const int r = got + __popcll(bal & ((1ull << lane) - 1ull));
          lk[r] = mkv[i];
          lv[r] = mvv[i];
        }
        got += __popcll(bal);
        base += __builtin_amdgcn_readlane(incl, 63);
        scan += 64;
        // keys grow with the block index: once one passes this split's share, the rest do too
        const bool past = !last_split && __ballot(w > 0 && key >= hi_key) != 0;
        finished = past || scan >= a.nb;
      }
    }
    if (got == 0) break;
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");

    const int ntiles = got * TPB;
    auto mk_of = [&](int n) { return __builtin_amdgcn_readfirstlane(lk[n / TPB]); };
    auto mv_of = [&](int n) { return __builtin_amdgcn_readfirstlane(lv[n / TPB]); };
    int mk0 = mk_of(0), mv0 = mv_of(0);
    issue(mk0, mv0, 0, 0);
    for (int n = 0; n < ntiles; ++n) {
      int mk1 = 0, mv1 = 0;
      if (n + 1 < ntiles) {
        mk1 = mk_of(n + 1);
        mv1 = mv_of(n + 1);
        issue(mk1, mv1, (n + 1) % TPB, (n + 1) & 1);
        wait_tile(tile_loads<B>(mk1, mv1));
      } else {
        wait_tile(0);
      }
      const char *kl = lds + (n & 1) * kStage;

      // ---- S^T = K Q^T ----
      f32x4 sacc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (mk0 > 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int s = 0; s < 4; ++s)
            sacc[t] = mfma16<E>(*reinterpret_cast<const uint4 *>(kl + rk[s] + 4096 * t), qr[s],
                             sacc[t]);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2) {
            const uint4 kv = *reinterpret_cast<const uint4 *>(kl + rkn[c2] + 2048 * t);
            const uint32_t ix = *reinterpret_cast<const uint16_t *>(kl + rkm + 256 * t + 8 * c2);
            sacc[t] = smfmac16<E>(kv, qr[2 * c2], qr[2 * c2 + 1], ix, sacc[t]);
          }
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
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float psum = 0.f;
      uint32_t pp[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float p0 = __builtin_amdgcn_exp2f(sacc[t][0] - m_new);
        const float p1 = __builtin_amdgcn_exp2f(sacc[t][1] - m_new);
        const float p2 = __builtin_amdgcn_exp2f(sacc[t][2] - m_new);
        const float p3 = __builtin_amdgcn_exp2f(sacc[t][3] - m_new);
        psum += (p0 + p1) + (p2 + p3);
        pp[2 * t] = pack2<E>(p0, p1);
        pp[2 * t + 1] = pack2<E>(p2, p3);
      }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) oacc[ct] *= alpha;
      const uint4 plo = make_uint4(pp[0], pp[1], pp[2], pp[3]);  // tokens 8g .. 8g+7
      const uint4 phi = make_uint4(pp[4], pp[5], pp[6], pp[7]);  // tokens 32+8g .. 32+8g+7

      // ---- O^T += V^T P^T ----
      if (mv0 > 0) {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          oacc[ct] = mfma16<E>(*reinterpret_cast<const uint4 *>(kl + rvd[0] + 2048 * ct), plo,
                            oacc[ct]);
          oacc[ct] = mfma16<E>(*reinterpret_cast<const uint4 *>(kl + rvd[1] + 2048 * ct), phi,
                            oacc[ct]);
        }
      } else {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          const uint4 vv = *reinterpret_cast<const uint4 *>(kl + rvn + 1024 * ct);
          const uint32_t ix = *reinterpret_cast<const uint16_t *>(kl + rvm + 128 * ct);
          oacc[ct] = smfmac16<E>(vv, plo, phi, ix, oacc[ct]);
        }
      }
      mk0 = mk1;
      mv0 = mv1;
    }
  }

  // ---- normalised output of this split and its log-sum-exp ----
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (!live) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  const float lse_s = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  if (a.splits == 1) {  // the whole head in one split: this is the output
    const size_t orow = (size_t)bi * a.hq + hq0 + col;
    uint16_t *op = a.o + orow * kD + 4 * g;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
      *reinterpret_cast<uint2 *>(op + 16 * ct) =
          make_uint2(pack2<E>(oacc[ct][0] * inv, oacc[ct][1] * inv),
                     pack2<E>(oacc[ct][2] * inv, oacc[ct][3] * inv));
    if (a.lse && g == 0) a.lse[orow] = lse_s;
    return;
  }
  const size_t row = ((size_t)bi * a.hq + hq0 + col) * a.splits + split;
  float *po = a.part_o + row * kD + 4 * g;
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
    *reinterpret_cast<f32x4 *>(po + 16 * ct) = oacc[ct] * inv;
  if (g == 0) a.part_lse[row] = lse_s;
}

// ---- log-sum-exp combine of the splits, §IV-C: one wave per (batch entry, query head) merges the
// partials the split kernel left in the workspace. It is a second launch on the same stream, so the
// stream order alone makes every split's partials visible to it.
template <class E>
__global__ __launch_bounds__(64) void k_decode_combine(DecodeArgs a) {
  combine_row<E>(a, blockIdx.x, threadIdx.x);
}

}  // namespace

hipError_t launch_decode(const Dims &d, const CacheView &c, const uint16_t *q, uint16_t *o,
                         float *lse, float scale_log2, int splits, float *part_o, float *part_lse,
                         hipStream_t stream) {
  // Loads of one head's visible blocks (the per-tile counts of tile_loads, times tiles per block).
  const int total_w =
      (d.B / kTile) * (d.ndk * 16 + d.nsk * 9 + d.ndv * 16 + d.nsv * (d.B == 64 ? 9 : 12));
  DecodeArgs a{c, q, o, lse, part_o, part_lse, d.nb, total_w, d.hkv, d.hq, d.G, splits,
               scale_log2};
  const int col_groups = (d.G + 15) / 16;
  const dim3 grid(splits, d.hkv * col_groups, d.b), grid_c(d.b * d.hq);
  if (d.dtype == kF16) {
    if (d.B == 64)
      k_decode_split<64, _Float16><<<grid, 64, 0, stream>>>(a);
    else
      k_decode_split<128, _Float16><<<grid, 64, 0, stream>>>(a);
    if (splits > 1) k_decode_combine<_Float16><<<grid_c, 64, 0, stream>>>(a);
  } else {
    if (d.B == 64)
      k_decode_split<64, __bf16><<<grid, 64, 0, stream>>>(a);
    else
      k_decode_split<128, __bf16><<<grid, 64, 0, stream>>>(a);
    if (splits > 1) k_decode_combine<__bf16><<<grid_c, 64, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace hs
