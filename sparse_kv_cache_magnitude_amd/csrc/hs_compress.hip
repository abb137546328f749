// hs_compress.hip -- magnitude-based hierarchical compressor for gfx950.
//
// "HieraSparse" (arXiv 2604.16864v2) §III-A Eq. (2a)-(2d), §III-B memory pools / signed block
// index map, §IV-B fused magnitude compression. Three kernels, all streaming K and V from HBM:
//   k_score  one workgroup per (head, block): reads the K and V block once and reduces the three
//            integer losses of the block (K 2:4 loss, V 2:4 loss, whole-block magnitude).
//   k_rank   one workgroup per head: bitonic sorts of (loss, block index) in LDS choose the pruned,
//            K 2:4 and V 2:4 blocks, then a prefix count over block order assigns pool slots -- the
//            paper's sequential dense / sparse counters, computed in parallel.
//   k_pack   one workgroup per (head, block): copies dense blocks (V transposed to channel-major)
//            and writes kept values + 2-bit positions of 2:4 blocks.
// Losses are integer sums of floor(|x| * 2^24), so the result does not depend on summation order
// and equal inputs give equal bytes.
#include "hs_device.h"
#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kD = 128;  // head_dim handled on the GPU

// ----------------------------------------------------------------------------------------------
// k_score

// floor(|x| * 2^24) of an fp16 magnitude (bits & 0x7FFF): a normal value is (1024 + m) *
// 2^(e - 25), so the key is (1024 + m) shifted by e - 1; a subnormal one is m * 2^-24, key m.
// Every fp16 value is a multiple of 2^-24, so the key is exact.
__device__ __forceinline__ uint64_t fixed_mag_f16(uint32_t a) {
  const uint32_t e = a >> 10, m = a & 0x3FFu;
  return e ? (uint64_t)(m | 0x400u) << (e - 1) : (uint64_t)m;
}
template <class E>
__device__ __forceinline__ uint64_t fixed_mag_e(uint32_t a) {
  if constexpr (__is_same(E, _Float16))
    return fixed_mag_f16(a);
  else
    return fixed_mag(a);
}

template <class E>
__device__ __forceinline__ void score_group(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                            uint64_t &drop, uint64_t &all) {
  uint32_t a0 = x0 & 0x7FFFu, a1 = x1 & 0x7FFFu, a2 = x2 & 0x7FFFu, a3 = x3 & 0x7FFFu;
  uint64_t f0 = fixed_mag_e<E>(a0), f1 = fixed_mag_e<E>(a1), f2 = fixed_mag_e<E>(a2),
           f3 = fixed_mag_e<E>(a3);
  uint32_t keep = keep_mask(a0, a1, a2, a3);
  all += f0 + f1 + f2 + f3;
  drop += ((keep & 1u) ? 0ull : f0) + ((keep & 2u) ? 0ull : f1) + ((keep & 4u) ? 0ull : f2) +
          ((keep & 8u) ? 0ull : f3);
}

// Fast form of the same keys for magnitudes below 256 (bf16 magnitude bits a < 0x4380): the bf16
// bits are the high half of the fp32 value, and the product with 2^24 is exact (denormal inputs
// become normal values below 1 that truncate to 0, their floor as well), so the truncating
// conversion gives floor(|x| * 2^24) < 2^32. Before the conversion the product is clamped to
// 4294967040 (the largest fp32 below 2^32; an infinite product, or a NaN one from a non-finite
// pattern, gives the clamp value too), so every 15-bit pattern converts in range. Magnitudes of
// 256 or more therefore key to 0xFFFFFF00, above every in-range key (255 * 2^24 = 0xFF000000):
// the caller detects that and redoes the block with score_group.
// fp16: the value converted to fp32 and scaled by 2^24 is an integer, exact below 256 (largest
// key floor(255.875 * 2^24) = 0xFFE00000), clamped the same way from 256 on.
template <class E>
__device__ __forceinline__ uint32_t fixed_mag_small(uint32_t a) {
  float v;
  if constexpr (__is_same(E, _Float16))
    v = (float)__builtin_bit_cast(_Float16, (uint16_t)a) * 16777216.0f;
  else
    v = __uint_as_float(a << 16) * 16777216.0f;
  return (uint32_t)fminf(v, 4294967040.0f);
}
// The two dropped values of a group are its two smallest keys (the key is monotone in the
// magnitude, and which of two equal magnitudes is dropped does not change the sum).
template <class E>
__device__ __forceinline__ void score_group_fast(uint32_t x0, uint32_t x1, uint32_t x2,
                                                 uint32_t x3, uint64_t &drop, uint64_t &all,
                                                 uint32_t &fmax) {
  const uint32_t f0 = fixed_mag_small<E>(x0 & 0x7FFFu), f1 = fixed_mag_small<E>(x1 & 0x7FFFu);
  const uint32_t f2 = fixed_mag_small<E>(x2 & 0x7FFFu), f3 = fixed_mag_small<E>(x3 & 0x7FFFu);
  const uint32_t l1 = min(f0, f1), h1 = max(f0, f1), l2 = min(f2, f3), h2 = max(f2, f3);
  all += ((uint64_t)f0 + f1) + ((uint64_t)f2 + f3);
  drop += (uint64_t)min(l1, l2) + min(max(l1, l2), min(h1, h2));
  fmax = max(fmax, max(h1, h2));
}
// The largest fast-path key: floor(255 * 2^24) for bf16, floor(255.875 * 2^24) for fp16.
template <class E>
constexpr uint32_t kMaxSmallKey = __is_same(E, _Float16) ? 0xFFE00000u : 0xFF000000u;

__device__ __forceinline__ uint32_t elem(const uint4 &v, int e) {
  uint32_t w = e < 2 ? v.x : (e < 4 ? v.y : (e < 6 ? v.z : v.w));
  return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// 16-byte load with the nontemporal cache policy: K and V are streamed once per pass.
typedef uint32_t u32x4nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldnt(const uint16_t *p) {
  const u32x4nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4nt *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int B, class E>
__global__ __launch_bounds__(256) void k_score(const uint16_t *__restrict__ K,
                                               const uint16_t *__restrict__ V,
                                               uint64_t *__restrict__ keys, int L) {
  const int i = blockIdx.x, nb = gridDim.x, tid = threadIdx.x;
  const size_t base = (size_t)blockIdx.y * L * kD + (size_t)i * B * kD;
  const uint16_t *Kb = K + base, *Vb = V + base;
  uint64_t kk = 0, kv = 0, kp = 0;
  uint32_t fmax = 0;
  const int c8 = tid & 15;  // eight consecutive channels
#pragma unroll
  for (int g = tid >> 4; g < B / 4; g += 16) {  // four consecutive tokens
    uint4 kr[4], vr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      kr[r] = ldnt(Kb + (size_t)(4 * g + r) * kD + 8 * c8);
      vr[r] = ldnt(Vb + (size_t)(4 * g + r) * kD + 8 * c8);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {  // K: groups of four channels of one token
      score_group_fast<E>(kr[r].x & 0xFFFFu, kr[r].x >> 16, kr[r].y & 0xFFFFu, kr[r].y >> 16, kk,
                       kp, fmax);
      score_group_fast<E>(kr[r].z & 0xFFFFu, kr[r].z >> 16, kr[r].w & 0xFFFFu, kr[r].w >> 16, kk,
                       kp, fmax);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)  // V: groups of four tokens of one channel
      score_group_fast<E>(elem(vr[0], e), elem(vr[1], e), elem(vr[2], e), elem(vr[3], e), kv, kp,
                       fmax);
  }
  if (__ballot(fmax > kMaxSmallKey<E>) != 0) {
    // A magnitude of 256 or more in this wave's share: redo the share with the 64-bit keys.
    kk = kv = kp = 0;
    for (int g = tid >> 4; g < B / 4; g += 16) {
      uint4 kr[4], vr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        kr[r] = *reinterpret_cast<const uint4 *>(Kb + (size_t)(4 * g + r) * kD + 8 * c8);
        vr[r] = *reinterpret_cast<const uint4 *>(Vb + (size_t)(4 * g + r) * kD + 8 * c8);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        score_group<E>(kr[r].x & 0xFFFFu, kr[r].x >> 16, kr[r].y & 0xFFFFu, kr[r].y >> 16, kk, kp);
        score_group<E>(kr[r].z & 0xFFFFu, kr[r].z >> 16, kr[r].w & 0xFFFFu, kr[r].w >> 16, kk, kp);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        score_group<E>(elem(vr[0], e), elem(vr[1], e), elem(vr[2], e), elem(vr[3], e), kv, kp);
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    kk += shfl_xor_u64(kk, m);
    kv += shfl_xor_u64(kv, m);
    kp += shfl_xor_u64(kp, m);
  }
  __shared__ uint64_t part[4][3];
  if ((tid & 63) == 0) {
    part[tid >> 6][0] = kk;
    part[tid >> 6][1] = kv;
    part[tid >> 6][2] = kp;
  }
  __syncthreads();
  if (tid < 3) {
    uint64_t s = part[0][tid] + part[1][tid] + part[2][tid] + part[3][tid];
    keys[((size_t)blockIdx.y * nb + i) * 3 + tid] = s;
  }
}

// ----------------------------------------------------------------------------------------------
// k_rank

constexpr int kRankThreads = 1024;

// Ascending bitonic sort of (key, idx) pairs of length n (a power of two) in LDS by 'nthreads'
// threads of the workgroup (thread number 'th' among them); every thread of the workgroup calls it
// with the same n, so the barriers match.
__device__ void bitonic_sort(uint64_t *key, uint16_t *idx, int n, int th, int nthreads) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int t = th; t < n / 2; t += nthreads) {
        int a = (t / j) * 2 * j + (t % j), b = a + j;
        bool up = (a & k) == 0;
        uint64_t ka = key[a], kb = key[b];
        uint16_t ia = idx[a], ib = idx[b];
        bool a_gt_b = ka > kb || (ka == kb && ia > ib);
        if (a_gt_b == up) {
          key[a] = kb;
          key[b] = ka;
          idx[a] = ib;
          idx[b] = ia;
        }
      }
      __syncthreads();
    }
  }
}

// Blocks i < dense_lo or i >= dense_hi are kept dense for K and V and take no part in the
// ranking (the sink and local-window tokens); the counts apply to the blocks in between.
__global__ __launch_bounds__(kRankThreads) void k_rank(const uint64_t *__restrict__ keys, int nb,
                                                       int n_p, int n_sk, int n_sv, int dense_lo,
                                                       int dense_hi, int32_t *__restrict__ map_k,
                                                       int32_t *__restrict__ map_v) {
  __shared__ uint64_t skey[2][kMaxBlocks];
  __shared__ uint16_t sidx[2][kMaxBlocks];
  __shared__ uint8_t mode[2][kMaxBlocks];  // 0 pruned, 1 dense, 2 2:4
  __shared__ int scan[4][kRankThreads];
  const int hd = blockIdx.x, tid = threadIdx.x;
  const uint64_t *hk = keys + (size_t)hd * nb * 3;
  int n = 2;
  while (n < nb) n <<= 1;

  // Pruned blocks: the n_p smallest whole-block magnitudes among the blocks that may be pruned
  // (a kept-dense block carries the largest key, which no real loss reaches).
  auto ranked = [&](int t) { return t < nb && t >= dense_lo && t < dense_hi; };
  for (int t = tid; t < n; t += kRankThreads) {
    skey[0][t] = ranked(t) ? hk[3 * t + 2] : ~0ull;
    sidx[0][t] = (uint16_t)t;
  }
  __syncthreads();
  bitonic_sort(skey[0], sidx[0], n, tid, kRankThreads);
  for (int t = tid; t < nb; t += kRankThreads) {
    uint8_t m = t < n_p ? 0 : 1;
    mode[0][sidx[0][t]] = m;
    mode[1][sidx[0][t]] = m;
  }
  __syncthreads();

  // Eq. (2d) per tensor among the survivors: the n_s smallest 2:4 losses become 2:4. Pruned
  // blocks carry the largest key, which no real loss reaches (|x| < 2^24 keeps losses < 2^63).
  // K (x = 0) and V (x = 1) are sorted at once, each by half of the workgroup.
  for (int x = 0; x < 2; ++x)
    for (int t = tid; t < n; t += kRankThreads) {
      skey[x][t] = (ranked(t) && mode[x][t] != 0) ? hk[3 * t + x] : ~0ull;
      sidx[x][t] = (uint16_t)t;
    }
  __syncthreads();
  {
    constexpr int kHalf = kRankThreads / 2;
    const int x = tid / kHalf;
    bitonic_sort(skey[x], sidx[x], n, tid % kHalf, kHalf);
  }
  for (int x = 0; x < 2; ++x) {
    const int want = x ? n_sv : n_sk;
    for (int t = tid; t < want; t += kRankThreads) mode[x][sidx[x][t]] = 2;
  }
  __syncthreads();

  // Pool slots in block order: exclusive prefix counts of dense and 2:4 blocks, both tensors in
  // one scan (counters: K dense, K 2:4, V dense, V 2:4).
  constexpr int kPer = kMaxBlocks / kRankThreads;
  int cnt[4] = {0, 0, 0, 0};
  for (int e = 0; e < kPer; ++e) {
    int i = tid * kPer + e;
    if (i < nb) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        cnt[2 * x] += mode[x][i] == 1;
        cnt[2 * x + 1] += mode[x][i] == 2;
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) scan[c][tid] = cnt[c];
  __syncthreads();
  for (int off = 1; off < kRankThreads; off <<= 1) {
    int v[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = tid >= off ? scan[c][tid - off] : 0;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) scan[c][tid] += v[c];
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int ns = x ? n_sv : n_sk, nd = nb - n_p - ns;
    int rd = scan[2 * x][tid] - cnt[2 * x] + hd * nd;
    int rs = scan[2 * x + 1][tid] - cnt[2 * x + 1] + hd * ns;
    int32_t *map = (x ? map_v : map_k) + (size_t)hd * nb;
    for (int e = 0; e < kPer; ++e) {
      int i = tid * kPer + e;
      if (i < nb) {
        uint8_t m = mode[x][i];
        map[i] = m == 0 ? 0 : (m == 1 ? ++rd : -(++rs));
      }
    }
  }
}

// ----------------------------------------------------------------------------------------------
// k_pack

template <int B>
__global__ __launch_bounds__(256) void k_pack(const uint16_t *__restrict__ K,
                                              const uint16_t *__restrict__ V,
                                              const int32_t *__restrict__ map_k,
                                              const int32_t *__restrict__ map_v, CacheView c,
                                              int L) {
  constexpr int BD = B * kD;
  const int i = blockIdx.x, nb = gridDim.x, tid = threadIdx.x;
  const size_t base = (size_t)blockIdx.y * L * kD + (size_t)i * BD;
  const int32_t mk = map_k[(size_t)blockIdx.y * nb + i], mv = map_v[(size_t)blockIdx.y * nb + i];

  // K: dense copy, or per token: four groups of four channels -> 8 kept values + 1 meta word.
  if (mk > 0) {
    uint4 *dst = reinterpret_cast<uint4 *>(c.k_dense + (size_t)(mk - 1) * BD);
#pragma unroll
    for (int e = tid; e < BD / 8; e += 256) dst[e] = ldnt(K + base + 8 * e);
  } else if (mk < 0) {
    const size_t s = (size_t)(-mk - 1);
    uint16_t *nnz = c.k_nnz + s * (BD / 2), *meta = c.k_meta + s * (BD / 16);
#pragma unroll
    for (int item = tid; item < B * (kD / 16); item += 256) {
      const int t = item >> 3, w = item & 7;
      const uint16_t *p = K + base + (size_t)t * kD + 16 * w;
      const uint4 x0 = ldnt(p), x1 = ldnt(p + 8);
      const uint32_t wd[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      uint32_t pairs[4], word = 0;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint32_t e0 = wd[2 * g] & 0xFFFFu, e1 = wd[2 * g] >> 16;
        uint32_t e2 = wd[2 * g + 1] & 0xFFFFu, e3 = wd[2 * g + 1] >> 16;
        uint32_t nib = mask_to_nibble(
            keep_mask(e0 & 0x7FFFu, e1 & 0x7FFFu, e2 & 0x7FFFu, e3 & 0x7FFFu));
        pairs[g] = kept_pair(nib, e0, e1, e2, e3);
        word |= nib << (4 * g);
      }
      *reinterpret_cast<uint4 *>(nnz + (size_t)t * (kD / 2) + 8 * w) =
          make_uint4(pairs[0], pairs[1], pairs[2], pairs[3]);
      meta[(size_t)t * (kD / 16) + w] = (uint16_t)word;
    }
  }

  // V: both pools are channel-major (row = one channel's B tokens), the block token-major. The
  // block goes through LDS (16-byte unit u of token row t at unit u ^ ((t >> 3) & 7), so that the
  // column reads below hit distinct banks), then each lane emits 16 contiguous bytes of one
  // channel row: a wave writes 1 KB of consecutive rows at a time.
  if (mv != 0) {
    __shared__ __attribute__((aligned(16))) uint16_t vt[B * kD];
    const bool dense = mv > 0;
    const size_t s = dense ? (size_t)(mv - 1) : (size_t)(-mv - 1);
    auto at = [](int t, int ch) { return t * kD + 8 * ((ch >> 3) ^ ((t >> 3) & 7)) + (ch & 7); };
#pragma unroll
    for (int idx = tid; idx < B * 16; idx += 256) {
      const int t = idx >> 4, u = idx & 15;
      *reinterpret_cast<uint4 *>(vt + at(t, 8 * u)) = ldnt(V + base + (size_t)t * kD + 8 * u);
    }
    __syncthreads();
    if (dense) {
      uint16_t *dst = c.v_dense + s * BD;
#pragma unroll
      for (int idx = tid; idx < kD * (B / 8); idx += 256) {  // (channel, 8 tokens)
        const int ch = idx / (B / 8), j = idx % (B / 8);
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          w[k] = (uint32_t)vt[at(8 * j + 2 * k, ch)] | ((uint32_t)vt[at(8 * j + 2 * k + 1, ch)] << 16);
        *reinterpret_cast<uint4 *>(dst + (size_t)ch * B + 8 * j) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    } else {
      uint16_t *nnz = c.v_nnz + s * (BD / 2), *meta = c.v_meta + s * (BD / 16);
#pragma unroll
      for (int idx = tid; idx < kD * (B / 16); idx += 256) {  // (channel, 16 tokens)
        const int ch = idx / (B / 16), wd = idx % (B / 16);
        uint32_t pairs[4], word = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // groups of four tokens
          const int t0 = 16 * wd + 4 * q;
          const uint32_t x0 = vt[at(t0, ch)], x1 = vt[at(t0 + 1, ch)], x2 = vt[at(t0 + 2, ch)],
                         x3 = vt[at(t0 + 3, ch)];
          const uint32_t nib = mask_to_nibble(
              keep_mask(x0 & 0x7FFFu, x1 & 0x7FFFu, x2 & 0x7FFFu, x3 & 0x7FFFu));
          pairs[q] = kept_pair(nib, x0, x1, x2, x3);
          word |= nib << (4 * q);
        }
        *reinterpret_cast<uint4 *>(nnz + (size_t)ch * (B / 2) + 8 * wd) =
            make_uint4(pairs[0], pairs[1], pairs[2], pairs[3]);
        meta[(size_t)ch * (B / 16) + wd] = (uint16_t)word;
      }
    }
  }
}

}  // namespace

hipError_t launch_compress(const Dims &d, const uint16_t *k, const uint16_t *v, const CacheView &c,
                           uint64_t *keys, hipStream_t stream, int dense_lo, int dense_hi) {
  const dim3 grid(d.nb, d.b * d.hkv);
  if (d.dtype == kF16) {
    if (d.B == 64)
      k_score<64, _Float16><<<grid, 256, 0, stream>>>(k, v, keys, d.L);
    else
      k_score<128, _Float16><<<grid, 256, 0, stream>>>(k, v, keys, d.L);
  } else {
    if (d.B == 64)
      k_score<64, __bf16><<<grid, 256, 0, stream>>>(k, v, keys, d.L);
    else
      k_score<128, __bf16><<<grid, 256, 0, stream>>>(k, v, keys, d.L);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_rank<<<d.b * d.hkv, kRankThreads, 0, stream>>>(keys, d.nb, d.np, d.nsk, d.nsv, dense_lo,
                                                   dense_hi < 0 ? d.nb : dense_hi, c.map_k,
                                                   c.map_v);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_pack(d, k, v, c, stream);
}

hipError_t launch_pack(const Dims &d, const uint16_t *k, const uint16_t *v, const CacheView &c,
                       hipStream_t stream) {
  const dim3 grid(d.nb, d.b * d.hkv);
  if (d.B == 64)
    k_pack<64><<<grid, 256, 0, stream>>>(k, v, c.map_k, c.map_v, c, d.L);
  else
    k_pack<128><<<grid, 256, 0, stream>>>(k, v, c.map_k, c.map_v, c, d.L);
  return hipGetLastError();
}

}  // namespace hs
