// hs_masked.hip -- block modes chosen by the caller: validation and pool slots (gfx950).
//
// "HieraSparse" (arXiv 2604.16864v2) §III-A (the cache pruner takes a block-level mask and an
// element-level mask from any pruning algorithm) and §IV-B (the generic compression kernel: dense
// blocks are copied, sparse blocks of an input that already has the element mask applied keep
// their non-zero values and positions). The caller gives the block level as one mode byte per
// (batch entry, KV head, block) and tensor; k_modes turns it into the signed index maps with the
// same per-head slot ranges the magnitude compressor assigns, after which the pack kernel writes
// the pools. Keeping the two largest magnitudes of a group of four (lower position on ties) is
// the same as keeping its non-zero values, padded with the lowest zero positions, whenever the
// group holds at most two non-zeros, so the pack kernel serves both compressors unchanged.
//
// k_modes: one workgroup per (batch entry, KV head). A head is rejected -- its maps written as all
// pruned, its pool slots left untouched -- if a mode byte is above 2, K and V disagree on a
// pruned block, or its counts differ from the per-head counts the pools are sized for; that keeps
// every pool write inside the head's own slot range whatever the mode bytes hold.
#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kThreads = 1024;
constexpr int kPer = kMaxBlocks / kThreads;  // blocks per thread

__global__ __launch_bounds__(kThreads) void k_modes(const uint8_t *__restrict__ mode_k,
                                                    const uint8_t *__restrict__ mode_v, int nb,
                                                    int n_p, int n_sk, int n_sv,
                                                    int32_t *__restrict__ map_k,
                                                    int32_t *__restrict__ map_v,
                                                    int32_t *__restrict__ head_status) {
  __shared__ int scan[4][kThreads];  // dense K, 2:4 K, dense V, 2:4 V counts, then prefix sums
  __shared__ int n_pruned;
  const int hd = blockIdx.x, tid = threadIdx.x;
  const uint8_t *mk = mode_k + (size_t)hd * nb, *mv = mode_v + (size_t)hd * nb;
  uint8_t m[2][kPer];
  if (tid == 0) n_pruned = 0;
  int cnt[4] = {0, 0, 0, 0}, pruned = 0, bad_value = 0, bad_pair = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int i = tid * kPer + e;
    m[0][e] = i < nb ? mk[i] : 1;
    m[1][e] = i < nb ? mv[i] : 1;
    if (i < nb) {
      bad_value |= m[0][e] > 2 || m[1][e] > 2;
      bad_pair |= (m[0][e] == 0) != (m[1][e] == 0);
      pruned += m[0][e] == 0;
      cnt[0] += m[0][e] == 1;
      cnt[1] += m[0][e] == 2;
      cnt[2] += m[1][e] == 1;
      cnt[3] += m[1][e] == 2;
    }
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) scan[x][tid] = cnt[x];
  __syncthreads();
  if (pruned) atomicAdd(&n_pruned, pruned);
  const int any_value = __syncthreads_or(bad_value), any_pair = __syncthreads_or(bad_pair);
  // Inclusive prefix sums of the four counts over the threads (Hillis-Steele in LDS).
  for (int off = 1; off < kThreads; off <<= 1) {
    int add[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) add[x] = tid >= off ? scan[x][tid - off] : 0;
    __syncthreads();
#pragma unroll
    for (int x = 0; x < 4; ++x) scan[x][tid] += add[x];
    __syncthreads();
  }
  const int last = kThreads - 1;
  const int status = (any_value ? 1 : 0) | (any_pair ? 2 : 0) |
                     (n_pruned != n_p || scan[1][last] != n_sk || scan[3][last] != n_sv ? 4 : 0);
  if (head_status && tid == 0) head_status[hd] = status;
  const int ndk = nb - n_p - n_sk, ndv = nb - n_p - n_sv;
  int rd[2] = {scan[0][tid] - cnt[0] + hd * ndk, scan[2][tid] - cnt[2] + hd * ndv};
  int rs[2] = {scan[1][tid] - cnt[1] + hd * n_sk, scan[3][tid] - cnt[3] + hd * n_sv};
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int i = tid * kPer + e;
    if (i < nb) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const uint8_t q = m[x][e];
        int32_t v = 0;
        if (status == 0 && q == 1) v = ++rd[x];
        else if (status == 0 && q == 2) v = -(++rs[x]);
        (x ? map_v : map_k)[(size_t)hd * nb + i] = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_modes(const Dims &d, const uint8_t *mode_k, const uint8_t *mode_v,
                        const CacheView &c, int32_t *head_status, hipStream_t stream) {
  k_modes<<<d.b * d.hkv, kThreads, 0, stream>>>(mode_k, mode_v, d.nb, d.np, d.nsk, d.nsv, c.map_k,
                                                c.map_v, head_status);
  return hipGetLastError();
}

}  // namespace hs
