// hs_recompress.hip -- re-compression of a compressed cache with new block counts (gfx950).
//
// "HieraSparse" (arXiv 2604.16864v2) §III, Fig. 3: the cache can be compressed differently for
// prefill and for decode (for example K dense and V 2:4 while the prompt is processed, then K and
// V both 2:4 for decode). Re-compression is defined as compression (§III-A Eq. (2a)-(2d), §III-B)
// of the dense tensors a compressed cache stands for: kept values in place, zeros where a 2:4
// group dropped an element and over pruned blocks. k_unpack rebuilds those tensors in the
// workspace; the compressor then runs unchanged on them. A block that is already 2:4 or pruned
// carries no loss for staying so, so it is chosen first again for that mode.
//
// k_unpack: one workgroup per (block, KV head, batch entry). K tiles are token-major in both the
// pools and the output, so dense blocks are copied and 2:4 groups expanded directly (16 output
// bytes per thread step, coalesced). V pools are channel-major (V^T), the output token-major: the
// workgroup builds the block's V^T in LDS (rows padded by 4 bytes to spread the column reads
// below over the banks) and writes it out transposed.
#include "hs_device.h"
#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kD = 128;
constexpr int kThreads = 256;

// Eight bf16 values (16 bytes) from two packed 2:4 groups: kept pair words and their 8 metadata
// bits (group 0 in the low nibble).
__device__ __forceinline__ uint4 expand8(uint2 pairs, uint32_t bits) {
  const uint2 g0 = expand_group(pairs.x, bits & 15u), g1 = expand_group(pairs.y, (bits >> 4) & 15u);
  return make_uint4(g0.x, g0.y, g1.x, g1.y);
}

template <int B>
__global__ __launch_bounds__(kThreads) void k_unpack(CacheView c, uint16_t *k_out, uint16_t *v_out,
                                                    int L, int nb) {
  constexpr int kRowV = B + 2;  // LDS row of V^T, in bf16 elements
  __shared__ __attribute__((aligned(16))) uint16_t vt[kD * kRowV];
  const int j = blockIdx.x, head = blockIdx.y, tid = threadIdx.x;
  const int mk = c.map_k[(size_t)head * nb + j], mv = c.map_v[(size_t)head * nb + j];
  constexpr int kChunks = B * kD / 8;  // 16-byte chunks of one tile

  // ---- K: token-major in and out; chunk q = (token t, 8 channels 8 * (q % 16)).
  uint4 *ko = reinterpret_cast<uint4 *>(k_out + ((size_t)head * L + (size_t)j * B) * kD);
  if (mk > 0) {
    const uint4 *src = reinterpret_cast<const uint4 *>(c.k_dense + (size_t)(mk - 1) * B * kD);
    for (int q = tid; q < kChunks; q += kThreads) ko[q] = src[q];
  } else if (mk < 0) {
    const size_t slot = (size_t)(-mk - 1);
    const uint2 *nnz = reinterpret_cast<const uint2 *>(c.k_nnz + slot * B * (kD / 2));
    const uint8_t *meta = reinterpret_cast<const uint8_t *>(c.k_meta + slot * B * (kD / 16));
    // Chunk q of token t covers groups 2q', 2q'+1 (q' = q % 16): kept pairs at uint2 index q and
    // metadata byte q (low nibble group 2q', high nibble group 2q'+1).
    for (int q = tid; q < kChunks; q += kThreads) ko[q] = expand8(nnz[q], meta[q]);
  } else {
    for (int q = tid; q < kChunks; q += kThreads) ko[q] = make_uint4(0, 0, 0, 0);
  }

  // ---- V: the block's V^T [D][B] into LDS, then out token-major.
  if (mv > 0) {
    const uint4 *src = reinterpret_cast<const uint4 *>(c.v_dense + (size_t)(mv - 1) * B * kD);
    for (int q = tid; q < kChunks; q += kThreads) {
      const int ch = q / (B / 8), t8 = q % (B / 8);
      const uint4 x = src[q];
      uint32_t *row = reinterpret_cast<uint32_t *>(vt + ch * kRowV + 8 * t8);
      row[0] = x.x; row[1] = x.y; row[2] = x.z; row[3] = x.w;
    }
  } else if (mv < 0) {
    const size_t slot = (size_t)(-mv - 1);
    const uint2 *nnz = reinterpret_cast<const uint2 *>(c.v_nnz + slot * kD * (B / 2));
    const uint8_t *meta = reinterpret_cast<const uint8_t *>(c.v_meta + slot * kD * (B / 16));
    for (int q = tid; q < kChunks; q += kThreads) {
      const int ch = q / (B / 8), t8 = q % (B / 8);
      const uint4 x = expand8(nnz[q], meta[q]);
      uint32_t *row = reinterpret_cast<uint32_t *>(vt + ch * kRowV + 8 * t8);
      row[0] = x.x; row[1] = x.y; row[2] = x.z; row[3] = x.w;
    }
  }
  __syncthreads();
  uint4 *vo = reinterpret_cast<uint4 *>(v_out + ((size_t)head * L + (size_t)j * B) * kD);
  for (int q = tid; q < kChunks; q += kThreads) {
    // Output chunk q = (token t, channels 8 c8 .. 8 c8 + 7), channel chunks fastest.
    const int t = q / (kD / 8), c8 = q % (kD / 8);
    uint4 y = make_uint4(0, 0, 0, 0);
    if (mv != 0) {
      const uint16_t *col = vt + 8 * c8 * kRowV + t;
      y.x = col[0] | (uint32_t)col[kRowV] << 16;
      y.y = col[2 * kRowV] | (uint32_t)col[3 * kRowV] << 16;
      y.z = col[4 * kRowV] | (uint32_t)col[5 * kRowV] << 16;
      y.w = col[6 * kRowV] | (uint32_t)col[7 * kRowV] << 16;
    }
    vo[q] = y;
  }
}

}  // namespace

hipError_t launch_unpack(const Dims &d, const CacheView &c, uint16_t *k_out, uint16_t *v_out,
                         hipStream_t stream) {
  const dim3 grid(d.nb, d.b * d.hkv);
  if (d.B == 64)
    k_unpack<64><<<grid, kThreads, 0, stream>>>(c, k_out, v_out, d.L, d.nb);
  else
    k_unpack<128><<<grid, kThreads, 0, stream>>>(c, k_out, v_out, d.L, d.nb);
  return hipGetLastError();
}

}  // namespace hs
