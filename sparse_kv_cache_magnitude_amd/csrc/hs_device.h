// hs_device.h -- device-side building blocks shared by the gfx950 kernels of libhierasparse.
//
// Operand layouts of the matrix-core instructions used below (wave64, one 16x16 output tile,
// "chunk" = l / 16 for lane l):
//   v_mfma_f32_16x16x32_bf16   A[16][32] x B[32][16]: lane l holds row (A) / column (B) l % 16
//                              and k = 8*chunk .. 8*chunk + 7.
//   v_smfmac_f32_16x16x64_bf16 A is 2:4 along k. Lane l holds 8 kept values of row l % 16 for
//                              the logical k = 16*chunk .. 16*chunk + 15 (four groups of four);
//                              value e sits at position bits [2e+1:2e] of the low 16 index bits
//                              (abid 0) inside group e / 2. B lane l holds column l % 16 at
//                              k = 8*chunk + s for slots s = 0..7 and 32 + 8*chunk + (s - 8) for
//                              slots 8..15, i.e. two 16x16x32 B operands back to back.
//   accumulator                lane l holds rows 4*chunk .. 4*chunk + 3 of column l % 16.
// These were checked on gfx950 hardware against a CPU product of random integer-valued operands.
// Consequences used by the kernels:
//   * the index word of one lane is exactly one 16-bit metadata word of the packed format
//     (four groups, first kept position in the low two bits of each nibble);
//   * the B registers of a 64-deep SMFMAC are the B registers of two consecutive 32-deep dense
//     MFMAs, so dense and 2:4 tiles share the same query (GEMM1) and probability (GEMM2) registers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs {

// Element types of K, V, Q and O: E = __bf16 (the default) or _Float16. The packed format, the
// metadata and the 2:4 selection work on the 16-bit patterns and are the same for both; the
// matrix-core instructions, the fp32 -> 16-bit conversions and the magnitude keys differ.
template <class E> using vec2 = E __attribute__((ext_vector_type(2)));
template <class E> using vec8 = E __attribute__((ext_vector_type(8)));
template <class E> using vec16 = E __attribute__((ext_vector_type(16)));
typedef vec8<__bf16> bf16x8;
typedef vec16<__bf16> bf16x16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLn2 = 0.6931471805599453f;

template <class E>
__device__ __forceinline__ vec8<E> as8(uint4 v) { return __builtin_bit_cast(vec8<E>, v); }
template <class E>
__device__ __forceinline__ vec16<E> as16(uint4 lo, uint4 hi) {
  struct P {
    uint4 a, b;
  } p{lo, hi};
  return __builtin_bit_cast(vec16<E>, p);
}
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return as8<__bf16>(v); }
__device__ __forceinline__ bf16x16 as_bf16x16(uint4 lo, uint4 hi) { return as16<__bf16>(lo, hi); }

// Matrix-core instructions by element type (same operand layouts for both).
__device__ __forceinline__ f32x4 mma16x32(vec8<__bf16> a, vec8<__bf16> b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16x32(vec8<_Float16> a, vec8<_Float16> b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 smma16x64(vec8<__bf16> a, vec16<__bf16> b, f32x4 c, int idx) {
  return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a, b, c, idx, 0, 0);
}
__device__ __forceinline__ f32x4 smma16x64(vec8<_Float16> a, vec16<_Float16> b, f32x4 c,
                                           int idx) {
  return __builtin_amdgcn_smfmac_f32_16x16x64_f16(a, b, c, idx, 0, 0);
}
__device__ __forceinline__ f32x16 mma32x16(vec8<__bf16> a, vec8<__bf16> b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma32x16(vec8<_Float16> a, vec8<_Float16> b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// kSet selects the 16-bit index set of the index word: 0 = bits [15:0], 1 = bits [31:16].
template <int kSet = 0>
__device__ __forceinline__ f32x16 smma32x32(vec8<__bf16> a, vec16<__bf16> b, f32x16 c, int idx) {
  return __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a, b, c, idx, 0, kSet);
}
template <int kSet = 0>
__device__ __forceinline__ f32x16 smma32x32(vec8<_Float16> a, vec16<_Float16> b, f32x16 c,
                                            int idx) {
  return __builtin_amdgcn_smfmac_f32_32x32x32_f16(a, b, c, idx, 0, kSet);
}

template <class E = __bf16>
__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
  return mma16x32(as8<E>(a), as8<E>(b), c);
}

// 2:4 sparse A (8 kept values of 16 logical k) times dense B (two 16x16x32 B operands).
template <class E = __bf16>
__device__ __forceinline__ f32x4 smfmac16(uint4 a, uint4 b_lo, uint4 b_hi, uint32_t idx,
                                          f32x4 c) {
  return smma16x64(as8<E>(a), as16<E>(b_lo, b_hi), c, (int)idx);
}

// Two fp32 -> two packed 16-bit values (round to nearest even: one gfx950 v_cvt_pk_bf16_f32 or
// v_cvt_pk_f16_f32).
template <class E>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, vec2<E>));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) { return pack2<__bf16>(lo, hi); }

// acc + x.lo + x.hi for two packed 16-bit values (one v_dot2 with ones).
__device__ __forceinline__ float add_pair(vec2<__bf16> x, float acc) {
  const vec2<__bf16> one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(x, one, acc, false);
}
__device__ __forceinline__ float add_pair(vec2<_Float16> x, float acc) {
  const vec2<_Float16> one = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(x, one, acc, false);
}
template <class E>
__device__ __forceinline__ float add_pair_bits(uint32_t x, float acc) {
  return add_pair(__builtin_bit_cast(vec2<E>, x), acc);
}

// ----------------------------------------------------------------------------------------------
// Magnitude pruning of one group of four bf16 values.

// floor(|x| * 2^24) of a bf16 magnitude (bits & 0x7FFF), |x| < 2^24. A normal bf16 is
// (128 + m) * 2^(e - 134); scaled by 2^24 that is (128 + m) shifted by e - 110.
__device__ __forceinline__ uint64_t fixed_mag(uint32_t a) {
  int s = (int)(a >> 7) - 110;
  uint32_t man = (a & 0x7Fu) | 0x80u;
  uint64_t up = (uint64_t)man << (s > 0 ? s : 0);
  uint32_t down = (s > -8) ? (man >> (s < 0 ? -s : 0)) : 0u;
  return s >= 0 ? up : (uint64_t)down;
}

// Keep the two largest magnitudes of (a0..a3); equal magnitudes keep the lower position.
// Returns the 4-bit kept mask; element j is kept when fewer than two others beat it, where k
// beats j if a_k > a_j, or a_k == a_j and k < j.
__device__ __forceinline__ uint32_t keep_mask(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3) {
  uint32_t b01 = a0 >= a1, b02 = a0 >= a2, b03 = a0 >= a3;
  uint32_t b12 = a1 >= a2, b13 = a1 >= a3, b23 = a2 >= a3;
  uint32_t r0 = 3u - b01 - b02 - b03;
  uint32_t r1 = b01 + 2u - b12 - b13;
  uint32_t r2 = b02 + b12 + 1u - b23;
  uint32_t r3 = b03 + b13 + b23;
  return (uint32_t)(r0 < 2) | ((uint32_t)(r1 < 2) << 1) | ((uint32_t)(r2 < 2) << 2) |
         ((uint32_t)(r3 < 2) << 3);
}

// Kept mask -> metadata nibble (first position in bits 1:0, second in bits 3:2). The six valid
// masks 0b0011, 0b0101, 0b0110, 0b1001, 0b1010, 0b1100 map to 0x4, 0x8, 0x9, 0xC, 0xD, 0xE.
__device__ __forceinline__ uint32_t mask_to_nibble(uint32_t mask) {
  constexpr uint64_t kTable = (0x4ull << 12) | (0x8ull << 20) | (0x9ull << 24) | (0xCull << 36) |
                              (0xDull << 40) | (0xEull << 48);
  return (uint32_t)(kTable >> (4 * mask)) & 0xFu;
}

// Pack the two kept values of a group (x0..x3 as bf16 bits) into one dword, first kept in the
// low half.
__device__ __forceinline__ uint32_t kept_pair(uint32_t nib, uint32_t x0, uint32_t x1, uint32_t x2,
                                              uint32_t x3) {
  uint32_t i0 = nib & 3u, i1 = nib >> 2;
  uint32_t v0 = i0 == 0 ? x0 : (i0 == 1 ? x1 : x2);
  uint32_t v1 = i1 == 1 ? x1 : (i1 == 2 ? x2 : x3);
  return v0 | (v1 << 16);
}

// Expand one packed group (pair = first | second << 16, nibble) back to its four slots, as two
// dwords (slots 0,1 and slots 2,3) with zeros in the dropped slots.
__device__ __forceinline__ uint2 expand_group(uint32_t pair, uint32_t nib) {
  uint32_t i0 = nib & 3u, i1 = nib >> 2;
  uint32_t lo = pair & 0xFFFFu, hi = pair >> 16;
  uint32_t s0 = (i0 == 0 ? lo : 0u);
  uint32_t s1 = (i0 == 1 ? lo : 0u) | (i1 == 1 ? hi : 0u);
  uint32_t s2 = (i0 == 2 ? lo : 0u) | (i1 == 2 ? hi : 0u);
  uint32_t s3 = (i1 == 3 ? hi : 0u);
  return make_uint2(s0 | (s1 << 16), s2 | (s3 << 16));
}

// ----------------------------------------------------------------------------------------------
// Token order inside a 64-token tile.
//
// GEMM1 (S^T = K Q^T) produces four 16-row accumulator tiles; lane chunk g of tile t holds rows
// 4g..4g+3. GEMM2 (O^T = V^T P^T) wants, in lane chunk g, the probabilities of tokens
// 8g..8g+7 (B slots 0..7) and 32+8g..32+8g+7 (B slots 8..15). Feeding GEMM1 row r of tile t with
// token tile_token(t, r) makes the accumulators land exactly there, so P^T needs no data movement
// between lanes: each lane only packs its own fp32 values to bf16.
__device__ __forceinline__ int tile_token(int t, int r) {
  return 32 * (t >> 1) + 8 * (r >> 2) + 4 * (t & 1) + (r & 3);
}

// ----------------------------------------------------------------------------------------------
// Direct global -> LDS loads (gfx950 global_load_lds_dwordx4 / _dword).
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
// dma16 with the nontemporal cache policy: for data read once (the decode's stream), so that it
// does not displace reused lines.
__device__ __forceinline__ void dma16_nt(const void *gbase, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2 nt\n\t"
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
// N (1, 2 or 4) direct loads of one lane pattern: load i reads 16 bytes per lane at g[i] + voff
// into LDS m0 + 1024-byte slot, m0 = lds0 + i * lstride. M0 is saved once and restored once for the
// run (one load per M0 write, with the one wait state an M0 write needs before a direct load). The
// M0 additions write SCC, so SCC is declared clobbered: a 64-bit address add split around the run
// must not take its carry from them.
template <int N>
__device__ __forceinline__ void dma16_run(const char *const (&g)[N], uint32_t voff, uint32_t lds0,
                                          uint32_t lstride) {
  uint32_t saved;
  if constexpr (N == 1) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(lds0), "s"(g[0])
        : "memory", "scc");
  } else if constexpr (N == 2) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %4\n\t"
        "s_add_u32 m0, m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %5\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(lds0), "s"(lstride), "s"(g[0]), "s"(g[1])
        : "memory", "scc");
  } else {
    static_assert(N == 4, "runs of 1, 2 or 4 loads");
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %4\n\t"
        "s_add_u32 m0, m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %5\n\t"
        "s_add_u32 m0, m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %6\n\t"
        "s_add_u32 m0, m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %7\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(lds0), "s"(lstride), "s"(g[0]), "s"(g[1]), "s"(g[2]), "s"(g[3])
        : "memory", "scc");
  }
}

// Wait until at most n of this wave's vector-memory operations are outstanding (n in 0..24; larger
// values wait for all).
__device__ __forceinline__ void wait_vmem(int n) {
  switch (n) {
    case 24: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
    case 23: asm volatile("s_waitcnt vmcnt(23)" ::: "memory"); break;
    case 22: asm volatile("s_waitcnt vmcnt(22)" ::: "memory"); break;
    case 21: asm volatile("s_waitcnt vmcnt(21)" ::: "memory"); break;
    case 20: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
    case 19: asm volatile("s_waitcnt vmcnt(19)" ::: "memory"); break;
    case 18: asm volatile("s_waitcnt vmcnt(18)" ::: "memory"); break;
    case 17: asm volatile("s_waitcnt vmcnt(17)" ::: "memory"); break;
    case 16: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 15: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
    case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
    case 13: asm volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
    case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
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

// ----------------------------------------------------------------------------------------------
// Wave helpers.

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  uint32_t lo = __shfl_xor((uint32_t)v, mask, 64), hi = __shfl_xor((uint32_t)(v >> 32), mask, 64);
  return ((uint64_t)hi << 32) | lo;
}

}  // namespace hs
