// hs_peaks.hip -- measurement kernels of libhspeaks.so (include/hs_peaks.h): the measured
// ceilings of one MI355X that the attention kernels are compared with, and how the softmax's
// vector work shares a SIMD with the matrix cores. Nothing of the method is computed here.
//
// Every loop keeps its operands in registers and its rounds independent enough that the unit
// under test, not a dependency chain, sets the pace: four accumulators per wave for the matrix
// cores (a 32x32 accumulator is written back long before its chain issues again), eight chains
// for the vector ALU.
#include <hip/hip_runtime.h>
#include <math.h>

#include "hs_device.h"
#include "hs_peaks.h"

#define HSP_API extern "C" __attribute__((visibility("default")))

namespace {

int status(hipError_t e) { return e == hipSuccess ? 0 : (int)e; }

using hs::f32x16;
using hs::f32x4;

// Every loop kernel holds 96 KB of LDS, so that one workgroup runs per CU and the waves per SIMD
// are the workgroup's waves / 4 (256 workgroups fill the 256 CUs once).
constexpr int kPadFloats = 96 * 1024 / 4;
__device__ __forceinline__ float through_lds(float *pad, float s) {
  pad[threadIdx.x] = s;
  __syncthreads();
  return pad[(threadIdx.x + 1) % blockDim.x];
}

// Clock samples of wave 0 of workgroup 0: shader clock counter and 100 MHz counter.
__device__ __forceinline__ void clock_mark(uint64_t *clk, int i) {
  if (clk && blockIdx.x == 0 && threadIdx.x == 0) {
    const uint64_t t = __builtin_amdgcn_s_memtime();
    const uint64_t r = __builtin_amdgcn_s_memrealtime();
    clk[2 * i] = t;
    clk[2 * i + 1] = r;
  }
}

// Operand registers filled from the thread index (finite bf16 values; the values do not matter).
__device__ __forceinline__ uint4 seed4(int tid, int k) {
  const uint32_t a = 0x3F80u + ((tid + k) & 7), b = 0x3F00u + ((tid * 3 + k) & 7);
  const uint32_t w = a | (b << 16);
  return make_uint4(w, w ^ 0x00010000u, w ^ 1u, w);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// NACC accumulators per wave, used round-robin: with one, every instruction accumulates into the
// result of the one before it (a dependent chain).
template <int KIND, int NACC = 4>
__device__ __forceinline__ float matrix_rounds(int iters, int tid) {
  const uint4 a = seed4(tid, 1), b0 = seed4(tid, 2), b1 = seed4(tid, 3);
  const uint32_t idx = 0x44444444u;  // 2:4 positions 0 and 1 of every group
  float s = 0.f;
  if constexpr (KIND == HSP_MFMA_32X32X16 || KIND == HSP_SMFMAC_32X32X32) {
    f32x16 acc[NACC];
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = zero16();
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = k % NACC;
        if constexpr (KIND == HSP_MFMA_32X32X16)
          acc[j] = hs::mma32x16(hs::as8<__bf16>(a), hs::as8<__bf16>(b0), acc[j]);
        else
          acc[j] = hs::smma32x32<0>(hs::as8<__bf16>(a), hs::as16<__bf16>(b0, b1), acc[j],
                                    (int)idx);
      }
    }
#pragma unroll
    for (int j = 0; j < NACC; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[j][e];
  } else {
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (KIND == HSP_MFMA_16X16X32)
          acc[j] = hs::mfma16<__bf16>(a, b0, acc[j]);
        else
          acc[j] = hs::smfmac16<__bf16>(a, b0, b1, idx, acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) s += acc[j][e];
  }
  return s;
}

template <int KIND, int NACC = 4>
__global__ __launch_bounds__(1024) void k_matrix_loop(float *out, int iters, uint64_t *clk) {
  __shared__ float pad[kPadFloats];
  clock_mark(clk, 0);
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  out[tid] = through_lds(pad, matrix_rounds<KIND, NACC>(iters, threadIdx.x));
  clock_mark(clk, 1);
}

// One vector operation on one chain value. c1, c2 are kernel arguments, so nothing folds.
template <int OP>
__device__ __forceinline__ float valu_op(float x, float c1, float c2) {
  if constexpr (OP == HSP_VALU_EXP2) return __builtin_amdgcn_exp2f(-fabsf(x));
  if constexpr (OP == HSP_VALU_FMA) return fmaf(x, c1, c2);
  if constexpr (OP == HSP_VALU_MAX3) return fmaxf(fmaxf(x, c1), c2);
  if constexpr (OP == HSP_VALU_DOT2) return hs::add_pair_bits<__bf16>(__float_as_uint(c2), x);
  return __uint_as_float(hs::pack2<__bf16>(c1, x));  // OP == HSP_VALU_CVT
}

// NCH independent chains per wave, 8 operations per round and chain group: plain operations
// ('iters' rounds of eight), or the softmax's per-score mix (HSP_VALU_SOFTMAX: per eight scores
// eight FMAs, eight exponentials, four bf16 packs, four pair sums and four max3).
template <int OP, int NCH>
__device__ __forceinline__ float valu_rounds(int iters, int tid, float c1, float c2) {
  float x[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) x[j] = 0.25f + 0.01f * (float)((tid + j) & 15);
  if constexpr (OP == HSP_VALU_SOFTMAX) {
    float sum = 0.f, mx = 0.f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j0 = 0; j0 < NCH; j0 += 8) {
#pragma unroll
        for (int j = j0; j < j0 + 8; ++j) x[j] = __builtin_amdgcn_exp2f(fmaf(-fabsf(x[j]), c1, -c2));
#pragma unroll
        for (int j = j0; j < j0 + 8; j += 2) {
          const uint32_t pk = hs::pack2<__bf16>(x[j], x[j + 1]);
          sum = hs::add_pair_bits<__bf16>(pk, sum);
          mx = fmaxf(fmaxf(mx, x[j]), x[j + 1]);
        }
      }
    }
    return sum + mx + x[0];
  } else {
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int j = 0; j < NCH; ++j) x[j] = valu_op<OP>(x[j], c1, c2);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) s += x[j];
    return s;
  }
}

template <int OP, int NCH>
__global__ __launch_bounds__(1024) void k_valu_loop(float *out, int iters, float c1, float c2,
                                                    uint64_t *clk) {
  __shared__ float pad[kPadFloats];
  clock_mark(clk, 0);
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  out[tid] = through_lds(pad, valu_rounds<OP, NCH>(iters, threadIdx.x, c1, c2));
  clock_mark(clk, 1);
}

// Four 32x32x16 MFMAs and NEXP vector operations OP (exponential or FMA) per round in one wave.
template <int OP, int NEXP>
__global__ __launch_bounds__(1024) void k_mix_wave(float *out, int iters, float c1, float c2,
                                                   uint64_t *clk) {
  __shared__ float pad[kPadFloats];
  clock_mark(clk, 0);
  const int t = threadIdx.x, tid = blockIdx.x * blockDim.x + t;
  const uint4 a = seed4(t, 1), b = seed4(t, 2);
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = zero16();
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = 0.25f + 0.01f * (float)((t + j) & 15);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[j] = hs::mma32x16(hs::as8<__bf16>(a), hs::as8<__bf16>(b), acc[j]);
#pragma unroll
      for (int e = 0; e < NEXP / 4; ++e) {
        const int c = (j * (NEXP / 4) + e) & 7;
        x[c] = valu_op<OP>(x[c], c1, c2);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x[j];
  out[tid] = through_lds(pad, s);
  clock_mark(clk, 1);
}

// Waves 0-3 matrix loop, waves 4-7 vector loop OP (two waves per SIMD).
template <int OP>
__global__ __launch_bounds__(512) void k_mix_split(float *out, int mfma_iters, int exp_iters,
                                                   float c1, float c2, uint64_t *clk) {
  __shared__ float pad[kPadFloats];
  clock_mark(clk, 0);
  const int t = threadIdx.x, tid = blockIdx.x * blockDim.x + t;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const float s = wave < 4 ? matrix_rounds<HSP_MFMA_32X32X16>(mfma_iters, t)
                           : valu_rounds<OP, 8>(exp_iters, t, c1, c2);
  out[tid] = through_lds(pad, s);
  clock_mark(clk, 1);
}

// Each wave alternates a matrix phase (eight 32x32x16 MFMAs over four accumulators) and a vector
// phase (8 chains, VR / 2 pairs of an FMA round and an exponential round) that depends on the
// matrix results, whose bf16 pack feeds the next matrix phase, as a tile of attention does (GEMM,
// softmax, GEMM). PART 0: both phases; 1: the matrix phase only; 2: the vector phase only.
template <int PART, int VR>
__global__ __launch_bounds__(512) void k_mix_phase(float *out, int iters, float c1, float c2,
                                                   uint64_t *clk) {
  __shared__ float pad[kPadFloats];
  clock_mark(clk, 0);
  const int t = threadIdx.x, tid = blockIdx.x * blockDim.x + t;
  const uint4 a = seed4(t, 1);
  uint4 b = seed4(t, 2);
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = zero16();
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = 0.25f + 0.01f * (float)((t + j) & 15);
  for (int i = 0; i < iters; ++i) {
    if constexpr (PART != 2) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        acc[k & 3] = hs::mma32x16(hs::as8<__bf16>(a), hs::as8<__bf16>(b), acc[k & 3]);
    }
    if constexpr (PART != 1) {
#pragma unroll
      for (int c = 0; c < 8; ++c) x[c] = fmaf(acc[c & 3][c], 1e-6f, x[c]);
#pragma unroll
      for (int r = 0; r < VR / 2; ++r) {
#pragma unroll
        for (int c = 0; c < 8; ++c) x[c] = fmaf(x[c], c1, c2);
#pragma unroll
        for (int c = 0; c < 8; ++c) x[c] = __builtin_amdgcn_exp2f(-fabsf(x[c]));
      }
      b.x = hs::pack2<__bf16>(x[0], x[1]);
      b.y = hs::pack2<__bf16>(x[2], x[3]);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x[j];
  out[tid] = through_lds(pad, s);
  clock_mark(clk, 1);
}

// LDS read bandwidth: every wave streams ds_read_b128 over a 64 KB window (each wave instruction
// reads 1 KB of consecutive bytes, conflict-free), eight reads in flight; the values are only
// made live (an empty asm statement takes them), so no vector arithmetic shares the issue slots.
typedef uint32_t lds_u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(1024) void k_lds_read(float *out, int iters, uint64_t *clk) {
  __shared__ __attribute__((aligned(16))) lds_u32x4 buf[kPadFloats / 4];
  const int t = threadIdx.x;
  for (int i = t; i < kPadFloats / 4; i += blockDim.x) buf[i] = lds_u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  clock_mark(clk, 0);
  // eight fixed addresses per lane, 8 KB apart (t + 512 u < 6144 entries); the lane's index
  // passes through an empty asm statement every round, so the reads cannot be hoisted out of the
  // loop, and the 8 KB steps fold into the instructions' offset fields
  int idx = t;
  for (int it = 0; it < iters; ++it) {
    asm volatile("" : "+v"(idx));
    lds_u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = buf[idx + 512 * u];
#pragma unroll
    for (int u = 0; u < 8; ++u) asm volatile("" ::"v"(v[u].x), "v"(v[u].y), "v"(v[u].z), "v"(v[u].w));
  }
  __syncthreads();
  out[blockIdx.x * blockDim.x + t] = 0.f;
  clock_mark(clk, 1);
}

// Streaming reads: workgroup g reads bytes [g * chunk, (g + 1) * chunk); chunk % 32 KB == 0.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void k_read_regs(const u32x4 *src, size_t chunk16,
                                                   uint32_t *out) {
  const u32x4 *p = src + (size_t)blockIdx.x * chunk16;
  uint32_t acc = 0;
  for (size_t i = threadIdx.x; i < chunk16; i += 256 * 8) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + i + 256 * u);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// Direct loads into LDS: each wave keeps two batches of eight 1 KB loads in flight (16 KB of LDS
// per wave, never read).
template <bool kNT>
__global__ __launch_bounds__(256) void k_read_lds(const char *src, size_t chunk, uint32_t *out) {
  __shared__ __attribute__((aligned(1024))) char lds[4 * 16384];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lds_base = (uint32_t)(size_t)(__attribute__((address_space(3))) char *)lds;
  const char *base = src + (size_t)blockIdx.x * chunk + wave * 1024;
  int half = 0;
  for (size_t off = 0; off < chunk; off += 32768) {
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if constexpr (kNT)
        hs::dma16_nt(hs::uniform_ptr(base + off + 4096 * u), 16 * lane,
                     lds_base + wave * 16384 + half * 8192 + 1024 * u);
      else
        hs::dma16(hs::uniform_ptr(base + off + 4096 * u), 16 * lane,
                  lds_base + wave * 16384 + half * 8192 + 1024 * u);
    half ^= 1;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = 0u;
}

}  // namespace

HSP_API int hsp_matrix_loop(int kind, int grid, int waves, int iters, float *out, uint64_t *clk,
                            void *stream) {
  if (!out || grid <= 0 || waves < 1 || waves > 16 || iters < 0) return -1;
  const dim3 g(grid), b(64 * waves);
  hipStream_t s = (hipStream_t)stream;
  switch (kind) {
    case HSP_MFMA_32X32X16: k_matrix_loop<HSP_MFMA_32X32X16><<<g, b, 0, s>>>(out, iters, clk); break;
    case HSP_SMFMAC_32X32X32: k_matrix_loop<HSP_SMFMAC_32X32X32><<<g, b, 0, s>>>(out, iters, clk); break;
    case HSP_MFMA_16X16X32: k_matrix_loop<HSP_MFMA_16X16X32><<<g, b, 0, s>>>(out, iters, clk); break;
    case HSP_SMFMAC_16X16X64: k_matrix_loop<HSP_SMFMAC_16X16X64><<<g, b, 0, s>>>(out, iters, clk); break;
    default: return -1;
  }
  return status(hipGetLastError());
}

HSP_API int hsp_matrix_chain(int kind, int accumulators, int grid, int waves, int iters,
                             float *out, uint64_t *clk, void *stream) {
  if (!out || grid <= 0 || waves < 1 || waves > 16 || iters < 0) return -1;
  const dim3 g(grid), b(64 * waves);
  hipStream_t s = (hipStream_t)stream;
  if (kind == HSP_MFMA_32X32X16) {
    if (accumulators == 1) k_matrix_loop<HSP_MFMA_32X32X16, 1><<<g, b, 0, s>>>(out, iters, clk);
    else if (accumulators == 2) k_matrix_loop<HSP_MFMA_32X32X16, 2><<<g, b, 0, s>>>(out, iters, clk);
    else return -1;
  } else if (kind == HSP_SMFMAC_32X32X32) {
    if (accumulators == 1) k_matrix_loop<HSP_SMFMAC_32X32X32, 1><<<g, b, 0, s>>>(out, iters, clk);
    else if (accumulators == 2) k_matrix_loop<HSP_SMFMAC_32X32X32, 2><<<g, b, 0, s>>>(out, iters, clk);
    else return -1;
  } else {
    return -1;
  }
  return status(hipGetLastError());
}

template <int NCH>
int valu_loop(int op, dim3 g, dim3 b, int iters, float *out, uint64_t *clk, hipStream_t s) {
  const float c1 = 0.99990f, c2 = 1e-4f;
  switch (op) {
    case HSP_VALU_EXP2: k_valu_loop<HSP_VALU_EXP2, NCH><<<g, b, 0, s>>>(out, iters, c1, c2, clk); break;
    case HSP_VALU_FMA: k_valu_loop<HSP_VALU_FMA, NCH><<<g, b, 0, s>>>(out, iters, c1, c2, clk); break;
    case HSP_VALU_MAX3: k_valu_loop<HSP_VALU_MAX3, NCH><<<g, b, 0, s>>>(out, iters, c1, c2, clk); break;
    case HSP_VALU_CVT: k_valu_loop<HSP_VALU_CVT, NCH><<<g, b, 0, s>>>(out, iters, c1, c2, clk); break;
    case HSP_VALU_SOFTMAX: k_valu_loop<HSP_VALU_SOFTMAX, NCH><<<g, b, 0, s>>>(out, iters, c1, c2, clk); break;
    case HSP_VALU_DOT2: k_valu_loop<HSP_VALU_DOT2, NCH><<<g, b, 0, s>>>(out, iters, c1, c2, clk); break;
    default: return -1;
  }
  return status(hipGetLastError());
}

HSP_API int hsp_valu_loop(int op, int chains, int grid, int waves, int iters, float *out,
                          uint64_t *clk, void *stream) {
  if (!out || grid <= 0 || waves < 1 || waves > 16 || iters < 0) return -1;
  const dim3 g(grid), b(64 * waves);
  hipStream_t s = (hipStream_t)stream;
  if (chains == 8) return valu_loop<8>(op, g, b, iters, out, clk, s);
  if (chains == 16) return valu_loop<16>(op, g, b, iters, out, clk, s);
  return -1;
}

template <int OP>
int mix_wave(int nops, dim3 g, dim3 b, int iters, float *out, uint64_t *clk, hipStream_t s) {
  const float c1 = 0.99990f, c2 = 1e-4f;
  switch (nops) {
    case 0: k_mix_wave<OP, 0><<<g, b, 0, s>>>(out, iters, c1, c2, clk); break;
    case 8: k_mix_wave<OP, 8><<<g, b, 0, s>>>(out, iters, c1, c2, clk); break;
    case 16: k_mix_wave<OP, 16><<<g, b, 0, s>>>(out, iters, c1, c2, clk); break;
    case 32: k_mix_wave<OP, 32><<<g, b, 0, s>>>(out, iters, c1, c2, clk); break;
    case 64: k_mix_wave<OP, 64><<<g, b, 0, s>>>(out, iters, c1, c2, clk); break;
    default: return -1;
  }
  return status(hipGetLastError());
}

HSP_API int hsp_mix_wave(int op, int nops, int grid, int waves, int iters, float *out,
                         uint64_t *clk, void *stream) {
  if (!out || grid <= 0 || waves < 1 || waves > 16 || iters < 0) return -1;
  const dim3 g(grid), b(64 * waves);
  hipStream_t s = (hipStream_t)stream;
  if (op == HSP_VALU_EXP2) return mix_wave<HSP_VALU_EXP2>(nops, g, b, iters, out, clk, s);
  if (op == HSP_VALU_FMA) return mix_wave<HSP_VALU_FMA>(nops, g, b, iters, out, clk, s);
  return -1;
}

HSP_API int hsp_mix_split(int op, int mfma_iters, int valu_iters, int grid, float *out,
                          uint64_t *clk, void *stream) {
  if (!out || grid <= 0 || mfma_iters < 0 || valu_iters < 0) return -1;
  hipStream_t s = (hipStream_t)stream;
  const float c1 = 0.99990f, c2 = 1e-4f;
  switch (op) {
    case HSP_VALU_EXP2: k_mix_split<HSP_VALU_EXP2><<<grid, 512, 0, s>>>(out, mfma_iters, valu_iters, c1, c2, clk); break;
    case HSP_VALU_FMA: k_mix_split<HSP_VALU_FMA><<<grid, 512, 0, s>>>(out, mfma_iters, valu_iters, c1, c2, clk); break;
    case HSP_VALU_SOFTMAX: k_mix_split<HSP_VALU_SOFTMAX><<<grid, 512, 0, s>>>(out, mfma_iters, valu_iters, c1, c2, clk); break;
    case HSP_VALU_MAX3: k_mix_split<HSP_VALU_MAX3><<<grid, 512, 0, s>>>(out, mfma_iters, valu_iters, c1, c2, clk); break;
    case HSP_VALU_CVT: k_mix_split<HSP_VALU_CVT><<<grid, 512, 0, s>>>(out, mfma_iters, valu_iters, c1, c2, clk); break;
    case HSP_VALU_DOT2: k_mix_split<HSP_VALU_DOT2><<<grid, 512, 0, s>>>(out, mfma_iters, valu_iters, c1, c2, clk); break;
    default: return -1;
  }
  return status(hipGetLastError());
}

HSP_API int hsp_mix_phase(int part, int waves, int iters, int vrounds, int grid, float *out,
                          uint64_t *clk, void *stream) {
  if (!out || grid <= 0 || (waves != 4 && waves != 8) || iters < 0 || part < 0 || part > 2)
    return -1;
  hipStream_t s = (hipStream_t)stream;
  const float c1 = 0.99990f, c2 = 1e-4f;
  const dim3 g(grid), b(64 * waves);
  switch (part * 16 + vrounds) {
    case 2: k_mix_phase<0, 2><<<g, b, 0, s>>>(out, iters, c1, c2, clk); break;
    case 4: k_mix_phase<0, 4><<<g, b, 0, s>>>(out, iters, c1, c2, clk); break;
    case 8: k_mix_phase<0, 8><<<g, b, 0, s>>>(out, iters, c1, c2, clk); break;
    case 18: k_mix_phase<1, 2><<<g, b, 0, s>>>(out, iters, c1, c2, clk); break;
    case 20: k_mix_phase<1, 4><<<g, b, 0, s>>>(out, iters, c1, c2, clk); break;
    case 24: k_mix_phase<1, 8><<<g, b, 0, s>>>(out, iters, c1, c2, clk); break;
    case 34: k_mix_phase<2, 2><<<g, b, 0, s>>>(out, iters, c1, c2, clk); break;
    case 36: k_mix_phase<2, 4><<<g, b, 0, s>>>(out, iters, c1, c2, clk); break;
    case 40: k_mix_phase<2, 8><<<g, b, 0, s>>>(out, iters, c1, c2, clk); break;
    default: return -1;
  }
  return status(hipGetLastError());
}

HSP_API int hsp_lds_read(int grid, int waves, int iters, float *out, uint64_t *clk,
                         void *stream) {
  if (!out || grid <= 0 || waves < 1 || waves > 16 || iters < 0) return -1;
  k_lds_read<<<grid, 64 * waves, 0, (hipStream_t)stream>>>(out, iters, clk);
  return status(hipGetLastError());
}

HSP_API int hsp_read(int mode, const void *src, size_t bytes, int grid, uint32_t *out,
                     void *stream) {
  if (!src || !out || grid <= 0 || bytes % ((size_t)grid * 32768) != 0 || bytes == 0) return -1;
  if (((uintptr_t)src & 15) != 0) return -1;
  const size_t chunk = bytes / grid;
  hipStream_t s = (hipStream_t)stream;
  if (mode == 0)
    k_read_regs<<<grid, 256, 0, s>>>((const u32x4 *)src, chunk / 16, out);
  else if (mode == 1)
    k_read_lds<false><<<grid, 256, 0, s>>>((const char *)src, chunk, out);
  else if (mode == 2)
    k_read_lds<true><<<grid, 256, 0, s>>>((const char *)src, chunk, out);
  else
    return -1;
  return status(hipGetLastError());
}
