/*
 * hs_peaks.h -- C ABI of libhspeaks.so: measurement kernels that give the measured ceilings the
 * attention kernels of libhierasparse.so are compared with (the roofline of the sparse KV
 * attention of "HieraSparse: Hierarchical Semi-Structured Sparse KV Attention", §III-D, Eq. (6)-(11),
 * prices decode by bytes and prefill by matrix-core work; these kernels measure what one MI355X
 * delivers of each, and how the softmax's vector work shares a SIMD with the matrix cores).
 *
 * They compute nothing of the method. Every kernel runs a fixed number of loop rounds per wave and
 * writes one value per thread to 'out' (so nothing is optimised away), and wave 0 of workgroup 0
 * stores four uint64 clock samples to 'clk' (NULL = not wanted): the shader clock counter
 * (s_memtime) and the constant 100 MHz counter (s_memrealtime) at its start and at its end, from
 * which the caller derives the shader clock.
 *
 * Every loop kernel reserves 96 KB of LDS, so one workgroup runs per CU: a workgroup of w waves
 * puts w / 4 waves on each SIMD, and 256 workgroups fill the 256 CUs once.
 * Pointers are device pointers owned by the caller; 'out' holds grid * threads floats (or uint32).
 * Work is enqueued on 'stream' (a hipStream_t; NULL = default stream). Return value: 0 on
 * success, -1 for an invalid argument (nothing launched), otherwise the hipError_t of the launch.
 */
#ifndef HS_PEAKS_H
#define HS_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core instruction kinds of hsp_matrix_loop and hsp_mix_wave. */
enum {
  HSP_MFMA_32X32X16 = 0,   /* v_mfma_f32_32x32x16_bf16: 32768 flops per wave instruction */
  HSP_SMFMAC_32X32X32 = 1, /* v_smfmac_f32_32x32x32_bf16: 65536 logical flops (half executed) */
  HSP_MFMA_16X16X32 = 2,   /* v_mfma_f32_16x16x32_bf16: 16384 flops */
  HSP_SMFMAC_16X16X64 = 3  /* v_smfmac_f32_16x16x64_bf16: 32768 logical flops */
};

/* Vector-ALU operations of hsp_valu_loop. */
enum {
  HSP_VALU_EXP2 = 0, /* v_exp_f32 (the softmax exponential) */
  HSP_VALU_FMA = 1,  /* v_fma_f32 */
  HSP_VALU_MAX3 = 2, /* v_max3_f32 */
  HSP_VALU_CVT = 3,  /* v_cvt_pk_bf16_f32 (probabilities packed to bf16) */
  HSP_VALU_SOFTMAX = 4, /* the softmax's per-score mix: per 8 scores 8 FMA, 8 exp, 4 pack, 4 pair
                           sums (v_dot2), 4 max3 */
  HSP_VALU_DOT2 = 5     /* v_dot2c_f32_bf16 (sum of a bf16 pair into an fp32 accumulator) */
};

/* 'iters' rounds of four independent matrix-core instructions of 'kind' per wave; workgroups of
   'waves' waves (1..16), 'grid' workgroups. */
int hsp_matrix_loop(int kind, int grid, int waves, int iters, float *out, uint64_t *clk,
                    void *stream);

/* hsp_matrix_loop with the four instructions of a round spread round-robin over 'accumulators'
   (1 or 2) accumulators, so that each accumulates into the result of the one 1 or 2 instructions
   before it (a dependent chain); 'kind' HSP_MFMA_32X32X16 or HSP_SMFMAC_32X32X32. */
int hsp_matrix_chain(int kind, int accumulators, int grid, int waves, int iters, float *out,
                     uint64_t *clk, void *stream);

/* 'iters' rounds of 'chains' (8 or 16) independent operations 'op' per wave (HSP_VALU_SOFTMAX:
   'chains' scores per round). */
int hsp_valu_loop(int op, int chains, int grid, int waves, int iters, float *out, uint64_t *clk,
                  void *stream);

/* One wave stream holding both: per round four independent v_mfma_f32_32x32x16_bf16 and 'nops'
   independent vector operations 'op' (HSP_VALU_EXP2 or HSP_VALU_FMA; nops in {0, 8, 16, 32, 64}),
   'iters' rounds. */
int hsp_mix_wave(int op, int nops, int grid, int waves, int iters, float *out, uint64_t *clk,
                 void *stream);

/* Two wave kinds on one SIMD: in workgroups of 8 waves (two per SIMD), waves 0-3 run
   'mfma_iters' rounds of hsp_matrix_loop's 32x32x16 loop and waves 4-7 run 'valu_iters' rounds of
   hsp_valu_loop's loop of 'op' (any HSP_VALU_* operation; 8 chains); either count may be 0. */
int hsp_mix_split(int op, int mfma_iters, int valu_iters, int grid, float *out, uint64_t *clk,
                  void *stream);

/* A tile of attention in miniature: every wave of a workgroup of 'waves' (4 or 8: one or two
   per SIMD) runs 'iters' rounds of a matrix phase (eight v_mfma_f32_32x32x16_bf16 over four
   accumulators) followed by a vector phase of 'vrounds' (2, 4 or 8) rounds over 8 chains (FMA and
   exponential rounds in turn) that reads the matrix results, its bf16 pack being the next matrix
   phase's B operand. 'part' 0 runs both phases, 1 the matrix phase only, 2 the vector phase
   only. */
int hsp_mix_phase(int part, int waves, int iters, int vrounds, int grid, float *out, uint64_t *clk,
                  void *stream);

/* LDS read bandwidth: 'iters' rounds of eight ds_read_b128 per wave (1 KB of consecutive bytes
   each, conflict-free) in workgroups of 'waves' waves (1..16). */
int hsp_lds_read(int grid, int waves, int iters, float *out, uint64_t *clk, void *stream);

/* Streaming read of 'bytes' (a multiple of 16 * 64 * 8) from 'src': mode 0 = 16-byte loads into
   registers (nontemporal), each workgroup one contiguous chunk; mode 1 = the same chunks through
   direct global->LDS loads (global_load_lds_dwordx4), the loads the attention kernels stage tiles
   with, default cache policy; mode 2 = mode 1 with the nontemporal policy (the decode's loads).
   Workgroups of 256 threads; out: grid * 256 uint32. */
int hsp_read(int mode, const void *src, size_t bytes, int grid, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* HS_PEAKS_H */
