/*
 * moe_probes.h — measurement probes for the MI355X (gfx950) MoE expert-layer library.
 *
 * These are not part of the layer.  They measure the hardware the layer runs on, so that
 * the choices in the layer (which matrix instruction feeds the intermediate requant, what
 * fraction of the matrix-core and HBM peaks is reachable) rest on numbers anyone can
 * re-take:
 *   - moe_probe_mfma_gemm: the result of small GEMMs computed with one matrix-instruction
 *     form, to compare against an exact host dot product (accumulation precision);
 *   - moe_probe_mfma_loop: a timed loop of independent FP8 matrix instructions
 *     (achievable matrix-core rate);
 *   - moe_probe_hbm_read: a timed streaming read (achievable HBM read bandwidth);
 *   - moe_probe_dma_stream: the grouped GEMMs' operand stream without their arithmetic
 *     (direct global-to-LDS loads into a ring of 64 KB stages, per-CU load-path rate from
 *     HBM or from L2-resident data);
 *   - moe_probe_cvt_bf16: the scaled FP8 / FP4 -> BF16 conversions (exactness).
 * The pages this library follows define the efficiency yardstick as useful FLOPs over the
 * kernel's latency, against the chip's peak ("DSV4 o_proj: fuse fp8/UE8M0 quantize into
 * o_a proj", Description: SOL = 2*M*N*K / latency); the probes give the achievable side
 * of that ratio.
 *
 * Conventions: device pointers, caller-owned; asynchronous on `stream` (a hipStream_t,
 * NULL = the null stream); no allocation; a nonzero return is a hipError_t (or -1 for
 * an argument out of range, checked before any launch).
 */
#ifndef MOE_PROBES_H_
#define MOE_PROBES_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Instruction forms of moe_probe_mfma_gemm. */
typedef enum {
  MOE_PROBE_SCALED_32X32X64 = 0,   /* v_mfma_scale_f32_32x32x64_f8f6f4, unit scales, chained in C */
  MOE_PROBE_SCALED_16X16X128 = 1,  /* v_mfma_scale_f32_16x16x128_f8f6f4, unit scales, chained in C */
  MOE_PROBE_FP8_32X32X16 = 2,      /* v_mfma_f32_32x32x16_fp8_fp8 (E4M3 x E4M3 only), chained in C */
  MOE_PROBE_BF16_32X32X16 = 3,     /* operands converted to BF16 in registers (exact), then
                                      v_mfma_f32_32x32x16_bf16, chained in C */
  MOE_PROBE_FP32_FMA = 4,          /* control: exact products summed with fp32 fused multiply-add
                                      in ascending K order */
  MOE_PROBE_SCALED_32X32X64_SPLIT = 5  /* the scaled 32x32x64 instruction from a zero accumulator
                                          per 64-wide K step, the steps added in fp32 */
} moe_probe_form;

/* n problems, each C[p] = A[p] . B[p]^T with A[p] and B[p] of 32 rows by K values:
 *   a  E4M3 codes [n][32][K]
 *   b  E4M3 codes [n][32][K] (b_fp4 = 0) or E2M1 pairs [n][32][K/2], element 2i in the low
 *      nibble of byte i (b_fp4 = 1; not with MOE_PROBE_FP8_32X32X16)
 *   c  float32 [n][32][32], C[p][m][j] = sum_k A[p][m][k] * B[p][j][k]
 * K is a positive multiple of 128; 1 <= n <= 65535.  One wave per problem; all scales 1. */
int moe_probe_mfma_gemm(int form, int n, int K, int b_fp4, const uint8_t* a, const uint8_t* b, float* c,
                        void* stream);

/* Matrix-core rate probe: `blocks` workgroups of 256 threads; every wave issues `iters`
 * rounds of 4 independent v_mfma_scale_f32_32x32x64_f8f6f4 instructions (FP8 x FP8, or
 * FP8 x FP4 when b_fp4 = 1) on register operands and writes one float per lane to sink
 * [blocks * 256].  FLOPs = blocks * 4 waves * iters * 4 * 2 * 32 * 32 * 64.
 * 1 <= blocks <= 2^20, 1 <= iters <= 2^20. */
int moe_probe_mfma_loop(int blocks, int iters, int b_fp4, float* sink, void* stream);

/* HBM read probe: reads `bytes` (a multiple of 16) from src with 16-byte non-temporal
 * loads spread over `blocks` workgroups of 256 threads (grid-stride), and writes one
 * float per thread to sink [blocks * 256].  1 <= blocks <= 2^20. */
int moe_probe_hbm_read(const void* src, size_t bytes, int blocks, float* sink, void* stream);

/* Operand-stream probe: the load path of the grouped GEMMs without their arithmetic.  Each of
 * `blocks` workgroups of 512 threads streams a panel of 512 rows of K bytes (row stride K)
 * into a ring of two 64 KB LDS stages with 16-byte direct global-to-LDS loads, 128 bytes of
 * every row per stage, `passes` times over the panel.  Before each stage is treated as consumed
 * the workgroup waits for it to land and passes a barrier, as the GEMM K loop does.  depth
 * (1 or 2) is the number of stages in flight while the workgroup waits.  The GEMM loop keeps one
 * ahead, because a slot is refilled only after its fragments have been read.
 *   panels = 0: workgroup b streams panel b, so src holds `blocks` panels (data from HBM or the
 *     Infinity Cache, depending on the total size);
 *   panels = n > 0: workgroup b streams panel b % n.  With n = 8, the 32 workgroups of an XCD
 *     share one panel (dispatch is round-robin over the XCDs), which stays in that XCD's L2
 *     after the first pass when 512 K fits there.
 * One float per thread goes to sink [blocks * 512].  Bytes moved = blocks * passes * 512 * K.
 * Limits: K a multiple of 128 in [128, 65536]; src_bytes >= (panels ? panels : blocks) * 512 * K;
 * 1 <= blocks <= 65536; 0 <= panels <= blocks; 1 <= passes <= 65536; depth 1 or 2. */
int moe_probe_dma_stream(const void* src, size_t src_bytes, int K, int blocks, int panels, int passes, int depth,
                         float* sink, void* stream);

/* Scaled conversion probe: out[i] = the BF16 bits the gfx950 scaled conversion instruction
 * gives for code i with scale 2^(scale_bytes[i/32] - 127), passed as the float whose bit
 * pattern is scale_byte << 23 (the denormal 2^-127 for byte 0).  fmt 0: codes are E4M3 bytes
 * [n]; 1: E5M2 bytes [n]; 2: E2M1 pairs [n/2], element 2i in the low nibble of byte i.
 * scale_bytes [n/32]; out uint16 [n]; n a positive multiple of 32, at most 2^28. */
int moe_probe_cvt_bf16(int fmt, int n, const uint8_t* codes, const uint8_t* scale_bytes, uint16_t* out,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBES_H_ */
