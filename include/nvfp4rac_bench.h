/*
 * nvfp4rac_bench.h - ceiling microbenchmarks exported by libnvfp4rac.so for
 * the measurement harness.  They measure, on the chip itself, the sustained
 * rate of the matrix-core instruction families the exact NVFP4 product and
 * its FP8 baseline can run on, and the sustained HBM read rate, so that a
 * kernel's roofline fraction can be read against measured ceilings as well
 * as the data sheet's.  They are not part of the method.
 *
 * Same conventions as nvfp4rac.h: device pointers owned by the caller, work
 * enqueued on `stream`, status codes of nvfp4_status.
 */
#ifndef NVFP4RAC_BENCH_H
#define NVFP4RAC_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  NVFP4_CEIL_F16 = 0,   /* v_mfma_f32_32x32x16_f16                          */
  NVFP4_CEIL_BF16 = 1,  /* v_mfma_f32_32x32x16_bf16                         */
  NVFP4_CEIL_FP8 = 2,   /* v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 x E4M3    */
  NVFP4_CEIL_FP4 = 3    /* v_mfma_scale_f32_32x32x64_f8f6f4, E2M1 x E2M1    */
};

/* Flops of one instruction of the given kind (2 * 32 * 32 * K). */
double nvfp4_ceiling_mfma_flops(int kind);

/* `workgroups` workgroups of four waves; every wave issues iters * 4 MFMAs
 * of the given kind on four independent accumulators.  out [workgroups * 256]
 * float32 receives one value per lane.  Total flops =
 * workgroups * 4 * iters * 4 * nvfp4_ceiling_mfma_flops(kind). */
int nvfp4_ceiling_mfma(int kind, int64_t iters, int64_t workgroups, float* out, void* stream);

/* The f16 (bf16 = 0) or bf16 (bf16 = 1) 32x32x16 MFMA fed with given
 * operand values: operands is 64 lanes x 16 registers x 16 bytes (16 KB of
 * 16-bit values, device memory); lane l takes registers 0..7 as its A and
 * 8..15 as its B operands, and every wave issues iters * 8 MFMAs rotating
 * through them, on four accumulators.  out [workgroups * 256] float32
 * receives one value per lane.  Total flops = workgroups * 4 * iters * 8 *
 * 2 * 32 * 32 * 16.  The matrix cores' sustained rate depends on the
 * operand bits, so this measures the ceiling for the values a GEMM
 * multiplies (e.g. exactly decoded NVFP4 operands). */
int nvfp4_ceiling_mfma_operands(int bf16, const void* operands, int64_t iters, int64_t workgroups,
                                float* out, void* stream);

/* Streaming read of `bytes` (a multiple of 16) from src, 16 bytes per lane
 * per nontemporal load, eight loads in flight per lane; out [1] uint32 is never written
 * for real data (it keeps the loads live). */
int nvfp4_ceiling_read(const void* src, int64_t bytes, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4RAC_BENCH_H */
