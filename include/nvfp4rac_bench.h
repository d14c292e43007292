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

/* Streaming read of `bytes` (a multiple of 16) from src, 16 bytes per lane
 * per nontemporal load, eight loads in flight per lane; out [1] uint32 is never written
 * for real data (it keeps the loads live). */
int nvfp4_ceiling_read(const void* src, int64_t bytes, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4RAC_BENCH_H */
