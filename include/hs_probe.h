/* Measurement probes for the MI355X rooflines (libhsprobe.so).
 *
 * These two kernels measure the machine, not the method: the attainable dense
 * bf16 MFMA rate and the attainable HBM copy rate on the GPU they run on.
 * Attention kernels are reported against these rates and against the vendor
 * peaks (2.5 PFLOP/s dense bf16, 8 TB/s HBM).
 *
 * Conventions: plain pointers to caller-owned device memory; the stream is a
 * hipStream_t passed as void* (NULL = default stream); calls are
 * asynchronous and never synchronise. Return 0 on success, -1 for an invalid
 * argument (checked on the host before any launch), -3 when the launch
 * reports a HIP error.
 */
#ifndef HS_PROBE_H
#define HS_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Dense MFMA loop: `workgroups` workgroups of 256 lanes (4 waves) each run
 * `iters` iterations of 4 independent v_mfma_f32_32x32x16_bf16 chains with
 * register operands (the shape that reaches the dense bf16 peak with few
 * chains), then write one float per lane to `out`
 * (device, float[workgroups * 256], 4-byte aligned). The launch performs
 * hs_probe_mfma_flops(workgroups, iters) floating-point operations.
 * workgroups in [1, 1 << 20], iters in [1, 1 << 24].
 * `clocks` (device, uint64[2], 8-byte aligned, or NULL): workgroup 0 writes
 * the shader-clock cycles and the 100 MHz reference-clock ticks that elapsed
 * around its loop, so cycles / (ticks / 1e8) is the shader clock in Hz while
 * the loop ran (with enough workgroups to fill the GPU at once). */
int hs_probe_mfma_bf16(int32_t workgroups, int32_t iters, float* out, uint64_t* clocks,
                       void* stream);

/* Floating-point operations of one hs_probe_mfma_bf16 launch:
 * workgroups * 4 waves * iters * 4 * (32 * 32 * 16 * 2). Host only. */
double hs_probe_mfma_flops(int32_t workgroups, int32_t iters);

/* Streaming copy of `bytes` bytes from `src` to `dst` (device, 16-byte
 * aligned, not overlapping); bytes must be a positive multiple of 16. The
 * launch reads `bytes` and writes `bytes`. */
int hs_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HS_PROBE_H */
