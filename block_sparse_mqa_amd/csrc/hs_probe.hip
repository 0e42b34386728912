// Roofline probes: the attainable dense bf16 MFMA rate and the attainable
// HBM copy rate of the GPU they run on. They measure the machine; nothing in
// the attention path calls them.
#include <hip/hip_runtime.h>

#include "hs_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Four independent accumulators of v_mfma_f32_32x32x16_bf16 per wave, each in
// its own named registers (an array of accumulators lets the compiler rotate
// registers through copies every iteration, which measures the copies).
#define HS_PROBE_MFMA(c) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0)

__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* out,
                                                        unsigned long long* clocks) {
  // shader-clock cycles and 100 MHz reference ticks around the loop, read
  // once by workgroup 0 (all workgroups are resident together)
  unsigned long long c0 = 0, r0 = 0;
  if (clocks != nullptr && blockIdx.x == 0) {
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)threadIdx.x + 0.25f * (float)i);
    b[i] = (__bf16)(0.5f - 0.0625f * (float)i);
  }
  f32x16 acc0, acc1, acc2, acc3;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc0[i] = acc1[i] = acc2[i] = acc3[i] = 0.f;
  for (int it = 0; it < iters; ++it) {
    HS_PROBE_MFMA(acc0);
    HS_PROBE_MFMA(acc1);
    HS_PROBE_MFMA(acc2);
    HS_PROBE_MFMA(acc3);
  }
  const f32x16 t = acc0 + acc1 + acc2 + acc3;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += t[i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (clocks != nullptr && blockIdx.x == 0 && threadIdx.x == 0) {
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    clocks[0] = c1 - c0;
    clocks[1] = r1 - r0;
  }
}

// 16 bytes per lane per access, four accesses in flight per lane, streaming
// (nontemporal) loads and stores: the fastest of the plain, unrolled and
// nontemporal forms tried on gfx950.
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(&src[i + u * stride]);
#pragma unroll
    for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], &dst[i + u * stride]);
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" {

int hs_probe_mfma_bf16(int32_t workgroups, int32_t iters, float* out, uint64_t* clocks,
                       void* stream) {
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 24) || out == nullptr ||
      ((uintptr_t)out & 3u) != 0 || ((uintptr_t)clocks & 7u) != 0)
    return -1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)workgroups), dim3(256), 0,
                     (hipStream_t)stream, (int)iters, out, (unsigned long long*)clocks);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

double hs_probe_mfma_flops(int32_t workgroups, int32_t iters) {
  return (double)workgroups * 4.0 * (double)iters * 4.0 * (32.0 * 32.0 * 16.0 * 2.0);
}

int hs_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (src == nullptr || dst == nullptr || bytes == 0 || (bytes & 15u) != 0 ||
      ((uintptr_t)src & 15u) != 0 || ((uintptr_t)dst & 15u) != 0)
    return -1;
  const uintptr_t s = (uintptr_t)src, d = (uintptr_t)dst;
  if (s < d + bytes && d < s + bytes) return -1;  // overlapping
  const size_t n = bytes / 16;
  const size_t want = (n + 255) / 256;
  const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)src, (u32x4*)dst, n);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
