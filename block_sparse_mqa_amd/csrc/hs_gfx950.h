// gfx950 building blocks shared by the bf16 attention engine and the gradient
// kernels: vector types, the swizzled LDS layout of a 64-row latent tile, the
// direct-to-LDS copy, and compile-time unrolling.
//
// LDS layout of a 64-row tile of 576 bf16 columns: nine groups of 64 columns;
// group G holds, for each row k, the 128 B of columns 64G .. 64G+63 at
// [G * 8192 + k * 128]. Inside those 128 B, 16-byte chunk c sits in slot
// c ^ sw(k), sw(k) = 3 * bit2(k) + 4 * bit1(k): the 16-byte fragment reads
// of the MFMA operands and the LDS transpose reads are free of bank
// conflicts. A 32-row half tile uses the same layout with a 4096-byte group
// stride.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <utility>

namespace hs {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define HS_LDS __attribute__((address_space(3)))

// Chunk swizzle of row k inside a tile (depends on bits 1 and 2 only).
__device__ __forceinline__ int swz(int k) { return 3 * ((k >> 2) & 1) + 4 * ((k >> 1) & 1); }

// One LDS DMA instruction: lane l copies 16 B from src (per lane) to LDS
// byte lds + 16 l, the LDS base taken from M0 (the compiler sets it from the
// operand; one wait state separates that write from the DMA). Issued as
// inline assembly so that the compiler's wait analysis does not take it for
// an out-of-order LDS operation and drain every LDS read in flight; it is
// counted by vmcnt only, and callers wait for it with s_waitcnt vmcnt.
__device__ __forceinline__ void dma16(const char* src, char* lds) {
  const unsigned m = (unsigned)(uintptr_t)(HS_LDS char*)lds;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m) : "memory");
}

template <typename Fn, int... Is>
__device__ __forceinline__ void static_for_impl(Fn&& fn, std::integer_sequence<int, Is...>) {
  (fn(std::integral_constant<int, Is>{}), ...);
}
// fn(std::integral_constant<int, i>) for i = 0 .. N-1, with i a constant.
template <int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
  static_for_impl(fn, std::make_integer_sequence<int, N>{});
}

// Copy one 64-row tile of 576 bf16 columns (rows base + start .. + len - 1,
// clamped to the last one) into an LDS buffer laid out as above.
// Instruction n = (G, kq) = (n / 8, n % 8) fills rows 8kq .. 8kq+7 of column
// group G; lane l takes row 8kq + l/8 and stores slot l%8, i.e. chunk
// (l%8) ^ sw(row). Wave w issues n = w + 4i, so kq alternates between w and
// w + 4 (same row bit 3) and G = i / 2: two source rows per lane, immediate
// offsets otherwise.
__device__ __forceinline__ void stage_tile(char* buf, const bf16* base, int start, int len,
                                           int wave_u, int lane) {
  constexpr int DK = 576, NGR = 9, GR_BYTES = 64 * 128;
  const int kl = lane >> 3;                                    // row inside the octet
  const int c8 = (lane & 7) ^ swz(8 * wave_u + kl);
  const int ka = min(8 * wave_u + kl, len - 1);               // kq = w
  const int kb = min(8 * (wave_u + 4) + kl, len - 1);         // kq = w + 4
  const char* src_a = (const char*)(base + (size_t)(start + ka) * DK) + 16 * c8;
  const char* src_b = (const char*)(base + (size_t)(start + kb) * DK) + 16 * c8;
  char* dst = buf + wave_u * 1024;
#pragma unroll
  for (int G = 0; G < NGR; ++G) {
    dma16(src_a + 128 * G, dst + G * GR_BYTES);
    dma16(src_b + 128 * G, dst + G * GR_BYTES + 4096);
  }
}

}  // namespace hs
