// fp32 attention kernels for small head counts and widths (H <= 16,
// Dk <= 128): causal attention with block scores, block-sparse gather and
// sliding-window attention, each with the optional per-head sink (page
// "HySparse MQA sparse attention (FA4 block scoring + SWA MQA + block-sparse
// DSA gather)", section "Core").
//
// One workgroup per query token walks the same 64-key block tiles as the
// bf16 MFMA engine; the contractions are plain fp32 FMAs over LDS-staged
// tiles, so results carry fp32 rounding only (no reduced-precision operand).
#include <hip/hip_runtime.h>

#include "hs_common.h"
#include "hs_kernels.h"

namespace hs {

namespace f32k {
constexpr int MAXH = 16, MAXD = 128, BS = 64, NT = 256, KSTRIDE = MAXD + 1;
constexpr int MAXO = (MAXH * MAXD + NT - 1) / NT;  // output elements per thread
}  // namespace f32k

__device__ __forceinline__ float wsum64(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wmax64(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

template <int OP>
__global__ __launch_bounds__(f32k::NT) void attn_f32_kernel(AttnF32Args a) {
  using namespace f32k;
  __shared__ float qs[MAXH * MAXD];
  __shared__ float ks[BS * KSTRIDE];
  __shared__ float xs[MAXH * BS];
  __shared__ float m_run[MAXH], l_run[MAXH], alpha_s[MAXH], blh[MAXH];
  __shared__ int tile_list[64];
  __shared__ int tile_count;

  const Geom& g = a.g;
  const int H = g.H, Dk = g.Dk, Dv = g.Dv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int w = blockIdx.x;
  const int b = w / g.Sq;
  const int r = g.Sq - 1 - (w % g.Sq);
  const size_t row = (size_t)b * g.Sq + r;
  const RowRange rr = row_range(g, OP, b, r, a.window);
  const int nb_b = nb_of_entry(g, b);

  int ntiles;
  if (OP == kGather) {
    if (wave == 0) {
      int j = -1;
      bool ok = false;
      if (lane < a.top_k) {
        j = a.block_idx[row * a.top_k + lane];
        if (j >= 0 && j < nb_b) {
          const Blk bk = block_rows(g, b, j);
          ok = !(bk.start > rr.hi || bk.start + bk.len - 1 < rr.lo);
        }
      }
      const unsigned long long m = __ballot(ok);
      if (ok) tile_list[__popcll(m & ((1ull << lane) - 1ull))] = j;
      if (lane == 0) tile_count = __popcll(m);
    }
    __syncthreads();
    ntiles = tile_count;
  } else {
    ntiles = rr.j_last - rr.j_first + 1;
  }

  if (OP == kScore) {
    float* blr = a.block_logit + row * g.NB;
    for (int j = tid; j < g.NB; j += NT)
      if (j < rr.j_first || j > rr.j_last) blr[j] = -INFINITY;
  }
  for (int i = tid; i < H * Dk; i += NT) qs[(i / Dk) * MAXD + (i % Dk)] = a.q[row * H * Dk + i];
  if (tid < H) {
    const float sk = a.sink ? a.sink[tid] * kLog2e : -INFINITY;
    m_run[tid] = sk;
    l_run[tid] = sk > -INFINITY ? 1.0f : 0.0f;
  }
  float o[MAXO];
#pragma unroll
  for (int i = 0; i < MAXO; ++i) o[i] = 0.f;

  const float* kv_entry = a.kv + (size_t)b * g.Skv * Dk;
  for (int t = 0; t < ntiles; ++t) {
    const int j = OP == kGather ? tile_list[t] : rr.j_first + t;
    const Blk blk = block_rows(g, b, j);
    __syncthreads();
    for (int i = tid; i < BS * Dk; i += NT) {
      const int k = i / Dk, d = i % Dk;
      const int key = blk.start + min(k, blk.len - 1);
      ks[k * KSTRIDE + d] = kv_entry[(size_t)key * Dk + d];
    }
    __syncthreads();
    for (int i = tid; i < H * BS; i += NT) {
      const int h = i / BS, k = i % BS;
      float s = 0.f;
      for (int d = 0; d < Dk; ++d) s = fmaf(qs[h * MAXD + d], ks[k * KSTRIDE + d], s);
      const int key = blk.start + k;
      const bool ok = k < blk.len && key >= rr.lo && key <= rr.hi;
      xs[i] = ok ? s * g.scale_log2 : -INFINITY;
    }
    __syncthreads();
    for (int h = wave; h < H; h += NT / 64) {
      const float x = xs[h * BS + lane];
      const float mx = wmax64(x);
      const float p = mx == -INFINITY ? 0.f : exp2f(x - mx);
      const float sum = wsum64(p);
      const float m_old = m_run[h];
      const float m_new = fmaxf(m_old, mx);
      const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_old - m_new);
      const float f = mx == -INFINITY ? 0.f : exp2f(mx - m_new);
      xs[h * BS + lane] = p * f;
      if (lane == 0) {
        blh[h] = mx == -INFINITY ? -INFINITY : mx + log2f(sum);
        l_run[h] = l_run[h] * alpha + sum * f;
        m_run[h] = m_new;
        alpha_s[h] = alpha;
      }
    }
    __syncthreads();
    if (OP == kScore && tid == 0) {
      float v = -INFINITY;
      for (int h = 0; h < H; ++h) v = fmaxf(v, blh[h]);
      a.block_logit[row * g.NB + j] = v * kLn2;
    }
#pragma unroll
    for (int i = 0; i < MAXO; ++i) {
      const int e = tid + NT * i;
      if (e < H * Dv) {
        const int h = e / Dv, dv = e % Dv;
        float acc = o[i] * alpha_s[h];
        for (int k = 0; k < BS; ++k) acc = fmaf(xs[h * BS + k], ks[k * KSTRIDE + dv], acc);
        o[i] = acc;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < MAXO; ++i) {
    const int e = tid + NT * i;
    if (e < H * Dv) {
      const int h = e / Dv;
      const float l = l_run[h];
      a.out[row * H * Dv + e] = l > 0.f ? o[i] / l : 0.f;
    }
  }
  if (tid < H) {
    const float l = l_run[tid];
    a.lse[row * H + tid] = l > 0.f ? (m_run[tid] + log2f(l)) * kLn2 : -INFINITY;
  }
}

int attn_f32_launch(int op, const AttnF32Args& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.g.B * a.g.Sq)), block(f32k::NT);
  if (op == kScore) hipLaunchKernelGGL(attn_f32_kernel<kScore>, grid, block, 0, stream, a);
  else if (op == kGather) hipLaunchKernelGGL(attn_f32_kernel<kGather>, grid, block, 0, stream, a);
  else hipLaunchKernelGGL(attn_f32_kernel<kSwa>, grid, block, 0, stream, a);
  return (int)hipGetLastError();
}

}  // namespace hs
