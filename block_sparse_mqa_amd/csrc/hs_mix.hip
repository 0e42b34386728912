// Gated sum of the two branch outputs of a sliding-window layer, for the
// launches that run the branches separately (split decode, paged KV, fp32
// shapes); the one-pass kernel forms the same sum in its epilogue with the
// same operations (gated_mix). The combination rule is a reading: the page
// "HySparse MQA sparse attention (FA4 block scoring + SWA MQA + block-sparse
// DSA gather)" calls the method NSA-style (section "What") and leaves the rule
// unstated; NSA combines its branches by a gated sum with gates the model
// computes per token and head, which the caller passes here.
#include <hip/hip_runtime.h>

#include "hs_kernels.h"

namespace hs {

typedef __bf16 mix_bf16x4 __attribute__((ext_vector_type(4)));

// bf16 (Dv a multiple of 4): one thread per 4 consecutive columns of one
// (row, head); fp32 (any Dv): one thread per element.
template <bool BF16>
__global__ __launch_bounds__(256) void mix_kernel(MixArgs m) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const int per = BF16 ? m.dv / 4 : m.dv;
  if (i >= m.rows * per) return;
  const long long rh = i / per;
  const float ga = m.ga[rh], gb = m.gb[rh];
  if constexpr (BF16) {
    const mix_bf16x4 x = ((const mix_bf16x4*)m.a)[i];
    const mix_bf16x4 y = ((const mix_bf16x4*)m.b)[i];
    mix_bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (__bf16)gated_mix(ga, (float)x[e], gb, (float)y[e]);
    ((mix_bf16x4*)m.out)[i] = o;
  } else {
    ((float*)m.out)[i] = gated_mix(ga, ((const float*)m.a)[i], gb, ((const float*)m.b)[i]);
  }
}

int mix_launch(const MixArgs& m, hipStream_t stream) {
  const long long n = m.rows * (m.bf16 ? m.dv / 4 : m.dv);
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (m.bf16) hipLaunchKernelGGL(mix_kernel<true>, grid, block, 0, stream, m);
  else hipLaunchKernelGGL(mix_kernel<false>, grid, block, 0, stream, m);
  return (int)hipGetLastError();
}

}  // namespace hs
