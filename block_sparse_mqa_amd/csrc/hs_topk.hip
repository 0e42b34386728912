// Per-token top-k block selection (page "HySparse MQA sparse attention (FA4
// block scoring + SWA MQA + block-sparse DSA gather)", per-file overview row
// for pipeline.py: top-k block selection on the block scores, before the
// gather): one wave per row, four rows per workgroup.
#include <hip/hip_runtime.h>

#include "hs_common.h"
#include "hs_kernels.h"
#include "hs_topk_row.h"

namespace hs {

template <int PER>
__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  __shared__ unsigned pack[4][192];   // one packing buffer per wave
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rowi = blockIdx.x * 4 + wave;
  if (rowi >= a.g.B * a.g.Sq) return;
  float lmax2 = 0.f;
  if (a.block_prob != nullptr) {
    float m = -INFINITY;
    for (int h = lane; h < a.g.H; h += 64) m = fmaxf(m, a.lse[(size_t)rowi * a.g.H + h]);
    lmax2 = wave_max_f(m) * kLog2e;
  }
  topk_row<PER>(a.g, a.block_logit, a.block_idx, a.top_k, rowi, lane, pack[wave], a.block_prob,
                lmax2);
}

int topk_launch(const TopkArgs& a, hipStream_t stream) {
  const int rows = a.g.B * a.g.Sq;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  const int NB = a.g.NB;
  if (NB <= 64) hipLaunchKernelGGL(topk_kernel<1>, grid, block, 0, stream, a);
  else if (NB <= 128) hipLaunchKernelGGL(topk_kernel<2>, grid, block, 0, stream, a);
  else if (NB <= 256) hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, stream, a);
  else if (NB <= 512) hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, stream, a);
  else if (NB <= 1024) hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, stream, a);
  else if (NB <= 2048) hipLaunchKernelGGL(topk_kernel<32>, grid, block, 0, stream, a);
  else hipLaunchKernelGGL(topk_kernel<64>, grid, block, 0, stream, a);
  return (int)hipGetLastError();
}

}  // namespace hs
