// Kernel argument blocks and launchers of the forward kernels, used by the C
// ABI (hs_abi.hip); the gradient kernels' are in hs_bwd_args.h.
#pragma once

#include <hip/hip_runtime.h>

#include "hs_common.h"

namespace hs {

// Arguments of the attention kernels (both dtypes; q/kv/out are typed by the
// launcher). Passed by value.
struct AttnArgs {
  const __bf16* q;
  const __bf16* kv;
  const float* sink;         // [H] or nullptr
  __bf16* out;
  float* lse;
  float* block_logit;        // score operation only
  const int* block_idx;      // gather operation only
  __bf16* out2;              // window-and-sparse operation: the window branch's out
  float* lse2;               // and lse (out / lse hold the sparse branch's)
  const float* gate_a;       // window-and-sparse: optional gated sum of the branches,
  const float* gate_b;       // out_mix = gate_a * out2 + gate_b * out ([B, Sq, H] gates)
  __bf16* out_mix;
  int top_k;
  int window;
  int nsplit;                // > 1: split key range, partials merged after
  int split_tiles;           // tiles per split: split s covers [s, s+1) * split_tiles
  float* ws_o;               // [items * nsplit, H, Dv] fp32 partial O
  float* ws_ml;              // [items * nsplit, H, 2] fp32 (max, denominator)
  const int* page_table;     // [B, max_pages] page of each key block, or nullptr
  int max_pages;
  int* topk_idx;             // score operation: [B, Sq, topk_k] selection, or nullptr
  int topk_k;
  float* topk_prob;          // score operation: [B, Sq, NB] normalised block scores, or nullptr
  Geom g;
};

struct AttnF32Args {
  const float* q;
  const float* kv;
  const float* sink;
  float* out;
  float* lse;
  float* block_logit;
  const int* block_idx;
  int top_k;
  int window;
  Geom g;
};

// Gated sum of two attention outputs of one shape: out = ga * a + gb * b per
// (row, head), elementwise over Dv (the window-and-sparse call's combination
// when its branches run as separate launches).
struct MixArgs {
  const void* a;
  const void* b;
  const float* ga;
  const float* gb;
  void* out;
  long long rows;            // B * Sq * H
  int dv;
  int bf16;                  // 1: bf16 tensors, 0: fp32
};

struct TopkArgs {
  const float* block_logit;  // [B, Sq, NB]
  int* block_idx;            // [B, Sq, top_k]
  int top_k;
  const float* lse;          // [B, Sq, H]: read when block_prob is set
  float* block_prob;         // [B, Sq, NB] normalised block scores, or nullptr
  Geom g;
};

int attn_bf16_launch(int op, const AttnArgs& a, hipStream_t stream);
int attn_f32_launch(int op, const AttnF32Args& a, hipStream_t stream);
int topk_launch(const TopkArgs& a, hipStream_t stream);
int mix_launch(const MixArgs& a, hipStream_t stream);

// One element of the gated sum, the same operations wherever it is formed.
__device__ __forceinline__ float gated_mix(float ga, float a, float gb, float b) {
  return fmaf(gb, b, __fmul_rn(ga, a));
}

}  // namespace hs
