// Per-token top-k block selection of one row by one wave (page "HySparse MQA
// sparse attention (FA4 block scoring + SWA MQA + block-sparse DSA gather)",
// per-file overview row for pipeline.py: top-k block selection on the block
// scores, before the gather). Used by the top-k kernel and, for split decode,
// by the merge kernel of the attention engine.
//
// Candidates are the finite scores. When there are more than top_k, the row's
// own block is kept and the other top_k-1 (or top_k if the own block is not a
// candidate) are the best by (score descending, index ascending). The k-th
// best value is found exactly by a 32-step bitwise search over
// order-preserving uint32 keys of the fp32 scores; entries above it are taken,
// and ties at it are taken in ascending index order until the count is
// reached. The final scan runs in index order, so the output is already
// ascending; it is padded with -1.
#pragma once

#include <hip/hip_runtime.h>

#include "hs_common.h"

namespace hs {

// Order-preserving map of a non-NaN float to uint32 (+0 and -0 map equal).
__device__ __forceinline__ unsigned ord_key(float v) {
  unsigned u = __float_as_uint(v);
  if (v == 0.f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int wave_sum_i(int v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Top-k of row rowi (= b * Sq + r) by one wave; PER = ceil(NB / 64) values
// per lane.
template <int PER>
__device__ __forceinline__ void topk_row(const Geom& g, const float* block_logit, int* block_idx,
                                         int top_k, int rowi, int lane) {
  const int b = rowi / g.Sq, r = rowi % g.Sq;
  const int pos = kv_len_of<true>(g, b) - g.Sq + r;
  const Doc d = doc_of_pos<true>(g, b, pos);
  const int own = block_of_pos(g, d, pos);
  const int K = top_k;
  const float* bl = block_logit + (size_t)rowi * g.NB;
  int* outp = block_idx + (size_t)rowi * K;

  unsigned key[PER];
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = lane + 64 * i;
    const float v = j < g.NB ? bl[j] : -INFINITY;
    const bool cand = v > -INFINITY;
    key[i] = cand ? ord_key(v) : 0u;
    cnt += cand ? 1 : 0;
  }
  cnt = wave_sum_i(cnt);

  const bool all = cnt <= K;
  bool force_own = false;
  unsigned T = 0u;
  int take_ties = 0;
  if (!all) {
    force_own = own < g.NB && bl[own] > -INFINITY;
    if (force_own) {
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (lane + 64 * i == own) key[i] = 0u;
    }
    const int need = force_own ? K - 1 : K;
    for (int bit = 31; bit >= 0; --bit) {
      const unsigned Tc = T | (1u << bit);
      int c = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) c += key[i] >= Tc ? 1 : 0;
      if (wave_sum_i(c) >= need) T = Tc;
    }
    int gt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) gt += key[i] > T ? 1 : 0;
    take_ties = need - wave_sum_i(gt);
  }

  const unsigned long long lt = (1ull << lane) - 1ull;
  int written = 0, ties_seen = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = lane + 64 * i;
    bool s;
    if (all) {
      s = key[i] > 0u;
    } else {
      const bool tie = key[i] == T && key[i] > 0u;
      const unsigned long long tm = __ballot(tie);
      const int rank = ties_seen + __popcll(tm & lt);
      s = key[i] > T || (tie && rank < take_ties) || (force_own && j == own);
      ties_seen += __popcll(tm);
    }
    const unsigned long long m = __ballot(s);
    if (s) outp[written + __popcll(m & lt)] = j;
    written += __popcll(m);
  }
  for (int p = written + lane; p < K; p += 64) outp[p] = -1;
}

}  // namespace hs
