// Per-token top-k block selection of one row by one wave (page "HySparse MQA
// sparse attention (FA4 block scoring + SWA MQA + block-sparse DSA gather)",
// per-file overview row for pipeline.py: top-k block selection on the block
// scores, before the gather). Used by the top-k kernel and, for split decode,
// by the merge kernel of the attention engine.
//
// Candidates are the finite scores. When there are more than top_k, the row's
// own block is kept and the other top_k-1 (or top_k if the own block is not a
// candidate) are the best by (score descending, index ascending). The k-th
// best value is found exactly by a bitwise search over order-preserving
// uint32 keys of the fp32 scores: bits shared by every candidate are taken as
// they are, and each remaining bit (from the highest that differs) is one
// step that counts the keys at or above a trial threshold. Counts are wave
// ballots added with scalar popcounts, so a step needs no cross-lane
// shuffle. Entries above the k-th value are taken, and ties at it are taken
// in ascending index order until the count is reached. The final scan runs
// in index order, so the output is already ascending; it is padded with -1.
#pragma once

#include <hip/hip_runtime.h>

#include "hs_common.h"

namespace hs {

// Order-preserving map of a non-NaN float to uint32, on the bits alone (no
// floating-point operation, so denormals keep their order): -0 is taken as
// +0, negative values are complemented, non-negative ones get the top bit set.
__device__ __forceinline__ unsigned ord_key(float v) {
  unsigned u = __float_as_uint(v);
  u = u == 0x80000000u ? 0u : u;
  return u ^ ((unsigned)((int)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ unsigned wave_and_u(unsigned v) {
  for (int o = 32; o >= 1; o >>= 1) v &= (unsigned)__shfl_xor((int)v, o);
  return v;
}
__device__ __forceinline__ unsigned wave_or_u(unsigned v) {
  for (int o = 32; o >= 1; o >>= 1) v |= (unsigned)__shfl_xor((int)v, o);
  return v;
}
// Number of (lane, i) with pred(i) true, by ballots and scalar popcounts.
template <int PER, typename F>
__device__ __forceinline__ int wave_count(F pred) {
  int c = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) c += __popcll(__ballot(pred(i)));
  return c;
}

// Max over the wave of a float (every lane gets it).
__device__ __forceinline__ float wave_max_f(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Top-k of row rowi (= b * Sq + r) by one wave; PER = ceil(NB / 64) values
// per lane. rowi must be the same on every lane (it is kept in scalar
// registers, as are the search threshold and counts). With block_prob set,
// also the row's normalised block scores exp(block_logit - lse_max) (0 where
// block_logit is -inf), lse_max being the row's largest per-head lse (natural
// log, sink included), given in log2 units as lmax2 (page "HySparse MQA sparse
// attention (FA4 block scoring + SWA MQA + block-sparse DSA gather)", per-file
// row for pipeline.py: the block probabilities are recovered as
// exp(block_logit - lse)).
template <int PER>
__device__ __forceinline__ void topk_row(const Geom& g, const float* block_logit, int* block_idx,
                                         int top_k, int rowi, int lane,
                                         float* block_prob = nullptr, float lmax2 = 0.f) {
  rowi = __builtin_amdgcn_readfirstlane(rowi);
  const float* bl = block_logit + (size_t)rowi * g.NB;
  // The row's scores first, so that their loads overlap the geometry below.
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = lane + 64 * i;
    v[i] = j < g.NB ? bl[j] : -INFINITY;
  }
  const int b = rowi / g.Sq, r = rowi % g.Sq;
  const int pos = __builtin_amdgcn_readfirstlane(kv_len_of<true>(g, b)) - g.Sq + r;
  const Doc d = doc_of_pos<true>(g, b, pos);
  const int own = block_of_pos(g, d, pos);
  const int K = top_k;
  if (block_prob != nullptr) {
    float* pr = block_prob + (size_t)rowi * g.NB;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = lane + 64 * i;
      if (j < g.NB)
        pr[j] = v[i] > -INFINITY ? __builtin_amdgcn_exp2f(fmaf(v[i], kLog2e, -lmax2)) : 0.f;
    }
  }
  int* outp = block_idx + (size_t)rowi * K;

  unsigned key[PER];
  unsigned own_key = 0u;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    key[i] = v[i] > -INFINITY ? ord_key(v[i]) : 0u;   // finite scores have keys > 0
    if (lane + 64 * i == own) own_key = key[i];
  }
  const int cnt = wave_count<PER>([&](int i) { return key[i] > 0u; });

  const bool all = cnt <= K;
  bool force_own = false;
  unsigned T = 0u;
  int take_ties = 0;
  if (!all) {
    // the own block's key, from the lane that holds it (own is row-uniform)
    force_own = own >= 0 && own < g.NB &&
                __builtin_amdgcn_readlane((int)own_key, own & 63) != 0;
    if (force_own) {
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (lane + 64 * i == own) key[i] = 0u;
    }
    const int need = force_own ? K - 1 : K;
    // Bits common to every remaining candidate, and the highest that differs.
    unsigned kand = ~0u, kor = 0u;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (key[i] > 0u) {
        kand &= key[i];
        kor |= key[i];
      }
    kand = __builtin_amdgcn_readfirstlane(wave_and_u(kand));
    kor = __builtin_amdgcn_readfirstlane(wave_or_u(kor));
    const unsigned diff = kand ^ kor;
    const int top = diff ? 31 - __clz(diff) : -1;
    T = top >= 0 ? kand & ~((2u << top) - 1u) : kand;   // 2u << 31 wraps to 0: all bits
    if (top == 31) T = 0u;
    for (int bit = top; bit >= 0; --bit) {
      const unsigned Tc = T | (1u << bit);
      if (wave_count<PER>([&](int i) { return key[i] >= Tc; }) >= need) T = Tc;
    }
    take_ties = need - wave_count<PER>([&](int i) { return key[i] > T; });
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
