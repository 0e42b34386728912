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
// uint32 keys of the fp32 scores, after the keys that cannot be selected are
// pruned (below): bits shared by every remaining candidate are taken as they
// are, and each remaining bit (from the highest that differs) is one step
// that counts the keys at or above a trial threshold. Counts are wave
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

// AND / OR over the wave, returned in a scalar register. DPP moves: row
// shifts by 1, 2, 4 and 8 leave each 16-lane row's total in its last lane,
// then two row broadcasts carry rows 0 and 0-1 into the rows above, so lane
// 63 holds the total. Lanes whose source is outside the row keep the
// identity. No LDS round trip (a shuffle costs one per step).
template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned dpp_u(unsigned ident, unsigned v) {
  return (unsigned)__builtin_amdgcn_update_dpp((int)ident, (int)v, CTRL, ROWS, 0xf, false);
}
__device__ __forceinline__ unsigned wave_and_u(unsigned v) {
  v &= dpp_u<0x111, 0xf>(~0u, v);   // row_shr:1
  v &= dpp_u<0x112, 0xf>(~0u, v);   // row_shr:2
  v &= dpp_u<0x114, 0xf>(~0u, v);   // row_shr:4
  v &= dpp_u<0x118, 0xf>(~0u, v);   // row_shr:8
  v &= dpp_u<0x142, 0xa>(~0u, v);   // row_bcast:15
  v &= dpp_u<0x143, 0xc>(~0u, v);   // row_bcast:31
  return (unsigned)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ unsigned wave_or_u(unsigned v) {
  v |= dpp_u<0x111, 0xf>(0u, v);
  v |= dpp_u<0x112, 0xf>(0u, v);
  v |= dpp_u<0x114, 0xf>(0u, v);
  v |= dpp_u<0x118, 0xf>(0u, v);
  v |= dpp_u<0x142, 0xa>(0u, v);
  v |= dpp_u<0x143, 0xc>(0u, v);
  return (unsigned)__builtin_amdgcn_readlane((int)v, 63);
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
// pack: this wave's 192-entry LDS buffer (128 packed keys, a spare slot per
// lane).
template <int PER>
__device__ __forceinline__ void topk_row(const Geom& g, const float* block_logit, int* block_idx,
                                         int top_k, int rowi, int lane, unsigned* pack,
                                         float* block_prob = nullptr, float lmax2 = 0.f) {
  rowi = __builtin_amdgcn_readfirstlane(rowi);
  const float* bl = block_logit + (size_t)rowi * g.NB;
  // The row's scores first, so that their loads overlap the geometry below.
  // (a clamped index and a select instead of a guarded load: no divergent
  // branch, whose exec-mask bookkeeping runs on the scalar unit)
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = lane + 64 * i;
    const float x = bl[min(j, g.NB - 1)];
    v[i] = j < g.NB ? x : -INFINITY;
  }
  const int b = rowi / g.Sq, r = rowi % g.Sq;
  const int pos = __builtin_amdgcn_readfirstlane(kv_len_of<true>(g, b)) - g.Sq + r;
  const Doc d = doc_of_pos<true>(g, b, pos);
  // row-uniform values are pinned to scalar registers, so that the branches
  // that test them stay scalar branches (not exec-mask bookkeeping)
  const int own = __builtin_amdgcn_readfirstlane(block_of_pos(g, d, pos));
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
    // Pruning: at least need keys lie at or above the need-th largest of the
    // lanes' two largest keys, so no key below it can be selected. A short
    // search over those 128 values gives a bound B no larger than that value
    // (its bits below the 8 highest that differ among them are left 0); keys
    // under B are dropped, and when at most 128 remain they are packed into
    // two registers per lane (through this wave's LDS buffer, whose
    // operations complete in order), so each step of the exact search
    // compares 2 values per lane instead of PER.
    bool packed = false, c1_empty = false;
    unsigned c[2] = {0u, 0u};
    if (PER >= 2 && need >= 1) {
      // each lane's two largest keys: at least need keys lie at or above the
      // need-th largest of these 128 values, a tighter bound than the lane
      // maxima alone
      unsigned lm = 0u, lm2 = 0u;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        lm2 = max(lm2, min(lm, key[i]));
        lm = max(lm, key[i]);
      }
      if (__popcll(__ballot(lm > 0u)) + __popcll(__ballot(lm2 > 0u)) >= need) {
        const unsigned land = wave_and_u((lm > 0u ? lm : ~0u) & (lm2 > 0u ? lm2 : ~0u));
        const unsigned lor = wave_or_u(lm | lm2);
        unsigned B = land;   // every value equal
        if (land != lor) {
          const int ltop = 31 - __clz(land ^ lor);
          B = ltop == 31 ? 0u : land & ~((2u << ltop) - 1u);
          for (int bit = ltop; bit >= 0 && bit > ltop - 8; --bit) {
            const unsigned Bc = B | (1u << bit);
            if (__popcll(__ballot(lm >= Bc)) + __popcll(__ballot(lm2 >= Bc)) >= need) B = Bc;
          }
        }
#pragma unroll
        for (int i = 0; i < PER; ++i)
          if (key[i] < B) key[i] = 0u;
        const int C = wave_count<PER>([&](int i) { return key[i] > 0u; });
        if (C <= 128) {
          const unsigned long long ltm = (1ull << lane) - 1ull;
          int base = 0;
#pragma unroll
          for (int i = 0; i < PER; ++i) {
            // non-survivors write to their lane's spare slot (no branch)
            const unsigned long long m = __ballot(key[i] > 0u);
            pack[key[i] > 0u ? base + __popcll(m & ltm) : 128 + lane] = key[i];
            base += __popcll(m);
          }
          c[0] = lane < C ? pack[lane] : 0u;
          c[1] = lane + 64 < C ? pack[lane + 64] : 0u;
          packed = true;
          c1_empty = C <= 64;
        }
      }
    }
    // Bits common to every remaining candidate (or packed value), then the
    // threshold with them set and the highest bit that differs.
    auto common_prefix = [&](int& top_out) -> unsigned {
      unsigned kand = ~0u, kor = 0u;
      if (packed) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          if (c[i] > 0u) {
            kand &= c[i];
            kor |= c[i];
          }
      } else {
#pragma unroll
        for (int i = 0; i < PER; ++i)
          if (key[i] > 0u) {
            kand &= key[i];
            kor |= key[i];
          }
      }
      kand = wave_and_u(kand);
      kor = wave_or_u(kor);
      const unsigned diff = kand ^ kor;
      const int top = diff ? 31 - __clz(diff) : -1;
      top_out = top;
      if (top == 31) return 0u;
      return top >= 0 ? kand & ~((2u << top) - 1u) : kand;   // 2u << 31 wraps to 0: all bits
    };
    if (packed && c1_empty) {
      // At most 64 candidates left, one per lane: a bitonic sort across the
      // lanes (descending; vector work only) puts the need-th largest key in
      // lane need - 1.
      unsigned v = c[0];
#pragma unroll
      for (int k = 2; k <= 64; k <<= 1)
#pragma unroll
        for (int jj = k >> 1; jj > 0; jj >>= 1) {
          const unsigned o = (unsigned)__shfl_xor((int)v, jj);
          const bool keep_max = ((lane & jj) == 0) == ((lane & k) == 0);
          v = keep_max ? max(v, o) : min(v, o);
        }
      T = (unsigned)__builtin_amdgcn_readlane((int)v, need - 1);
      take_ties = need - wave_count<1>([&](int) { return c[0] > T; });
    } else if (packed) {
      int top;
      T = common_prefix(top);
      for (int bit = top; bit >= 0; --bit) {
        const unsigned Tc = T | (1u << bit);
        if (wave_count<2>([&](int i) { return c[i] >= Tc; }) >= need) T = Tc;
      }
      take_ties = need - wave_count<2>([&](int i) { return c[i] > T; });
    } else {
      int top;
      T = common_prefix(top);
      for (int bit = top; bit >= 0; --bit) {
        const unsigned Tc = T | (1u << bit);
        if (wave_count<PER>([&](int i) { return key[i] >= Tc; }) >= need) T = Tc;
      }
      take_ties = need - wave_count<PER>([&](int i) { return key[i] > T; });
    }
    T = __builtin_amdgcn_readfirstlane(T);
    take_ties = __builtin_amdgcn_readfirstlane(take_ties);
  }

  const unsigned long long lt = (1ull << lane) - 1ull;
  int written = 0, ties_seen = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = lane + 64 * i;
    // a slot with no key left (after pruning most are empty) selects nothing
    // unless it holds the row's own block
    if (PER > 1 && !(force_own && own >> 6 == i) && __ballot(key[i] > 0u) == 0ull) continue;
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
