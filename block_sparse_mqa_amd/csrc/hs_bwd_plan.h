// Index arithmetic of the gradient work plan, in host-and-device form: the
// kernels (hs_bwd.hip) and the host-side workspace layout (hs_bwd_plan.hip)
// run the same functions. Blocks restart at each document's first row and a
// row attends keys of its own document up to its position (review of
// PaddleFleet PR 1453, block-score PyLayer comments: block_bos; page
// "HySparse MQA sparse attention (FA4 block scoring + SWA MQA + block-sparse
// DSA gather)", section "Core").
#pragma once

#include <hip/hip_runtime.h>

#include "hs_common.h"

namespace hs {

// Host-and-device forms of the block helpers of hs_common.h (the workspace
// plan runs the same arithmetic on the host).
__host__ __device__ inline int blocks_of_entry(const Geom& g, int b) {
  if (g.n_docs == 0) return (g.kv_len[b] + g.BS - 1) / g.BS;
  return g.doc_blk0[g.n_docs];
}

__host__ __device__ inline Blk block_span(const Geom& g, int b, int j) {
  int s, e;
  if (g.n_docs == 0) {
    s = j * g.BS;
    e = g.kv_len[b];
  } else {
    int lo = 0, hi = g.n_docs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (g.doc_blk0[mid] <= j) lo = mid; else hi = mid - 1;
    }
    s = g.doc_start[lo] + (j - g.doc_blk0[lo]) * g.BS;
    e = g.doc_end[lo];
  }
  return Blk{s, e - s < g.BS ? e - s : g.BS};
}

// Whether row rr of entry b gathers block j (the forward's tile rule: a valid
// id whose block meets the row's allowed key range).
__host__ __device__ inline bool gather_hit(const Geom& g, int b, int nb_b, const RowRange& rr,
                                           int j) {
  if (j < 0 || j >= nb_b) return false;
  const Blk bk = block_span(g, b, j);
  return !(bk.start > rr.hi || bk.start + bk.len - 1 < rr.lo);
}

// Rows of entry b whose allowed keys meet block j, for the causal and window
// operations: a contiguous range [*first, *first + n) of row indices.
__host__ __device__ inline int block_row_range(const Geom& g, int op, int b, int j, int window,
                                               int* first) {
  *first = 0;
  if (j >= blocks_of_entry(g, b)) return 0;
  const int L = g.kv_len[b];
  const Blk blk = block_span(g, b, j);
  const Doc d = doc_of_pos(g, b, blk.start);
  const int p_lo = blk.start > L - g.Sq ? blk.start : L - g.Sq;
  int p_hi = d.end - 1;
  if (op == kSwa) {
    const long reach = (long)blk.start + blk.len - 1 + window - 1;
    if (reach < p_hi) p_hi = (int)reach;
  }
  if (p_hi < p_lo) return 0;
  *first = p_lo - (L - g.Sq);
  return p_hi - p_lo + 1;
}

// Sum over x = 0 .. n-1 of (x / bs + 1): the causal key blocks of the rows
// at positions 0 .. n-1 of a document that starts at position 0.
__host__ __device__ inline long long causal_tiles_upto(long long n, int bs) {
  if (n <= 0) return 0;
  const long long m = n / bs;
  return n + (long long)bs * m * (m - 1) / 2 + (n - (long long)bs * m) * m;
}

// Causal key blocks of rows 0 .. r-1 of entry b: a row at position p of a
// document starting at s walks (p - s) / bs + 1 blocks. Documents tile
// [0, Sq) with rows at their positions; without documents the rows of entry
// b sit at kv_len - Sq + r.
__host__ __device__ inline long long causal_tiles_before(const Geom& g, int b, int r) {
  if (g.n_docs == 0) {
    const long long p0 = g.kv_len[b] - g.Sq;
    return causal_tiles_upto(p0 + r, g.BS) - causal_tiles_upto(p0, g.BS);
  }
  long long t = 0;
  for (int d = 0; d < g.n_docs && g.doc_start[d] < r; ++d)
    t += causal_tiles_upto((g.doc_end[d] < r ? g.doc_end[d] : r) - g.doc_start[d], g.BS);
  return t;
}

// Work items of a (b, c, j) with n rows: one if it has rows, or with a split
// of m rows per item, ceil(n / m).
__host__ __device__ inline int items_of(int n, int m) {
  if (n <= 0) return 0;
  return m > 0 ? (n + m - 1) / m : 1;
}

// Rows of work item (b, c, j): a range [*first, *first + n) of row indices,
// or (gather) a range of positions in block j's row list.
__host__ __device__ inline int item_rows(const Geom& g, int op, int b, int c, int j, int window,
                                         int R, int T, const int* g_cnt, const int* g_total,
                                         const int* g_off, int* first) {
  if (op == kGather) {
    const int f = b * g.NB + j;
    const int t0 = c * (R / 64), t1 = (c + 1) * (R / 64);
    const int s0 = g_cnt[((size_t)b * T + t0) * g.NB + j];
    const int s1 = t1 < T ? g_cnt[((size_t)b * T + t1) * g.NB + j] : g_total[f];
    *first = g_off[f] + s0;
    return s1 - s0;
  }
  int bf;
  const int n = block_row_range(g, op, b, j, window, &bf);
  const int lo = bf > c * R ? bf : c * R;
  const int hi = bf + n < (c + 1) * R ? bf + n : (c + 1) * R;
  *first = lo;
  return hi > lo ? hi - lo : 0;
}

}  // namespace hs
