// Device-side problem geometry shared by the HIP kernels of the HySparse MQA
// forward path: positions, packed documents and key blocks.
//
// Blocks restart at each document's first row and never cross a document
// (review of PaddleFleet PR 1453, block-score PyLayer comments: the per-block
// start row block_bos). Block ids are global, numbered in document order.
// A query row r of batch entry b sits at position L_b - Sq + r (blog page on
// the unified sparse-attention dispatcher, decode paragraph: a decode token's
// key length is the cache plus the current token).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs {

constexpr int kMaxBatch = 256;
constexpr int kMaxDocs = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Copied by value into kernel arguments.
struct Geom {
  int B, Sq, Skv, H, Dk, Dv, BS, NB;
  int n_docs;
  float scale_log2;              // softmax scale * log2(e)
  int kv_len[kMaxBatch];         // valid KV rows per entry (Skv when not given)
  int doc_start[kMaxDocs];
  int doc_end[kMaxDocs];
  int doc_blk0[kMaxDocs + 1];    // first global block id of each document
  const int* kv_len_dev;         // device [B] valid KV rows, or nullptr: then kv_len
                                 // holds the capacity the host planned with
  const int* doc_dev;            // device [n_docs + 1] cumulative document starts, or
                                 // nullptr; n_docs is then the capacity and the host
                                 // arrays above are unused
};

// Valid KV rows of entry b. Launches given device lengths (DEV and
// kv_len_dev set) read them at run time; otherwise, and always on the host,
// the value in the arguments.
template <bool DEV = false>
__host__ __device__ inline int kv_len_of(const Geom& g, int b) {
#if defined(__HIP_DEVICE_COMPILE__)
  if (DEV && g.kv_len_dev != nullptr) return g.kv_len_dev[b];
#endif
  return g.kv_len[b];
}

struct Doc {
  int start, end, blk0;
};

struct Blk {
  int start, len;
};

#if defined(__HIP_DEVICE_COMPILE__)
// Document holding position p, from the device table of cumulative starts
// (at most 64 documents: lane l holds document l). Every lane of the wave must
// take part, with the same p. The holder is the last document starting at or
// before p; it cannot be empty, since the next start is past p. Its first
// block id is the sum of the block counts of the documents before it. Bounds
// are clamped into [0, Sq], so a malformed table cannot send reads outside
// the sequence.
__device__ inline Doc doc_of_pos_wave(const Geom& g, int p) {
  const int l = __lane_id();
  const int nd = g.n_docs;
  int s = 0x7fffffff, e = 0x7fffffff, nb = 0;
  if (l < nd) {
    s = min(max(g.doc_dev[l], 0), g.Sq);
    e = min(max(g.doc_dev[l + 1], s), g.Sq);
    nb = (e - s + g.BS - 1) / g.BS;
  }
  const unsigned long long m = __ballot(l < nd && s <= p);
  const int d = m ? 63 - __clzll((long long)m) : 0;
  int before = l < d ? nb : 0;
  for (int o = 32; o >= 1; o >>= 1) before += __shfl_xor(before, o);
  return Doc{__builtin_amdgcn_readlane(s, d), __builtin_amdgcn_readlane(e, d), before};
}
#endif

// Document holding position p of entry b. With a device document table (DEV
// launches only) every lane of the wave must call it with the same p.
template <bool DEV = false>
__host__ __device__ inline Doc doc_of_pos(const Geom& g, int b, int p) {
#if defined(__HIP_DEVICE_COMPILE__)
  if (DEV && g.doc_dev != nullptr) return doc_of_pos_wave(g, p);
#endif
  if (g.n_docs == 0) return Doc{0, kv_len_of<DEV>(g, b), 0};
  int lo = 0, hi = g.n_docs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (g.doc_start[mid] <= p) lo = mid; else hi = mid - 1;
  }
  return Doc{g.doc_start[lo], g.doc_end[lo], g.doc_blk0[lo]};
}

// Number of key blocks of entry b (with a device document table, the
// capacity NB).
template <bool DEV = false>
__device__ __forceinline__ int nb_of_entry(const Geom& g, int b) {
  if (g.n_docs == 0) return (kv_len_of<DEV>(g, b) + g.BS - 1) / g.BS;
  if (DEV && g.doc_dev != nullptr) return g.NB;
  return g.doc_blk0[g.n_docs];
}

// Rows [start, start + len) of block j of document d (j must be one of d's
// blocks; without documents d is the whole entry). A row only ever attends
// keys of its own document, so loops over a row's tiles use its document and
// need no lookup.
__device__ __forceinline__ Blk block_rows_in(const Geom& g, const Doc& d, int j) {
  const int s = d.start + (j - d.blk0) * g.BS;
  return Blk{s, min(g.BS, d.end - s)};
}

// Whether block j is one of document d's.
__device__ __forceinline__ bool block_in_doc(const Geom& g, const Doc& d, int j) {
  return j >= d.blk0 && j < d.blk0 + (d.end - d.start + g.BS - 1) / g.BS;
}

// Rows [start, start + len) of block j of entry b (j must be valid).
template <bool DEV = false>
__device__ __forceinline__ Blk block_rows(const Geom& g, int b, int j) {
  if (g.n_docs == 0) {
    int s = j * g.BS;
    return Blk{s, min(g.BS, kv_len_of<DEV>(g, b) - s)};
  }
  int lo = 0, hi = g.n_docs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (g.doc_blk0[mid] <= j) lo = mid; else hi = mid - 1;
  }
  int s = g.doc_start[lo] + (j - g.doc_blk0[lo]) * g.BS;
  return Blk{s, min(g.BS, g.doc_end[lo] - s)};
}

// Global block id of position p inside document d.
__host__ __device__ inline int block_of_pos(const Geom& g, const Doc& d, int p) {
  return d.blk0 + (p - d.start) / g.BS;
}

// Key range [lo, hi] a row may attend to for each operation, and the block
// range that covers it.
// kSwaSparse: both branches of a sliding-window layer in one pass, the
// window's tiles and then the selected blocks' (separate outputs).
enum Op { kScore = 0, kGather = 1, kSwa = 2, kSwaSparse = 3 };

struct RowRange {
  int pos, lo, hi, j_first, j_last;
  Doc doc;   // the row's document (the whole entry without documents)
};

template <bool DEV = false>
__host__ __device__ inline RowRange row_range(const Geom& g, int op, int b, int r, int window) {
  RowRange rr;
  rr.pos = kv_len_of<DEV>(g, b) - g.Sq + r;
  Doc d = doc_of_pos<DEV>(g, b, rr.pos);
  rr.doc = d;
  rr.lo = d.start;
  rr.hi = rr.pos;
  if (op == kSwa && rr.pos - window + 1 > rr.lo) rr.lo = rr.pos - window + 1;
  rr.j_first = block_of_pos(g, d, rr.lo);
  rr.j_last = block_of_pos(g, d, rr.hi);
  return rr;
}

}  // namespace hs
