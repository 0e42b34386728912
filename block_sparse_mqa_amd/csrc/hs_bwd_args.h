// Argument block, workspace layout and launcher of the gradient kernels
// (hs_bwd.hip), used by the C ABI (hs_abi.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "hs_common.h"

namespace hs {

// Arguments of the gradient kernels (both dtypes). The workspace pieces are
// laid out by bwd_layout().
struct BwdArgs {
  const void* q;             // [B, Sq, H, Dk] dtype
  const void* kv;            // [B, Skv, Dk] dtype
  const float* sink;         // [H] or nullptr
  const void* out;           // [B, Sq, H, Dv] dtype (forward output)
  const float* lse;          // [B, Sq, H] (forward output, natural log)
  const void* dout;          // [B, Sq, H, Dv] dtype
  const float* dlse;         // [B, Sq, H] incoming gradient of lse, or nullptr
  const int* block_idx;      // gather: [B, Sq, top_k]
  int top_k;
  int window;
  float* dq;                 // [B, Sq, H, Dk]
  float* dkv;                // [B, Skv, Dk]
  float* dsink;              // [H] or nullptr
  // workspace
  float* dsum;               // [B * Sq * H] dout . out per row and head
  float* sink_part;          // [n_pre, H] per-workgroup sink-gradient partials
  int n_pre, rows_per_pre;
  // Key-block gradient work items: one per (entry b, row chunk c, block j)
  // whose row set is not empty, in the order (b, c, j), so that the items
  // running together share the same query rows.
  int* plan_first;           // [B * C * NB] first row (range) or list position (gather)
  int* plan_nrows;           // [B * C * NB] rows of the item (0: no item)
  int* plan_pre;             // [B * C * NB + 1] item index (exclusive prefix)
  int* g_cnt;                // gather: [B, T, NB] per-row-tile counts, then offsets
  int* g_total;              // gather: [B * NB] rows that selected each block
  int* g_off;                // gather: [B * NB] start of each block's row list
  int* g_rows;               // gather: row lists of all blocks, rows ascending
  int* g_pos;                // gather with stored dS: each list entry's position in its
                             // row's selection (the row's stored tile), or nullptr
  float* part;               // [items, 64, Dk] per-item key-block gradient partials
  // Stored score gradients (bf16; nullptr: dq recomputes them). Tile t of a
  // row holds dS (scale included, bf16) of its 64 heads x the 64 keys of the
  // row's t-th block, in the dq kernel's operand order [head block 4][k-step
  // 2][lane 64][8]. Causal (ds_stride 0): row (b, r) owns tiles ds_entry[b] +
  // tiles_before(b, r) .. + its block count; window: tiles (b Sq + r)
  // ds_stride .. (ds_stride bounds a row's block count); gather: ds_stride =
  // top_k, tile t holding the block of selection entry t.
  __bf16* ds_tiles;
  int ds_stride;
  long long* ds_entry;       // causal: [B + 1] first tile of each entry; [B] = total
  __bf16* ds_dummy;          // 4 KB target of the no-op store of a stage with no predecessor
  int chunk_rows;            // R: rows per chunk (multiple of 64)
  int n_chunks;              // C = ceil(Sq / R)
  int items;                 // work items launched (exact or an upper bound)
  int split_rows;            // gather: rows per work item at most (a (b, c, j) with more
                             // rows becomes several items); 0: one item per (b, c, j)
  int row_tiles;             // T = ceil(Sq / 64)
  Geom g;
};

// Workspace layout of one gradient call: byte offsets of each piece and the
// total, plus the work split of the key-block gradient.
struct BwdLayout {
  size_t dsum, sink_part, first, nrows, pre, cnt, total_g, off_g, rows, pos, part, ds_entry,
      ds_dummy, ds_tiles, total;
  int n_pre, rows_per_pre, chunk_rows, n_chunks, items, row_tiles, ds_stride, split_rows;
  bool store_ds;
};

// store_ds: also lay out the stored score gradients.
BwdLayout bwd_layout(const Geom& g, int op, int top_k, int window, bool store_ds);
int bwd_launch(int op, const BwdArgs& a, bool bf16, hipStream_t stream);

}  // namespace hs
