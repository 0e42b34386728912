// Workspace layout of the gradient calls (host only): the byte offset of
// every piece of the workspace, the row chunking of the key-block gradient's
// work items and the stored score gradients' extent (the calls themselves
// are in hs_bwd.hip).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "hs_bwd_args.h"
#include "hs_bwd_plan.h"
#include "hs_common.h"

namespace hs {

namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

BwdLayout bwd_layout(const Geom& g, int op, int top_k, int window, bool store_ds) {
  BwdLayout L;
  std::memset(&L, 0, sizeof(L));
  const size_t rows = (size_t)g.B * g.Sq;
  L.rows_per_pre = (int)std::max<size_t>(8, (rows + 2047) / 2048);
  L.n_pre = (int)((rows + L.rows_per_pre - 1) / L.rows_per_pre);
  size_t off = 0;
  L.dsum = off;
  off = align256(off + rows * g.H * sizeof(float));
  L.sink_part = off;
  off = align256(off + (size_t)L.n_pre * g.H * sizeof(float));
  {
    L.row_tiles = (g.Sq + 63) / 64;
    // Row chunk R: the largest power of two from 512 down to 64 that still
    // gives about 1024 work items (four per compute unit). At R = 512 the Q
    // and dout rows of one chunk (71 MB) stay in the 256 MB last-level cache
    // while the chunk's items run (1024 and 256 measured within 2 % of it).
    // Longer sequences double R until at most 32768 items remain, which
    // bounds the partials at 32768 x 64 x Dk fp32 (4.8 GB for Dk = 576).
    auto items_for = [&](int R) -> long {
      const int C = (g.Sq + R - 1) / R;
      long it = 0;
      const int oc = op == kSwa ? kSwa : kScore;  // gather rows lie in the causal ones
      for (int b = 0; b < g.B; ++b)
        for (int c = 0; c < C; ++c)
          for (int j = 0; j < g.NB; ++j) {
            int first;
            it += item_rows(g, oc, b, c, j, window, R, 0, nullptr, nullptr, nullptr, &first) > 0;
          }
      return it;
    };
    int R = 512;
    while (R > 64 && items_for(R) < 1024) R >>= 1;
    while (R < g.Sq && items_for(R) > 32768) R <<= 1;
    L.chunk_rows = R;
    L.n_chunks = (g.Sq + R - 1) / R;
    L.items = (int)items_for(R);
    if (op == kGather || op == kSwa) {
      // Items differ in length: a gather block that many rows of a chunk
      // selected (the rows' own and recent blocks) against one that a few
      // did; a window block whose rows fill a chunk against one at a chunk's
      // edge. Long items among short ones leave compute units idle at the
      // end of the launch, so items are split into items of at most
      // split_rows rows, whose partials the reduction adds in order. Each
      // extra item takes split_rows of the B * Sq * per (row, block) pairs,
      // per = top_k, or for the window the most blocks W keys can meet, so
      // at most that many / split_rows are added (capped near 8192).
      const long per = op == kGather
                           ? std::max(top_k, 1)
                           : std::min<long>((window - 1 + (long)g.BS - 1) / g.BS + 1, g.NB);
      const long sel = (long)g.B * g.Sq * per;
      L.split_rows = (int)std::max<long>(128, (sel + 8191) / 8192);
      L.items += (int)((sel + L.split_rows - 1) / L.split_rows);
    }
    const size_t F = (size_t)g.B * L.n_chunks * g.NB;
    L.first = off;
    off = align256(off + F * sizeof(int));
    L.nrows = off;
    off = align256(off + F * sizeof(int));
    L.pre = off;
    off = align256(off + (F + 1) * sizeof(int));
    if (op == kGather) {
      const size_t FB = (size_t)g.B * g.NB;
      L.cnt = off;
      off = align256(off + (size_t)g.B * L.row_tiles * g.NB * sizeof(int));
      L.total_g = off;
      off = align256(off + FB * sizeof(int));
      L.off_g = off;
      off = align256(off + FB * sizeof(int));
      L.rows = off;
      off = align256(off + rows * std::max(top_k, 1) * sizeof(int));
      if (store_ds) {
        L.pos = off;
        off = align256(off + rows * std::max(top_k, 1) * sizeof(int));
      }
    }
    L.part = off;
    off = align256(off + (size_t)L.items * 64 * g.Dk * sizeof(float));
  }
  if (store_ds) {
    // 64 heads x 64 keys of bf16 per (row, block of its range); a window of
    // W keys meets at most ceil((W - 1) / BS) + 1 blocks; a gather row owns
    // one tile per selection entry
    long long tiles = 0;
    if (op == kScore) {
      for (int b = 0; b < g.B; ++b) tiles += causal_tiles_before(g, b, g.Sq);
    } else if (op == kGather) {
      L.ds_stride = std::max(top_k, 1);
      tiles = (long long)g.B * g.Sq * L.ds_stride;
    } else {
      const long long per = std::min<long long>((window - 1 + (long long)g.BS - 1) / g.BS + 1, g.NB);
      L.ds_stride = (int)per;
      tiles = (long long)g.B * g.Sq * per;
    }
    L.store_ds = true;
    L.ds_entry = off;
    off = align256(off + (size_t)(g.B + 1) * sizeof(long long));
    L.ds_dummy = off;
    off = align256(off + 4096);
    L.ds_tiles = off;
    off = align256(off + (size_t)tiles * 64 * 64 * sizeof(uint16_t));
  }
  L.total = off;
  return L;
}

}  // namespace hs
