// CPU debug build of the library's host side: the problem validation, the
// packed-document block table, the decode split plan, the gradient workspace
// layout and the index arithmetic they share with the kernels. Built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host (array-bounds
// checks included) and run without a GPU: the kernel launchers are replaced
// by stubs that check every pointer the entry points carve out of a
// workspace against the workspace's extent and return without launching.
//
// Each planner is compared with a brute-force restatement of the geometry
// written here from the definitions (blocks restart at each document's first
// row and never cross a document; a row at position p attends its document's
// keys up to p, the window's last W of them; review of PaddleFleet PR 1453,
// block-score PyLayer comments: block_bos; page "HySparse MQA sparse
// attention (FA4 block scoring + SWA MQA + block-sparse DSA gather)",
// section "Core"). Malformed problems must be rejected without a sanitizer
// report.
//
// Usage: hs_host_check [n_random_problems] [seed]; prints "all checks
// passed" and exits 0, or names the failed check and aborts.
#include "../../block_sparse_mqa_amd/csrc/hs_abi.hip"
#include "../../block_sparse_mqa_amd/csrc/hs_bwd_plan.hip"

#include <cstdlib>
#include <random>
#include <vector>

#define CHECK(cond, ...)                                                     \
  do {                                                                       \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "check failed at line %d: %s\n  ", __LINE__, #cond); \
      std::fprintf(stderr, __VA_ARGS__);                                     \
      std::fprintf(stderr, "\n");                                            \
      std::abort();                                                          \
    }                                                                        \
  } while (0)

// ---------------------------------------------------------------------------
// Launcher stubs: check what the entry points hand to the kernels.
// ---------------------------------------------------------------------------
namespace {
uintptr_t g_ws_lo = 0, g_ws_hi = 0;   // the workspace of the current call
long long g_launches = 0;
long long g_ds_tiles_expect = -1;     // stored-dS tiles the call must carve

void in_ws(const void* p, size_t bytes, const char* what) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  CHECK(a >= g_ws_lo && a + bytes <= g_ws_hi, "%s [%zx, +%zu) outside the workspace [%zx, %zx)",
        what, (size_t)a, bytes, (size_t)g_ws_lo, (size_t)g_ws_hi);
}
}  // namespace

namespace hs {
int attn_bf16_launch(int op, const AttnArgs& a, hipStream_t) {
  ++g_launches;
  CHECK(op >= kScore && op <= kSwaSparse, "op %d", op);
  CHECK(a.nsplit >= 1 && a.nsplit <= 64, "nsplit %d", a.nsplit);
  if (a.nsplit > 1) {
    const size_t slots = (size_t)a.g.B * a.g.Sq * a.nsplit * a.g.H;
    CHECK(a.split_tiles >= 4, "split_tiles %d", a.split_tiles);
    in_ws(a.ws_o, slots * a.g.Dv * sizeof(float), "split partial O");
    in_ws(a.ws_ml, slots * 2 * sizeof(float), "split max / denominator");
    CHECK(a.g.doc_dev == nullptr, "a launch with device documents split");
  }
  return 0;
}
int attn_f32_launch(int op, const AttnF32Args&, hipStream_t) {
  ++g_launches;
  CHECK(op >= kScore && op <= kSwa, "op %d", op);
  return 0;
}
int topk_launch(const TopkArgs& a, hipStream_t) {
  ++g_launches;
  CHECK(a.top_k >= 1 && a.top_k <= 64 && a.g.NB <= 4096, "top_k %d NB %d", a.top_k, a.g.NB);
  return 0;
}
int mix_launch(const MixArgs& a, hipStream_t) {
  ++g_launches;
  CHECK(a.rows >= 1 && a.dv >= 1, "mix rows %lld dv %d", a.rows, a.dv);
  return 0;
}
int bwd_launch(int op, const BwdArgs& a, bool, hipStream_t) {
  ++g_launches;
  const Geom& g = a.g;
  const size_t rows = (size_t)g.B * g.Sq;
  const size_t F = (size_t)g.B * a.n_chunks * g.NB;
  CHECK(a.chunk_rows >= 64 && a.chunk_rows % 64 == 0, "chunk_rows %d", a.chunk_rows);
  CHECK(a.n_chunks == (g.Sq + a.chunk_rows - 1) / a.chunk_rows, "n_chunks %d", a.n_chunks);
  CHECK((long)a.n_pre * a.rows_per_pre >= (long)rows, "pre covers %d x %d of %zu rows", a.n_pre,
        a.rows_per_pre, rows);
  in_ws(a.dsum, rows * g.H * sizeof(float), "dsum");
  in_ws(a.sink_part, (size_t)a.n_pre * g.H * sizeof(float), "sink partials");
  in_ws(a.plan_first, F * sizeof(int), "plan_first");
  in_ws(a.plan_nrows, F * sizeof(int), "plan_nrows");
  in_ws(a.plan_pre, (F + 1) * sizeof(int), "plan_pre");
  if (op == kGather) {
    in_ws(a.g_cnt, (size_t)g.B * a.row_tiles * g.NB * sizeof(int), "gather counts");
    in_ws(a.g_total, (size_t)g.B * g.NB * sizeof(int), "gather totals");
    in_ws(a.g_off, (size_t)g.B * g.NB * sizeof(int), "gather offsets");
    in_ws(a.g_rows, rows * a.top_k * sizeof(int), "gather row lists");
    if (a.ds_tiles != nullptr) {
      in_ws(a.g_pos, rows * a.top_k * sizeof(int), "gather list positions");
      CHECK(a.ds_stride == a.top_k, "gather dS stride %d, top_k %d", a.ds_stride, a.top_k);
    } else {
      CHECK(a.g_pos == nullptr, "gather list positions without stored dS");
    }
  }
  in_ws(a.part, (size_t)a.items * 64 * g.Dk * sizeof(float), "dkv partials");
  if (a.ds_tiles != nullptr) {
    CHECK(g_ds_tiles_expect >= 0, "stored dS carved where none was expected");
    in_ws(a.ds_entry, (g.B + 1) * sizeof(long long), "dS entry offsets");
    in_ws(a.ds_dummy, 4096, "dS dummy target");
    in_ws(a.ds_tiles, (size_t)g_ds_tiles_expect * 64 * 64 * 2, "stored dS tiles");
  }
  return 0;
}
}  // namespace hs

// ---------------------------------------------------------------------------
// Brute-force geometry.
// ---------------------------------------------------------------------------
namespace {

struct Spec {
  int B = 1, Sq = 1, Skv = 1;
  bool f32 = false;
  std::vector<int> lens;        // host kv_lens (empty: Skv for every entry)
  std::vector<int> docs;        // document lengths (B == 1, Sq == Skv), or empty
};

struct Brute {
  std::vector<int> L;                                      // per entry
  std::vector<std::vector<std::pair<int, int>>> blocks;    // per entry: (start, len)
  std::vector<std::pair<int, int>> doc;                    // [start, end) per document
  int NB = 0;
};

Brute brute(const Spec& s) {
  Brute r;
  for (int b = 0; b < s.B; ++b) r.L.push_back(s.lens.empty() ? s.Skv : s.lens[b]);
  if (!s.docs.empty()) {
    int st = 0;
    for (int n : s.docs) {
      r.doc.push_back({st, st + n});
      st += n;
    }
  }
  for (int b = 0; b < s.B; ++b) {
    std::vector<std::pair<int, int>> bl;
    if (r.doc.empty()) {
      for (int x = 0; x < r.L[b]; x += 64) bl.push_back({x, std::min(64, r.L[b] - x)});
    } else {
      for (auto& d : r.doc)
        for (int x = d.first; x < d.second; x += 64) bl.push_back({x, std::min(64, d.second - x)});
    }
    r.NB = std::max<int>(r.NB, (int)bl.size());
    r.blocks.push_back(bl);
  }
  return r;
}

// Allowed key range [lo, hi] of row r of entry b (op: kScore or kSwa).
std::pair<int, int> allowed(const Spec& s, const Brute& r, int b, int row, int op, int window) {
  const int p = r.L[b] - s.Sq + row;
  int lo = 0;
  for (auto& d : r.doc)
    if (d.first <= p && p < d.second) lo = d.first;
  if (op == hs::kSwa) lo = std::max(lo, p - window + 1);
  return {lo, p};
}

bool meets(std::pair<int, int> blk, std::pair<int, int> rng) {
  return blk.first <= rng.second && blk.first + blk.second - 1 >= rng.first;
}

struct Built {
  hs_problem p{};
  std::vector<int> lens, ds, de;
};

Built make_problem(const Spec& s) {
  Built m;
  m.p.batch = s.B;
  m.p.seqlen_q = s.Sq;
  m.p.seqlen_kv = s.Skv;
  m.p.block_size = 64;
  m.p.dtype = s.f32 ? HS_F32 : HS_BF16;
  m.p.num_heads = s.f32 ? 8 : 64;
  m.p.head_dim_qk = s.f32 ? 96 : 576;
  m.p.head_dim_v = s.f32 ? 64 : 512;
  m.lens = s.lens;
  if (!m.lens.empty()) {
    m.p.kv_lens = m.lens.data();
    m.p.n_kv_lens = (int)m.lens.size();
  }
  int st = 0;
  for (int n : s.docs) {
    m.ds.push_back(st);
    m.de.push_back(st + n);
    st += n;
  }
  if (!s.docs.empty()) {
    m.p.doc_start = m.ds.data();
    m.p.doc_end = m.de.data();
    m.p.n_docs = (int)s.docs.size();
  }
  return m;
}

long long g_rows_checked = 0, g_blocks_checked = 0, g_items_checked = 0;

// The planners and index helpers of one valid problem against brute force,
// then every entry point through the stubs.
void check_problem(const Spec& s, std::mt19937& rng) {
  Built m = make_problem(s);
  const Brute r = brute(s);
  hs::Geom g;
  CHECK(prepare(&m.p, g) == HS_OK, "valid problem rejected: %s", g_last_error.c_str());
  CHECK(g.NB == r.NB, "NB %d, brute force %d", g.NB, r.NB);
  CHECK(hs_num_blocks(&m.p) == r.NB, "hs_num_blocks");
  const int window = std::uniform_int_distribution<int>(1, 3 * s.Skv)(rng);
  const int top_k = std::uniform_int_distribution<int>(1, 64)(rng);

  for (int b = 0; b < s.B; ++b) {
    CHECK(hs::blocks_of_entry(g, b) == (int)r.blocks[b].size(), "blocks of entry %d", b);
    for (int j = 0; j < (int)r.blocks[b].size(); ++j) {
      const hs::Blk bk = hs::block_span(g, b, j);
      CHECK(bk.start == r.blocks[b][j].first && bk.len == r.blocks[b][j].second,
            "block_span(%d, %d) = (%d, %d), brute force (%d, %d)", b, j, bk.start, bk.len,
            r.blocks[b][j].first, r.blocks[b][j].second);
      ++g_blocks_checked;
    }
    long long tiles = 0;
    for (int row = 0; row < s.Sq; ++row) {
      CHECK(hs::causal_tiles_before(g, b, row) == tiles, "causal_tiles_before(%d, %d)", b, row);
      for (int op : {hs::kScore, hs::kSwa}) {
        const hs::RowRange rr = hs::row_range(g, op, b, row, window);
        const auto want = allowed(s, r, b, row, op, window);
        CHECK(rr.lo == want.first && rr.hi == want.second, "row_range(%d, %d) keys [%d, %d], want [%d, %d]",
              b, row, rr.lo, rr.hi, want.first, want.second);
        int jf = -1, jl = -1;
        for (int j = 0; j < (int)r.blocks[b].size(); ++j)
          if (meets(r.blocks[b][j], want)) {
            if (jf < 0) jf = j;
            jl = j;
          }
        CHECK(rr.j_first == jf && rr.j_last == jl, "row_range(%d, %d) blocks [%d, %d], want [%d, %d]",
              b, row, rr.j_first, rr.j_last, jf, jl);
        CHECK(rr.doc.start <= rr.lo && rr.hi < rr.doc.end, "row document");
        if (op == hs::kScore) tiles += jl - jf + 1;
      }
      ++g_rows_checked;
    }
    CHECK(hs::causal_tiles_before(g, b, s.Sq) == tiles, "causal_tiles_before(%d, Sq)", b);
    // rows whose allowed keys meet block j: one contiguous range
    for (int op : {hs::kScore, hs::kSwa})
      for (int j = 0; j < (int)r.blocks[b].size(); ++j) {
        int first = -1;
        const int n = hs::block_row_range(g, op, b, j, window, &first);
        int wf = -1, wn = 0;
        for (int row = 0; row < s.Sq; ++row)
          if (meets(r.blocks[b][j], allowed(s, r, b, row, op, window))) {
            if (wf < 0) wf = row;
            CHECK(row == wf + wn, "rows of block %d are not contiguous", j);
            ++wn;
          }
        CHECK(n == wn && (n == 0 || first == wf), "block_row_range(%d, %d, op %d) = (%d, %d), want (%d, %d)",
              b, j, op, first, n, wf, wn);
      }
  }

  // gradient layout: item counts by brute force, pieces aligned and disjoint
  for (int op : {hs::kScore, hs::kSwa, hs::kGather})
    for (bool store : {false, true}) {
      const hs::BwdLayout L = hs::bwd_layout(g, op, top_k, window, store);
      CHECK(L.chunk_rows >= 64 && (L.chunk_rows & (L.chunk_rows - 1)) == 0, "chunk_rows %d",
            L.chunk_rows);
      const int oc = op == hs::kSwa ? hs::kSwa : hs::kScore;
      long items = 0, split_items = 0;
      for (int b = 0; b < s.B; ++b)
        for (int c = 0; c < L.n_chunks; ++c)
          for (int j = 0; j < g.NB; ++j) {
            int first = 0;
            const int n = hs::item_rows(g, oc, b, c, j, window, L.chunk_rows, 0, nullptr, nullptr,
                                        nullptr, &first);
            int wn = 0;
            if (j < (int)r.blocks[b].size())
              for (int row = c * L.chunk_rows; row < std::min(s.Sq, (c + 1) * L.chunk_rows); ++row)
                wn += meets(r.blocks[b][j], allowed(s, r, b, row, oc, window));
            CHECK(n == wn, "item (%d, %d, %d) has %d rows, brute force %d", b, c, j, n, wn);
            CHECK(n == 0 || (first >= c * L.chunk_rows && first + n <= std::min(s.Sq, (c + 1) * L.chunk_rows)),
                  "item rows outside its chunk");
            items += n > 0;
            split_items += hs::items_of(n, L.split_rows);
            ++g_items_checked;
          }
      if (op == hs::kGather) {
        // the gather's rows lie within the causal ones; items of more than
        // split_rows rows split, adding at most ceil(B Sq top_k / split_rows)
        const long sel = (long)s.B * s.Sq * top_k;
        CHECK(L.split_rows >= 128 && sel / L.split_rows <= 8192, "split_rows %d", L.split_rows);
        items += (sel + L.split_rows - 1) / L.split_rows;
      } else if (op == hs::kSwa) {
        // window items split the same way: at most ceil(B Sq per / split_rows)
        // more, per = the most blocks a window meets; the exact split count
        // must fit the layout
        const long per = std::min<long>((window - 1 + 63) / 64 + 1, g.NB);
        const long sel = (long)s.B * s.Sq * per;
        CHECK(L.split_rows >= 128 && sel / L.split_rows <= 8192, "split_rows %d", L.split_rows);
        items += (sel + L.split_rows - 1) / L.split_rows;
        CHECK(split_items <= items, "window items after the split %ld, layout %ld", split_items,
              items);
      } else {
        CHECK(L.split_rows == 0, "split_rows %d for the causal gradient", L.split_rows);
      }
      CHECK(L.items == items, "items %d, brute force %ld", L.items, items);
      const size_t offs[] = {L.dsum, L.sink_part, L.first, L.nrows, L.pre, L.part, L.total};
      for (size_t i = 0; i + 1 < sizeof(offs) / sizeof(offs[0]); ++i)
        CHECK(offs[i] % 256 == 0 && offs[i] <= offs[i + 1], "layout piece %zu", i);
    }

  // entry points through the stubs, each with exactly the workspace it asks for
  const uintptr_t base = (uintptr_t)1 << 44;
  void* f = reinterpret_cast<void*>(base - 4096);   // any aligned non-null device pointer
  float* ff = static_cast<float*>(f);
  int* fi = static_cast<int*>(f);
  auto with_ws = [&](int op, int k, int w, auto call) {
    size_t n = 0;
    CHECK(hs_workspace_size(&m.p, op, k, w, &n) == HS_OK, "workspace size op %d: %s", op,
          g_last_error.c_str());
    g_ws_lo = base;
    g_ws_hi = base + n;
    const hs_status st = call(n ? reinterpret_cast<void*>(base) : nullptr, n);
    CHECK(st == HS_OK, "entry point op %d: %s", op, g_last_error.c_str());
  };
  with_ws(HS_OP_BLOCK_SCORE, 0, 0, [&](void* ws, size_t n) {
    return hs_block_score_fwd(&m.p, f, f, ff, f, ff, ff, ws, n, nullptr);
  });
  if (r.NB <= 4096)
    with_ws(HS_OP_BLOCK_SCORE, 0, 0, [&](void* ws, size_t n) {
      return hs_block_score_topk_fwd(&m.p, f, f, ff, top_k, f, ff, ff, fi, ff, ws, n, nullptr);
    });
  with_ws(HS_OP_SPARSE_GATHER, top_k, 0, [&](void* ws, size_t n) {
    return hs_sparse_gather_fwd(&m.p, f, f, ff, fi, top_k, f, ff, ws, n, nullptr);
  });
  with_ws(HS_OP_SWA, 0, window, [&](void* ws, size_t n) {
    return hs_swa_fwd(&m.p, f, f, ff, window, f, ff, ws, n, nullptr);
  });
  with_ws(HS_OP_SWA_SPARSE, top_k, window, [&](void* ws, size_t n) {
    return hs_swa_sparse_fwd(&m.p, f, f, ff, window, fi, top_k, f, ff, f, ff, ff, ff, f, ws, n,
                             nullptr);
  });
  long long causal_tiles = 0;
  for (int b = 0; b < s.B; ++b) causal_tiles += hs::causal_tiles_before(g, b, s.Sq);
  const long long per = std::min<long long>((window - 1 + 63) / 64 + 1, g.NB);
  struct BwdCase { int op, ws_op; long long tiles; };
  const BwdCase cases[] = {
      {HS_OP_BLOCK_SCORE, HS_OP_BLOCK_SCORE_BWD, -1},
      {HS_OP_BLOCK_SCORE, HS_OP_BLOCK_SCORE_BWD_STORE_DS, s.f32 ? -1 : causal_tiles},
      {HS_OP_SWA, HS_OP_SWA_BWD, -1},
      {HS_OP_SWA, HS_OP_SWA_BWD_STORE_DS, s.f32 ? -1 : (long long)s.B * s.Sq * per},
      {HS_OP_SPARSE_GATHER, HS_OP_SPARSE_GATHER_BWD, -1},
      {HS_OP_SPARSE_GATHER, HS_OP_SPARSE_GATHER_BWD_STORE_DS,
       s.f32 ? -1 : (long long)s.B * s.Sq * top_k}};
  for (const BwdCase& c : cases) {
    g_ds_tiles_expect = c.tiles;
    with_ws(c.ws_op, top_k, window, [&](void* ws, size_t n) {
      if (c.op == HS_OP_BLOCK_SCORE)
        return hs_block_score_bwd(&m.p, f, f, ff, f, ff, f, ff, ff, ff, ff, ws, n, nullptr);
      if (c.op == HS_OP_SWA)
        return hs_swa_bwd(&m.p, f, f, ff, window, f, ff, f, ff, ff, ff, ff, ws, n, nullptr);
      return hs_sparse_gather_bwd(&m.p, f, f, ff, fi, top_k, f, ff, f, ff, ff, ff, ff, ws, n,
                                  nullptr);
    });
    g_ds_tiles_expect = -1;
  }
}

Spec random_spec(std::mt19937& rng) {
  auto U = [&](int a, int b) { return std::uniform_int_distribution<int>(a, b)(rng); };
  Spec s;
  s.f32 = U(0, 4) == 0;
  const int kind = U(0, 3);
  if (kind == 0) {          // one sequence
    s.Sq = s.Skv = U(1, 700);
  } else if (kind == 1) {   // packed documents
    const int nd = U(1, 12);
    s.Sq = 0;
    for (int d = 0; d < nd; ++d) {
      s.docs.push_back(U(1, 150));
      s.Sq += s.docs.back();
    }
    s.Skv = s.Sq;
  } else if (kind == 2) {   // chunked prefill over caches of their own lengths
    s.B = U(1, 4);
    s.Sq = U(1, 100);
    s.Skv = s.Sq + U(0, 600);
    for (int b = 0; b < s.B; ++b) s.lens.push_back(U(s.Sq, s.Skv));
  } else {                  // decode
    s.B = U(1, 12);
    s.Sq = 1;
    s.Skv = U(1, 5000);
    for (int b = 0; b < s.B; ++b) s.lens.push_back(U(1, s.Skv));
  }
  return s;
}

// Malformed problems: every one must come back as an error (or, where it is
// valid after all, OK) without a sanitizer report.
void check_rejections(std::mt19937& rng, long long* rejected) {
  auto U = [&](int a, int b) { return std::uniform_int_distribution<int>(a, b)(rng); };
  for (int it = 0; it < 4000; ++it) {
    hs_problem p{};
    p.batch = U(-2, 300);
    p.seqlen_q = U(-2, 3000);
    p.seqlen_kv = U(-2, 3000);
    p.num_heads = U(0, 1) ? 64 : U(-1, 70);
    p.head_dim_qk = U(0, 1) ? 576 : U(-1, 600);
    p.head_dim_v = U(0, 1) ? 512 : U(-1, 600);
    p.block_size = U(0, 3) ? 64 : U(-1, 128);
    p.dtype = U(-1, 2);
    std::vector<int> lens(std::max(p.batch, 1)), ds(65), de(65);
    for (int& x : lens) x = U(-5, 3100);
    for (int i = 0; i < 65; ++i) {
      ds[i] = U(-5, 3100);
      de[i] = U(-5, 3100);
    }
    if (U(0, 2) == 0) {
      p.kv_lens = lens.data();
      p.n_kv_lens = U(0, 1) ? p.batch : U(0, 300);
      if (p.n_kv_lens > (int)lens.size()) p.n_kv_lens = (int)lens.size();
    }
    if (U(0, 2) == 0) {
      p.n_docs = U(0, 65);
      if (U(0, 1) && p.seqlen_q > 0) {   // a tiling of [0, seqlen_q) now and then
        int st = 0;
        const int nd = std::min(p.n_docs, 64);
        for (int d = 0; d < nd; ++d) {
          const int e = d + 1 == nd ? p.seqlen_q : std::min(p.seqlen_q, st + U(0, 200));
          ds[d] = st;
          de[d] = e;
          st = e;
        }
      }
      if (U(0, 5)) {
        p.doc_start = ds.data();
        p.doc_end = de.data();
      }
    }
    if (U(0, 5) == 0) p.page_table = reinterpret_cast<const int32_t*>(uintptr_t(U(0, 2) ? 4096 : 4098));
    if (U(0, 5) == 0) p.max_pages = U(-1, 60);
    if (U(0, 5) == 0) p.kv_lens_device = reinterpret_cast<const int32_t*>(uintptr_t(U(0, 2) ? 8192 : 8194));
    if (U(0, 5) == 0) p.doc_bounds_device = reinterpret_cast<const int32_t*>(uintptr_t(U(0, 2) ? 12288 : 12290));
    const int32_t nb = hs_num_blocks(&p);
    if (nb < 0) {
      ++*rejected;
      CHECK(!g_last_error.empty(), "an error without a message");
      continue;
    }
    hs::Geom g;
    CHECK(prepare(&p, g) == HS_OK && g.NB == nb, "accepted problem without a block count");
    for (int op = HS_OP_BLOCK_SCORE; op <= HS_OP_SWA_SPARSE; ++op) {
      size_t n = 0;
      (void)hs_workspace_size(&p, op, U(-1, 70), U(-1, 5000), &n);
    }
  }
}

}  // namespace

int main(int argc, char** argv) {
  const int n = argc > 1 ? std::atoi(argv[1]) : 150;
  const unsigned seed = argc > 2 ? (unsigned)std::atoi(argv[2]) : 1u;
  std::mt19937 rng(seed);
  // fixed edge cases first
  std::vector<Spec> specs;
  {
    Spec s; s.Sq = s.Skv = 1; specs.push_back(s);
    s.Sq = s.Skv = 64; specs.push_back(s);
    s.Sq = s.Skv = 65; specs.push_back(s);
    s.Sq = s.Skv = 130; specs.push_back(s);
    Spec d; d.docs = {70, 1, 63, 100, 66}; d.Sq = d.Skv = 300; specs.push_back(d);
    Spec e; e.docs = std::vector<int>(64, 3); e.Sq = e.Skv = 192; specs.push_back(e);
    Spec c; c.B = 2; c.Sq = 70; c.Skv = 200; c.lens = {200, 150}; specs.push_back(c);
    Spec k; k.B = 3; k.Sq = 1; k.Skv = 3000; k.lens = {3000, 1200, 64}; specs.push_back(k);
    Spec t; t.B = 256; t.Sq = 1; t.Skv = 2048;
    for (int b = 0; b < 256; ++b) t.lens.push_back(1 + (b * 37) % 2048);
    specs.push_back(t);
    Spec x; x.f32 = true; x.docs = {100, 2, 148}; x.Sq = x.Skv = 250; specs.push_back(x);
  }
  for (int i = 0; i < n; ++i) specs.push_back(random_spec(rng));
  for (const Spec& s : specs) check_problem(s, rng);
  long long rejected = 0;
  check_rejections(rng, &rejected);
  std::printf("problems %zu, rows %lld, blocks %lld, work items %lld, launches %lld, "
              "malformed problems rejected %lld\n",
              specs.size(), g_rows_checked, g_blocks_checked, g_items_checked, g_launches, rejected);
  std::printf("all checks passed\n");
  return 0;
}
