// Host side of the C ABI declared in include/hs.h: argument validation, the
// block table of packed documents, workspace sizing and kernel launches.
//
// Validation follows the error conventions of the pages: every check runs on
// the host before anything is launched and failures are reported, not
// asserted (review of PaddleFleet PR 1453, the request to replace assert
// checks with ValueError); an input the path cannot honour is rejected rather
// than dropped (page "Support attn sink in fa3", the sink discussion; page
// "TileLang CSA compressed indexer for DSv4", the request to raise instead of
// silently ignoring a document mask).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/hs.h"
#include "hs_common.h"
#include "hs_bwd_args.h"
#include "hs_kernels.h"

namespace {

thread_local std::string g_last_error;

hs_status fail(hs_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

// Validates the problem and fills the kernel geometry.
hs_status prepare(const hs_problem* p, hs::Geom& g) {
  g_last_error.clear();
  if (!p) return fail(HS_ERR_INVALID_ARG, "problem is NULL");
  if (p->batch < 1 || p->seqlen_q < 1 || p->seqlen_kv < 1)
    return fail(HS_ERR_INVALID_ARG, "batch, seqlen_q and seqlen_kv must be >= 1 (got %d, %d, %d)",
                p->batch, p->seqlen_q, p->seqlen_kv);
  if (p->num_heads < 1 || p->head_dim_qk < 1 || p->head_dim_v < 1)
    return fail(HS_ERR_INVALID_ARG, "num_heads, head_dim_qk and head_dim_v must be >= 1");
  if (p->head_dim_v > p->head_dim_qk)
    return fail(HS_ERR_INVALID_ARG,
                "head_dim_v (%d) > head_dim_qk (%d): the value is the leading region of the key",
                p->head_dim_v, p->head_dim_qk);
  if (p->dtype != HS_BF16 && p->dtype != HS_F32)
    return fail(HS_ERR_INVALID_ARG, "dtype %d is not an hs_dtype", p->dtype);
  if (p->block_size != 64)
    return fail(HS_ERR_UNSUPPORTED, "block_size %d: only 64 is built", p->block_size);
  if (!std::isfinite(p->scale))
    return fail(HS_ERR_INVALID_ARG, "scale must be finite");
  if (p->dtype == HS_BF16) {
    if (p->num_heads != 64 || p->head_dim_qk != 576 || p->head_dim_v != 512)
      return fail(HS_ERR_UNSUPPORTED,
                  "bf16 is built for H=64, Dk=576, Dv=512 only (got H=%d, Dk=%d, Dv=%d)",
                  p->num_heads, p->head_dim_qk, p->head_dim_v);
  } else {
    if (p->num_heads > 16 || p->head_dim_qk > 128)
      return fail(HS_ERR_UNSUPPORTED, "f32 is built for H <= 16 and Dk <= 128 (got H=%d, Dk=%d)",
                  p->num_heads, p->head_dim_qk);
  }
  if (p->batch > hs::kMaxBatch)
    return fail(HS_ERR_UNSUPPORTED, "batch %d exceeds %d", p->batch, hs::kMaxBatch);

  std::memset(&g, 0, sizeof(g));
  g.B = p->batch;
  g.Sq = p->seqlen_q;
  g.Skv = p->seqlen_kv;
  g.H = p->num_heads;
  g.Dk = p->head_dim_qk;
  g.Dv = p->head_dim_v;
  g.BS = p->block_size;
  const double scale = p->scale > 0.f ? (double)p->scale : 1.0 / std::sqrt((double)p->head_dim_qk);
  g.scale_log2 = (float)(scale * 1.4426950408889634);

  if (p->kv_lens) {
    if (p->n_kv_lens != p->batch)
      return fail(HS_ERR_INVALID_ARG, "n_kv_lens (%d) != batch (%d)", p->n_kv_lens, p->batch);
    for (int b = 0; b < p->batch; ++b) {
      const int L = p->kv_lens[b];
      if (L < p->seqlen_q || L > p->seqlen_kv)
        return fail(HS_ERR_INVALID_ARG, "kv_lens[%d] = %d outside [seqlen_q=%d, seqlen_kv=%d]", b, L,
                    p->seqlen_q, p->seqlen_kv);
      g.kv_len[b] = L;
    }
  } else {
    if (p->n_kv_lens != 0) return fail(HS_ERR_INVALID_ARG, "n_kv_lens set without kv_lens");
    if (p->seqlen_q > p->seqlen_kv)
      return fail(HS_ERR_INVALID_ARG, "seqlen_q (%d) > seqlen_kv (%d)", p->seqlen_q, p->seqlen_kv);
    for (int b = 0; b < p->batch; ++b) g.kv_len[b] = p->seqlen_kv;
  }

  if (p->doc_bounds_device) {
    // Packing read at run time; n_docs is the capacity (at most 64, one lane
    // of the device lookup each).
    if (p->dtype != HS_BF16)
      return fail(HS_ERR_UNSUPPORTED, "device-resident document bounds are built for bf16 only");
    if (p->doc_start || p->doc_end)
      return fail(HS_ERR_INVALID_ARG, "doc_bounds_device and doc_start/doc_end are exclusive");
    if (p->n_docs < 1)
      return fail(HS_ERR_INVALID_ARG, "doc_bounds_device needs n_docs >= 1 (the capacity)");
    if (p->n_docs > hs::kMaxDocs)
      return fail(HS_ERR_UNSUPPORTED, "n_docs %d exceeds %d", p->n_docs, hs::kMaxDocs);
    if (p->batch != 1 || p->kv_lens || p->kv_lens_device || p->page_table)
      return fail(HS_ERR_INVALID_ARG,
                  "documents require batch == 1 and no kv_lens, kv_lens_device or page_table");
    if (p->seqlen_q != p->seqlen_kv)
      return fail(HS_ERR_INVALID_ARG, "documents require seqlen_q == seqlen_kv");
    if (reinterpret_cast<uintptr_t>(p->doc_bounds_device) % 4 != 0)
      return fail(HS_ERR_INVALID_ARG, "doc_bounds_device is not 4-byte aligned");
    g.n_docs = p->n_docs;
    g.doc_dev = p->doc_bounds_device;
    g.NB = (p->seqlen_q + g.BS - 1) / g.BS + p->n_docs - 1;
  } else if (p->n_docs != 0 || p->doc_start || p->doc_end) {
    if (p->n_docs < 1 || !p->doc_start || !p->doc_end)
      return fail(HS_ERR_INVALID_ARG, "documents need doc_start, doc_end and n_docs >= 1");
    if (p->n_docs > hs::kMaxDocs)
      return fail(HS_ERR_UNSUPPORTED, "n_docs %d exceeds %d", p->n_docs, hs::kMaxDocs);
    if (p->batch != 1 || p->kv_lens)
      return fail(HS_ERR_INVALID_ARG, "documents require batch == 1 and no kv_lens");
    if (p->seqlen_q != p->seqlen_kv)
      return fail(HS_ERR_INVALID_ARG, "documents require seqlen_q == seqlen_kv");
    int expect = 0, blk = 0;
    for (int d = 0; d < p->n_docs; ++d) {
      const int s = p->doc_start[d], e = p->doc_end[d];
      if (s != expect || e <= s)
        return fail(HS_ERR_INVALID_ARG,
                    "documents must tile [0, seqlen) in order: doc %d is [%d, %d), expected start %d",
                    d, s, e, expect);
      g.doc_start[d] = s;
      g.doc_end[d] = e;
      g.doc_blk0[d] = blk;
      blk += (e - s + g.BS - 1) / g.BS;
      expect = e;
    }
    if (expect != p->seqlen_q)
      return fail(HS_ERR_INVALID_ARG, "documents end at %d, seqlen is %d", expect, p->seqlen_q);
    g.doc_blk0[p->n_docs] = blk;
    g.n_docs = p->n_docs;
    g.NB = blk;
  } else {
    int nb = 0;
    for (int b = 0; b < p->batch; ++b) nb = std::max(nb, (g.kv_len[b] + g.BS - 1) / g.BS);
    g.NB = nb;
  }

  if (p->kv_lens_device) {
    if (p->dtype != HS_BF16)
      return fail(HS_ERR_UNSUPPORTED, "device-resident lengths are built for bf16 only");
    if (g.n_docs != 0)
      return fail(HS_ERR_INVALID_ARG, "kv_lens_device does not take documents");
    if (p->kv_lens)
      return fail(HS_ERR_INVALID_ARG, "kv_lens and kv_lens_device are exclusive");
    if (reinterpret_cast<uintptr_t>(p->kv_lens_device) % 4 != 0)
      return fail(HS_ERR_INVALID_ARG, "kv_lens_device is not 4-byte aligned");
    g.kv_len_dev = p->kv_lens_device;  // kv_len[] keeps the capacity seqlen_kv
  }
  if (p->page_table || p->max_pages != 0) {
    if (!p->page_table || p->max_pages < 1)
      return fail(HS_ERR_INVALID_ARG, "paged KV needs page_table and max_pages >= 1");
    if (reinterpret_cast<uintptr_t>(p->page_table) % 4 != 0)
      return fail(HS_ERR_INVALID_ARG, "page_table is not 4-byte aligned");
    if (p->dtype != HS_BF16) return fail(HS_ERR_UNSUPPORTED, "paged KV is built for bf16 only");
    if (g.n_docs != 0) return fail(HS_ERR_INVALID_ARG, "paged KV does not take documents");
    for (int b = 0; b < p->batch; ++b)
      if (g.kv_len[b] > p->max_pages * g.BS)
        return fail(HS_ERR_INVALID_ARG, "entry %d holds %d keys, more than max_pages * %d", b,
                    g.kv_len[b], g.BS);
  }
  return HS_OK;
}

// Key-range split for few rows (decode): rows are cut into chunks of the same
// number of tiles, sized so that about 512 workgroups have work (two per CU),
// with at least 4 tiles per chunk and at most 64 chunks per row. Long rows get
// more chunks than short ones; chunks past the end of a row are empty and
// their workgroups exit at once. The gather's tile count is data dependent,
// so top_k stands in for it.
struct SplitPlan {
  int nsplit, tiles;
};

// max_ws bounds the partials' workspace: past it, rows take fewer, longer
// chunks.
SplitPlan plan_split(const hs::Geom& g, int op, int top_k, int window,
                     size_t max_ws = SIZE_MAX) {
  SplitPlan sp{1, 0};
  if (g.Dk != 576 || g.doc_dev != nullptr) return sp;   // the host cannot see device documents
  const int items = g.B * g.Sq;
  if (items >= 512) return sp;
  long total = 0;
  int longest = 1;
  for (int b = 0; b < g.B; ++b)
    for (int r = 0; r < g.Sq; ++r) {
      int n;
      if (op == HS_OP_SPARSE_GATHER) {
        n = top_k;
      } else {
        const hs::RowRange rr = hs::row_range(g, op == HS_OP_SWA ? hs::kSwa : hs::kScore, b, r,
                                              window);
        n = rr.j_last - rr.j_first + 1;
      }
      total += n;
      longest = std::max(longest, n);
    }
  int tiles = (int)std::max<long>(4, (total + 511) / 512);
  tiles = std::max(tiles, (longest + 63) / 64);
  int ns = (longest + tiles - 1) / tiles;
  const size_t per_split = (size_t)g.B * g.Sq * g.H * (g.Dv + 2) * sizeof(float);
  if (ns > 1 && (size_t)ns * per_split > max_ws) {
    ns = (int)std::min<size_t>(max_ws / per_split, (size_t)ns);
    if (ns > 1) {
      tiles = (longest + ns - 1) / ns;
      ns = (longest + tiles - 1) / tiles;
    }
  }
  if (ns > 1) sp = SplitPlan{ns, tiles};
  return sp;
}

size_t split_ws_bytes(const hs::Geom& g, int nsplit) {
  if (nsplit <= 1) return 0;
  const size_t slots = (size_t)g.B * g.Sq * nsplit * g.H;
  return slots * (size_t)g.Dv * sizeof(float) + slots * 2 * sizeof(float);
}

hs_status check_ptr(const void* ptr, const char* name, unsigned align = 16) {
  if (!ptr) return fail(HS_ERR_INVALID_ARG, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(ptr) % align != 0)
    return fail(HS_ERR_INVALID_ARG, "%s is not %u-byte aligned", name, align);
  return HS_OK;
}

hs_status hip_status(int err, const char* what) {
  if (err != 0)
    return fail(HS_ERR_HIP, "%s: %s", what, hipGetErrorString(static_cast<hipError_t>(err)));
  return HS_OK;
}

// Library-owned workspace of the no-allocation entry point: the split-decode
// partials of hs_block_score_topk_fwd_noalloc live here. Every GPU the library
// runs on holds its own copy until the process ends; host code uses the
// device address hipGetSymbolAddress returns, never the array's name.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

// Device address of this device's scratch array, looked up once per device
// (with that device current) and kept; nullptr and a message on failure.
void* scratch_ptr() {
  static std::mutex mu;
  static void* ptrs[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    fail(HS_ERR_HIP, "hipGetDevice failed or device index out of range");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      fail(HS_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      return nullptr;
    }
    ptrs[dev] = ptr;
  }
  return ptrs[dev];
}

// sel_idx (score operation only): also select each row's top sel_k blocks,
// and with sel_prob write the normalised block scores.
// use_scratch: plan the split within kScratchBytes and take the partials'
// workspace from the library's scratch array (ws and ws_bytes are ignored).
hs_status launch_attn(int op, const hs_problem* p, const void* q, const void* kv, const float* sink,
                      const int32_t* block_idx, int32_t top_k, int32_t window, void* out,
                      float* lse, float* block_logit, void* ws, size_t ws_bytes, void* stream,
                      int32_t* sel_idx = nullptr, int32_t sel_k = 0, float* sel_prob = nullptr,
                      bool use_scratch = false) {
  hs::Geom g;
  hs_status st = prepare(p, g);
  if (st != HS_OK) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(kv, "kv")) || (st = check_ptr(out, "out")) ||
      (st = check_ptr(lse, "lse", 4)))
    return st;
  if (op == HS_OP_BLOCK_SCORE && (st = check_ptr(block_logit, "block_logit", 4))) return st;
  if (sel_idx != nullptr || sel_k != 0) {
    if ((st = check_ptr(sel_idx, "block_idx", 4))) return st;
    if (sel_k < 1) return fail(HS_ERR_INVALID_ARG, "top_k must be >= 1 (got %d)", sel_k);
    if (sel_k > 64) return fail(HS_ERR_UNSUPPORTED, "top_k %d exceeds 64", sel_k);
    if (g.NB > 4096) return fail(HS_ERR_UNSUPPORTED, "%d blocks exceed 4096", g.NB);
  }
  if (sel_prob && (st = check_ptr(sel_prob, "block_prob", 4))) return st;
  if (op == HS_OP_SPARSE_GATHER) {
    if ((st = check_ptr(block_idx, "block_idx", 4))) return st;
    if (top_k < 1) return fail(HS_ERR_INVALID_ARG, "top_k must be >= 1 (got %d)", top_k);
    if (top_k > 64) return fail(HS_ERR_UNSUPPORTED, "top_k %d exceeds 64", top_k);
  }
  if (op == HS_OP_SWA && window < 1)
    return fail(HS_ERR_INVALID_ARG, "window must be >= 1 (got %d)", window);
  if (sink && reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return fail(HS_ERR_INVALID_ARG, "sink is not 4-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g.Sq * g.B == 0) return HS_OK;

  if (p->dtype == HS_BF16) {
    const SplitPlan sp =
        plan_split(g, op, top_k, window, use_scratch ? kScratchBytes : SIZE_MAX);
    const int nsplit = sp.nsplit;
    const size_t need = split_ws_bytes(g, nsplit);
    if (use_scratch) {
      if (need > kScratchBytes)
        return fail(HS_ERR_UNSUPPORTED, "partials of %zu bytes exceed the %zu-byte scratch array",
                    need, kScratchBytes);
      ws = need > 0 ? scratch_ptr() : nullptr;
      if (need > 0 && !ws) return HS_ERR_HIP;
      ws_bytes = kScratchBytes;
    }
    if (need > 0 && (!ws || ws_bytes < need))
      return fail(HS_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                  ws ? ws_bytes : (size_t)0);
    if (need > 0 && reinterpret_cast<uintptr_t>(ws) % 16 != 0)
      return fail(HS_ERR_WORKSPACE, "workspace is not 16-byte aligned");
    hs::AttnArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = static_cast<const __bf16*>(q);
    a.kv = static_cast<const __bf16*>(kv);
    a.sink = sink;
    a.out = static_cast<__bf16*>(out);
    a.lse = lse;
    a.block_logit = block_logit;
    a.block_idx = block_idx;
    a.top_k = top_k;
    a.window = window;
    a.nsplit = nsplit;
    a.split_tiles = sp.tiles;
    if (nsplit > 1) {
      const size_t slots = (size_t)g.B * g.Sq * nsplit * g.H;
      a.ws_o = static_cast<float*>(ws);
      a.ws_ml = static_cast<float*>(ws) + slots * g.Dv;
    }
    a.page_table = p->page_table;
    a.max_pages = p->page_table ? p->max_pages : 0;
    a.topk_idx = sel_idx;
    a.topk_k = sel_k;
    a.topk_prob = sel_prob;
    a.g = g;
    return hip_status(hs::attn_bf16_launch(op, a, s), "attention launch");
  }
  hs::AttnF32Args a;
  std::memset(&a, 0, sizeof(a));
  a.q = static_cast<const float*>(q);
  a.kv = static_cast<const float*>(kv);
  a.sink = sink;
  a.out = static_cast<float*>(out);
  a.lse = lse;
  a.block_logit = block_logit;
  a.block_idx = block_idx;
  a.top_k = top_k;
  a.window = window;
  a.g = g;
  st = hip_status(hs::attn_f32_launch(op, a, s), "attention launch");
  if (st != HS_OK || sel_idx == nullptr) return st;
  hs::TopkArgs t;
  std::memset(&t, 0, sizeof(t));
  t.block_logit = block_logit;
  t.block_idx = sel_idx;
  t.top_k = sel_k;
  t.lse = lse;
  t.block_prob = sel_prob;
  t.g = g;
  return hip_status(hs::topk_launch(t, s), "top-k launch");
}

// Gradients of one attention operation (op: HS_OP_BLOCK_SCORE, _SPARSE_GATHER
// or _SWA; the matching _BWD workspace).
hs_status launch_bwd(int op, const hs_problem* p, const void* q, const void* kv,
                     const float* sink, const int32_t* block_idx, int32_t top_k, int32_t window,
                     const void* out, const float* lse, const void* dout, const float* dlse,
                     float* dq, float* dkv, float* dsink, void* ws, size_t ws_bytes,
                     void* stream) {
  hs::Geom g;
  hs_status st = prepare(p, g);
  if (st != HS_OK) return st;
  if (p->page_table || p->kv_lens_device || p->doc_bounds_device)
    return fail(HS_ERR_UNSUPPORTED,
                "gradients take a contiguous kv with host lengths and documents (no paged KV)");
  if ((st = check_ptr(q, "q")) || (st = check_ptr(kv, "kv")) || (st = check_ptr(out, "out")) ||
      (st = check_ptr(lse, "lse", 4)) || (st = check_ptr(dout, "dout")) ||
      (st = check_ptr(dq, "dq")) || (st = check_ptr(dkv, "dkv")))
    return st;
  if (sink && reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return fail(HS_ERR_INVALID_ARG, "sink is not 4-byte aligned");
  if (dlse && reinterpret_cast<uintptr_t>(dlse) % 4 != 0)
    return fail(HS_ERR_INVALID_ARG, "dlse is not 4-byte aligned");
  if (dsink) {
    if (!sink) return fail(HS_ERR_INVALID_ARG, "dsink is set but there is no sink");
    if ((st = check_ptr(dsink, "dsink", 4))) return st;
  }
  if (op == HS_OP_SPARSE_GATHER) {
    if ((st = check_ptr(block_idx, "block_idx", 4))) return st;
    if (top_k < 1) return fail(HS_ERR_INVALID_ARG, "top_k must be >= 1 (got %d)", top_k);
    if (top_k > 64) return fail(HS_ERR_UNSUPPORTED, "top_k %d exceeds 64", top_k);
    if ((long)g.B * g.Sq * top_k > 0x7fffffffL)
      return fail(HS_ERR_UNSUPPORTED, "batch * seqlen_q * top_k exceeds 2^31 - 1");
    if (g.NB > 4096) return fail(HS_ERR_UNSUPPORTED, "%d blocks exceed 4096", g.NB);
  }
  if (op == HS_OP_SWA && window < 1)
    return fail(HS_ERR_INVALID_ARG, "window must be >= 1 (got %d)", window);
  const bool bf16 = p->dtype == HS_BF16;
  const int kop = op == HS_OP_SWA ? hs::kSwa : op == HS_OP_SPARSE_GATHER ? hs::kGather : hs::kScore;
  // The stored-score path (bf16) runs when the workspace also holds the score
  // gradients; otherwise dq recomputes them.
  hs::BwdLayout L = hs::bwd_layout(g, kop, top_k, window, false);
  if (bf16 && ws) {
    const hs::BwdLayout Ls = hs::bwd_layout(g, kop, top_k, window, true);
    if (ws_bytes >= Ls.total) L = Ls;
  }
  if (!ws || ws_bytes < L.total)
    return fail(HS_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", L.total,
                ws ? ws_bytes : (size_t)0);
  if (reinterpret_cast<uintptr_t>(ws) % 16 != 0)
    return fail(HS_ERR_WORKSPACE, "workspace is not 16-byte aligned");
  char* w = static_cast<char*>(ws);
  hs::BwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.kv = kv;
  a.sink = sink;
  a.out = out;
  a.lse = lse;
  a.dout = dout;
  a.dlse = dlse;
  a.block_idx = block_idx;
  a.top_k = top_k;
  a.window = window;
  a.dq = dq;
  a.dkv = dkv;
  a.dsink = dsink;
  a.dsum = reinterpret_cast<float*>(w + L.dsum);
  a.sink_part = reinterpret_cast<float*>(w + L.sink_part);
  a.n_pre = L.n_pre;
  a.rows_per_pre = L.rows_per_pre;
  {
    a.plan_first = reinterpret_cast<int*>(w + L.first);
    a.plan_nrows = reinterpret_cast<int*>(w + L.nrows);
    a.plan_pre = reinterpret_cast<int*>(w + L.pre);
    if (kop == hs::kGather) {
      a.g_cnt = reinterpret_cast<int*>(w + L.cnt);
      a.g_total = reinterpret_cast<int*>(w + L.total_g);
      a.g_off = reinterpret_cast<int*>(w + L.off_g);
      a.g_rows = reinterpret_cast<int*>(w + L.rows);
      if (L.store_ds) a.g_pos = reinterpret_cast<int*>(w + L.pos);
    }
    a.part = reinterpret_cast<float*>(w + L.part);
    if (L.store_ds) {
      a.ds_entry = reinterpret_cast<long long*>(w + L.ds_entry);
      a.ds_dummy = reinterpret_cast<__bf16*>(w + L.ds_dummy);
      a.ds_tiles = reinterpret_cast<__bf16*>(w + L.ds_tiles);
      a.ds_stride = L.ds_stride;
    }
    a.chunk_rows = L.chunk_rows;
    a.n_chunks = L.n_chunks;
    a.items = L.items;
    a.split_rows = L.split_rows;
    a.row_tiles = L.row_tiles;
  }
  a.g = g;
  return hip_status(hs::bwd_launch(kop, a, bf16, static_cast<hipStream_t>(stream)),
                    "gradient launch");
}

}  // namespace

extern "C" {

int32_t hs_version(void) { return 202; }

const char* hs_status_string(int32_t status) {
  switch (status) {
    case HS_OK: return "HS_OK";
    case HS_ERR_INVALID_ARG: return "HS_ERR_INVALID_ARG";
    case HS_ERR_UNSUPPORTED: return "HS_ERR_UNSUPPORTED";
    case HS_ERR_HIP: return "HS_ERR_HIP";
    case HS_ERR_WORKSPACE: return "HS_ERR_WORKSPACE";
    default: return "HS_UNKNOWN_STATUS";
  }
}

const char* hs_last_error(void) { return g_last_error.c_str(); }

int32_t hs_num_blocks(const hs_problem* p) {
  hs::Geom g;
  const hs_status st = prepare(p, g);
  return st == HS_OK ? g.NB : (int32_t)st;
}

hs_status hs_workspace_size(const hs_problem* p, int32_t op, int32_t top_k, int32_t window,
                            size_t* bytes) {
  hs::Geom g;
  hs_status st = prepare(p, g);
  if (st != HS_OK) return st;
  if (!bytes) return fail(HS_ERR_INVALID_ARG, "bytes is NULL");
  if (op < HS_OP_BLOCK_SCORE || op > HS_OP_SPARSE_GATHER_BWD_STORE_DS)
    return fail(HS_ERR_INVALID_ARG, "unknown op %d", op);
  if (op == HS_OP_SWA_SPARSE) {
    // the two branches run one after the other when they do not run as one
    // pass, so the larger of their workspaces serves both
    if (top_k < 1) return fail(HS_ERR_INVALID_ARG, "top_k must be >= 1 (got %d)", top_k);
    if (top_k > 64) return fail(HS_ERR_UNSUPPORTED, "top_k %d exceeds 64", top_k);
    if (window < 1) return fail(HS_ERR_INVALID_ARG, "window must be >= 1 (got %d)", window);
    *bytes = p->dtype == HS_BF16
                 ? std::max(split_ws_bytes(g, plan_split(g, HS_OP_SWA, top_k, window).nsplit),
                            split_ws_bytes(g, plan_split(g, HS_OP_SPARSE_GATHER, top_k, window).nsplit))
                 : 0;
    return HS_OK;
  }
  if (op >= HS_OP_BLOCK_SCORE_BWD) {
    if (p->doc_bounds_device)
      return fail(HS_ERR_UNSUPPORTED, "gradients take host document bounds");
    const int kop = (op == HS_OP_SWA_BWD || op == HS_OP_SWA_BWD_STORE_DS) ? hs::kSwa
                    : (op == HS_OP_SPARSE_GATHER_BWD || op == HS_OP_SPARSE_GATHER_BWD_STORE_DS)
                        ? hs::kGather
                        : hs::kScore;
    if (kop == hs::kGather && top_k < 1)
      return fail(HS_ERR_INVALID_ARG, "top_k must be >= 1 (got %d)", top_k);
    if (kop == hs::kGather && top_k > 64)
      return fail(HS_ERR_UNSUPPORTED, "top_k %d exceeds 64", top_k);
    if (kop == hs::kSwa && window < 1)
      return fail(HS_ERR_INVALID_ARG, "window must be >= 1 (got %d)", window);
    const bool store = (op == HS_OP_BLOCK_SCORE_BWD_STORE_DS || op == HS_OP_SWA_BWD_STORE_DS ||
                        op == HS_OP_SPARSE_GATHER_BWD_STORE_DS) &&
                       p->dtype == HS_BF16;
    *bytes = hs::bwd_layout(g, kop, top_k, window, store).total;
    return HS_OK;
  }
  *bytes = p->dtype == HS_BF16 ? split_ws_bytes(g, plan_split(g, op, top_k, window).nsplit) : 0;
  return HS_OK;
}

hs_status hs_block_score_fwd(const hs_problem* p, const void* q, const void* kv, const float* sink,
                             void* out, float* lse, float* block_logit, void* ws, size_t ws_bytes,
                             void* stream) {
  return launch_attn(HS_OP_BLOCK_SCORE, p, q, kv, sink, nullptr, 0, 0, out, lse, block_logit, ws,
                     ws_bytes, stream);
}

hs_status hs_block_score_topk_fwd(const hs_problem* p, const void* q, const void* kv,
                                  const float* sink, int32_t top_k, void* out, float* lse,
                                  float* block_logit, int32_t* block_idx, float* block_prob,
                                  void* ws, size_t ws_bytes, void* stream) {
  return launch_attn(HS_OP_BLOCK_SCORE, p, q, kv, sink, nullptr, 0, 0, out, lse, block_logit, ws,
                     ws_bytes, stream, block_idx, top_k, block_prob);
}

hs_status hs_block_score_topk_fwd_noalloc(const hs_problem* p, const void* q, const void* kv,
                                          const float* sink, int32_t top_k, void* out, float* lse,
                                          float* block_logit, int32_t* block_idx,
                                          float* block_prob, void* stream) {
  return launch_attn(HS_OP_BLOCK_SCORE, p, q, kv, sink, nullptr, 0, 0, out, lse, block_logit,
                     nullptr, 0, stream, block_idx, top_k, block_prob, true);
}

hs_status hs_swa_sparse_fwd(const hs_problem* p, const void* q, const void* kv, const float* sink,
                            int32_t window, const int32_t* block_idx, int32_t top_k, void* out_swa,
                            float* lse_swa, void* out_sparse, float* lse_sparse,
                            const float* gate_swa, const float* gate_sparse, void* out_mix,
                            void* ws, size_t ws_bytes, void* stream) {
  hs::Geom g;
  hs_status st = prepare(p, g);
  if (st != HS_OK) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(kv, "kv")) ||
      (st = check_ptr(out_swa, "out_swa")) || (st = check_ptr(lse_swa, "lse_swa", 4)) ||
      (st = check_ptr(out_sparse, "out_sparse")) || (st = check_ptr(lse_sparse, "lse_sparse", 4)) ||
      (st = check_ptr(block_idx, "block_idx", 4)))
    return st;
  if (top_k < 1) return fail(HS_ERR_INVALID_ARG, "top_k must be >= 1 (got %d)", top_k);
  if (top_k > 64) return fail(HS_ERR_UNSUPPORTED, "top_k %d exceeds 64", top_k);
  if (window < 1) return fail(HS_ERR_INVALID_ARG, "window must be >= 1 (got %d)", window);
  if (sink && reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return fail(HS_ERR_INVALID_ARG, "sink is not 4-byte aligned");
  const bool mix = gate_swa || gate_sparse || out_mix;
  if (mix && ((st = check_ptr(gate_swa, "gate_swa", 4)) || (st = check_ptr(gate_sparse, "gate_sparse", 4)) ||
              (st = check_ptr(out_mix, "out_mix"))))
    return st;
  // One pass over both branches on the in-place bf16 path when neither splits
  // its key range; otherwise the two operations, one after the other.
  const bool one_pass = p->dtype == HS_BF16 && !p->page_table && !p->kv_lens_device &&
                        plan_split(g, HS_OP_SWA, top_k, window).nsplit == 1 &&
                        plan_split(g, HS_OP_SPARSE_GATHER, top_k, window).nsplit == 1;
  if (!one_pass) {
    st = launch_attn(HS_OP_SWA, p, q, kv, sink, nullptr, 0, window, out_swa, lse_swa, nullptr, ws,
                     ws_bytes, stream);
    if (st != HS_OK) return st;
    st = launch_attn(HS_OP_SPARSE_GATHER, p, q, kv, sink, block_idx, top_k, 0, out_sparse,
                     lse_sparse, nullptr, ws, ws_bytes, stream);
    if (st != HS_OK || !mix) return st;
    hs::MixArgs m;
    m.a = out_swa;
    m.b = out_sparse;
    m.ga = gate_swa;
    m.gb = gate_sparse;
    m.out = out_mix;
    m.rows = (long long)g.B * g.Sq * g.H;
    m.dv = g.Dv;
    m.bf16 = p->dtype == HS_BF16 ? 1 : 0;
    return hip_status(hs::mix_launch(m, static_cast<hipStream_t>(stream)), "mix launch");
  }
  if (g.Sq * g.B == 0) return HS_OK;
  hs::AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = static_cast<const __bf16*>(q);
  a.kv = static_cast<const __bf16*>(kv);
  a.sink = sink;
  a.out = static_cast<__bf16*>(out_sparse);
  a.lse = lse_sparse;
  a.out2 = static_cast<__bf16*>(out_swa);
  a.lse2 = lse_swa;
  a.gate_a = gate_swa;
  a.gate_b = gate_sparse;
  a.out_mix = static_cast<__bf16*>(out_mix);
  a.block_idx = block_idx;
  a.top_k = top_k;
  a.window = window;
  a.nsplit = 1;
  a.g = g;
  return hip_status(hs::attn_bf16_launch(hs::kSwaSparse, a, static_cast<hipStream_t>(stream)),
                    "attention launch");
}

hs_status hs_sparse_gather_fwd(const hs_problem* p, const void* q, const void* kv,
                               const float* sink, const int32_t* block_idx, int32_t top_k,
                               void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return launch_attn(HS_OP_SPARSE_GATHER, p, q, kv, sink, block_idx, top_k, 0, out, lse, nullptr,
                     ws, ws_bytes, stream);
}

hs_status hs_swa_fwd(const hs_problem* p, const void* q, const void* kv, const float* sink,
                     int32_t window, void* out, float* lse, void* ws, size_t ws_bytes,
                     void* stream) {
  return launch_attn(HS_OP_SWA, p, q, kv, sink, nullptr, 0, window, out, lse, nullptr, ws, ws_bytes,
                     stream);
}

hs_status hs_topk_blocks(const hs_problem* p, const float* block_logit, int32_t top_k,
                         int32_t* block_idx, void* stream) {
  hs::Geom g;
  hs_status st = prepare(p, g);
  if (st != HS_OK) return st;
  if ((st = check_ptr(block_logit, "block_logit", 4)) || (st = check_ptr(block_idx, "block_idx", 4)))
    return st;
  if (top_k < 1) return fail(HS_ERR_INVALID_ARG, "top_k must be >= 1 (got %d)", top_k);
  if (top_k > 64) return fail(HS_ERR_UNSUPPORTED, "top_k %d exceeds 64", top_k);
  if (g.NB > 4096) return fail(HS_ERR_UNSUPPORTED, "%d blocks exceed 4096", g.NB);
  hs::TopkArgs a;
  std::memset(&a, 0, sizeof(a));
  a.block_logit = block_logit;
  a.block_idx = block_idx;
  a.top_k = top_k;
  a.g = g;
  return hip_status(hs::topk_launch(a, static_cast<hipStream_t>(stream)), "top-k launch");
}

hs_status hs_block_score_bwd(const hs_problem* p, const void* q, const void* kv, const float* sink,
                             const void* out, const float* lse, const void* dout,
                             const float* dlse, float* dq, float* dkv, float* dsink, void* ws,
                             size_t ws_bytes, void* stream) {
  return launch_bwd(HS_OP_BLOCK_SCORE, p, q, kv, sink, nullptr, 0, 0, out, lse, dout, dlse, dq,
                    dkv, dsink, ws, ws_bytes, stream);
}

hs_status hs_sparse_gather_bwd(const hs_problem* p, const void* q, const void* kv,
                               const float* sink, const int32_t* block_idx, int32_t top_k,
                               const void* out, const float* lse, const void* dout,
                               const float* dlse, float* dq, float* dkv, float* dsink, void* ws,
                               size_t ws_bytes, void* stream) {
  return launch_bwd(HS_OP_SPARSE_GATHER, p, q, kv, sink, block_idx, top_k, 0, out, lse, dout,
                    dlse, dq, dkv, dsink, ws, ws_bytes, stream);
}

hs_status hs_swa_bwd(const hs_problem* p, const void* q, const void* kv, const float* sink,
                     int32_t window, const void* out, const float* lse, const void* dout,
                     const float* dlse, float* dq, float* dkv, float* dsink, void* ws,
                     size_t ws_bytes, void* stream) {
  return launch_bwd(HS_OP_SWA, p, q, kv, sink, nullptr, 0, window, out, lse, dout, dlse, dq, dkv,
                    dsink, ws, ws_bytes, stream);
}

}  // extern "C"
