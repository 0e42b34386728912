// Gradients of the three attention operations of the HySparse MQA path:
// causal attention (the attention half of the block-score operation),
// block-sparse gather attention and sliding-window attention, each with the
// optional learnable per-head sink (page "HySparse MQA sparse attention (FA4
// block scoring + SWA MQA + block-sparse DSA gather)", section "Core": block
// scoring with gradients routed through the autograd layer, the analytic
// gradient of the sink; per-file table rows for windowed_mqa_attn*.py and
// block_sparse_mqa_dsa.py). The block scores take no gradient (review of
// PaddleFleet PR 1453, block-score PyLayer comments: the backward returns
// gradients for q, k and v only).
//
// For one row and head, with P_i = exp(s_i - lse) and Dsum = dout . out:
//   dS_i = P_i (dout . v_i - Dsum),           dq = scale sum_i dS_i k_i,
//   dkv_i += scale dS_i q + [P_i dout, 0],    dsink = -sum_rows exp(sigma - lse) Dsum
// (the latent row is both key and value: its key and value gradients add).
//
// Launch sequence (one stream):
//   pre     : Dsum per (row, head) and per-workgroup sink partials
//   sink    : fixed-order sum of the partials (when a sink gradient is asked)
//   plan    : rows reaching each key block, split into work items (the gather
//             first counts and lists, per block, the rows that selected it)
//   dq      : one workgroup per query row, walking the row's key tiles
//   dkv     : one workgroup per (key block, chunk of rows): partial gradients
//   reduce  : fixed-order sum of each block's partials into dkv
// With the larger causal or window workspace, dkv runs first and also stores
// the bf16 score gradients dS, and dq (one workgroup per pair of rows) reads
// them instead of recomputing the scores (bwd_dq_ds_bf16_kernel).
// Every workspace word is written before it is read (no memset), and every
// sum runs in a fixed order, so results are reproducible bit for bit.
//
// bf16 MFMA kernels (absorbed-MLA shape H = 64, Dk = 576, Dv = 512; page
// above, section "FlashMLA sparse kernel constraints"). The 16x16x32 bf16
// MFMA contracts 32 along k; lane l holds A[l%16][8(l/16)..+8],
// B[8(l/16)..+8][l%16] and D[4(l/16)..+4][l%16].
//   dq kernel (wave w owns heads 16w..16w+15, Q and dout rows in registers):
//     S^T[key, head]  = K_tile . Q^T    (A = K from LDS, B = Q)
//     dP^T[key, head] = V_tile . dout^T (the same K fragments: V is the
//                       leading 512 columns of the latent row)
//     dQ^T[dim, head] += K^T . dS^T     (A = K^T by LDS transpose reads,
//                       B = dS^T straight from the S^T registers; inside each
//                       32-key k-step both operands use one key permutation)
//   dkv kernel (wave w owns keys 16w..16w+15 of the block, K in registers):
//     per query row, two stages of 32 heads each: (Q, dout) half rows are
//     staged in LDS, double-buffered;
//     S[head, key]  = Q . K^T,   dP[head, key] = dout . V^T  (B = K registers)
//     dKV^T[dim, key] += Q^T . dS + [dout^T . P, 0]         (A by transpose reads)
// LDS tiles use the swizzled 64-column-group layout of hs_gfx950.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <utility>

#include "hs_common.h"
#include "hs_gfx950.h"
#include "hs_bwd_args.h"
#include "hs_bwd_plan.h"

namespace hs {

namespace {

namespace bw {
constexpr int H = 64, DK = 576, DV = 512, BS = 64, NT = 256;
constexpr int KSTEPS = DK / 32;     // 18
constexpr int VSTEPS = DV / 32;     // 16
constexpr int DBK = DK / 16;        // 36 column blocks of a latent row
constexpr int DBV = DV / 16;        // 32 column blocks of a value row
constexpr int GR = BS * 128;        // column group of a 64-row tile
constexpr int TILE = 9 * GR;        // 73728
constexpr int HGR = 32 * 128;       // column group of a 32-row half tile
constexpr int QH = 9 * HGR;         // 36864: 32 Q rows
constexpr int STAGE = QH + 8 * HGR; // + 32 dout rows = 69632
}  // namespace bw

constexpr int kMaxHeads = 64;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Operand stream: NF LDS fragments consumed in order, each requested LA
// places ahead of its use into its own ring register, so that LA reads are in
// flight while the MFMAs run (LDS reads complete in order; the compiler's
// wait for fragment i then leaves the later ones pending). pre(i) runs before
// fragment i is used; the scheduling barrier keeps this order.
template <int NF, int LA, typename Load, typename Use, typename Pre>
__device__ __forceinline__ void operand_stream(Load&& load, Use&& use, Pre&& pre) {
  constexpr int RB = LA + 1;
  bf16x8 fr[RB];
  static_for<LA>([&](auto F) __attribute__((always_inline)) {
    constexpr int f = decltype(F)::value;
    fr[f % RB] = load(F);
    __builtin_amdgcn_sched_barrier(0);
  });
  static_for<NF>([&](auto I) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value;
    pre(I);
    use(I, fr[i % RB]);
    if constexpr (i + LA < NF) fr[(i + LA) % RB] = load(std::integral_constant<int, i + LA>{});
    __builtin_amdgcn_sched_barrier(0);
  });
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ---------------------------------------------------------------------------
// Dsum and the sink-gradient partials.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ float dot_row(const T* x, const T* y, int n, int lane);

template <>
__device__ __forceinline__ float dot_row<bf16>(const bf16* x, const bf16* y, int n, int lane) {
  float s = 0.f;
  for (int d = 8 * lane; d < n; d += 512) {
    const bf16x8 a = *(const bf16x8*)(x + d);
    const bf16x8 b = *(const bf16x8*)(y + d);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf((float)a[e], (float)b[e], s);
  }
  return s;
}

template <>
__device__ __forceinline__ float dot_row<float>(const float* x, const float* y, int n, int lane) {
  float s = 0.f;
  for (int d = lane; d < n; d += 64) s = fmaf(x[d], y[d], s);
  return s;
}

// Workgroup w handles rows [w R, w R + R); each wave takes (row, head) pairs
// in turn and reduces one dot product across its lanes.
template <typename T>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  __shared__ float sacc[4][kMaxHeads];
  const Geom& g = a.g;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = g.H, Dv = g.Dv;
  const size_t rows = (size_t)g.B * g.Sq;
  const size_t r0 = (size_t)blockIdx.x * a.rows_per_pre;
  if (lane < H) sacc[wave][lane] = 0.f;
  const T* out = static_cast<const T*>(a.out);
  const T* dout = static_cast<const T*>(a.dout);
  for (int p = wave; p < a.rows_per_pre * H; p += 4) {
    const size_t row = r0 + p / H;
    const int h = p % H;
    if (row >= rows) break;
    const size_t off = (row * H + h) * (size_t)Dv;
    // An incoming gradient of lse enters every later formula as D - dlse.
    float d = wave_sum(dot_row<T>(out + off, dout + off, Dv, lane));
    if (a.dlse != nullptr) d -= a.dlse[row * H + h];
    if (lane == 0) {
      a.dsum[row * H + h] = d;
      if (a.sink != nullptr) {
        const float lse = a.lse[row * H + h];
        if (lse > -INFINITY) sacc[wave][h] -= __builtin_amdgcn_exp2f((a.sink[h] - lse) * kLog2e) * d;
      }
    }
  }
  __syncthreads();
  if (a.dsink != nullptr && threadIdx.x < (unsigned)H) {
    const int h = threadIdx.x;
    a.sink_part[(size_t)blockIdx.x * H + h] = ((sacc[0][h] + sacc[1][h]) + sacc[2][h]) + sacc[3][h];
  }
}

// One workgroup per head: thread t sums partials t, t + 256, .. in order,
// then a fixed tree over the 256 threads.
__global__ __launch_bounds__(256) void bwd_sink_kernel(BwdArgs a) {
  __shared__ float red[256];
  const int h = blockIdx.x, t = threadIdx.x;
  float s = 0.f;
  for (int w = t; w < a.n_pre; w += 256) s += a.sink_part[(size_t)w * a.g.H + h];
  red[t] = s;
  __syncthreads();
  for (int k = 128; k >= 1; k >>= 1) {
    if (t < k) red[t] += red[t + k];
    __syncthreads();
  }
  if (t == 0) a.dsink[h] = red[0];
}

// ---------------------------------------------------------------------------
// Work plan of the key-block gradient.
// ---------------------------------------------------------------------------
// Gather: counts of each block's selecting rows per tile of 64 rows.
__global__ __launch_bounds__(256) void bwd_gcount_kernel(BwdArgs a) {
  __shared__ int hist[4096];
  const Geom& g = a.g;
  const int T = a.row_tiles;
  const int b = blockIdx.x / T, tile = blockIdx.x % T;
  for (int j = threadIdx.x; j < g.NB; j += 256) hist[j] = 0;
  __syncthreads();
  const int nb_b = nb_of_entry(g, b);
  const int K = a.top_k;
  for (int e = threadIdx.x; e < 64 * K; e += 256) {
    const int r = tile * 64 + e / K;
    if (r >= g.Sq) continue;
    const int j = a.block_idx[((size_t)b * g.Sq + r) * K + e % K];
    const RowRange rr = row_range(g, kGather, b, r, 0);
    if (gather_hit(g, b, nb_b, rr, j)) atomicAdd(&hist[j], 1);
  }
  __syncthreads();
  int* cnt = a.g_cnt + ((size_t)b * T + tile) * g.NB;
  for (int j = threadIdx.x; j < g.NB; j += 256) cnt[j] = hist[j];
}

// Gather: per block, exclusive prefix of the tile counts (in place) and the
// block's total.
__global__ __launch_bounds__(256) void bwd_gscan_kernel(BwdArgs a) {
  const Geom& g = a.g;
  const int f = blockIdx.x * 256 + threadIdx.x;
  if (f >= g.B * g.NB) return;
  const int b = f / g.NB, j = f % g.NB;
  int run = 0;
  for (int t = 0; t < a.row_tiles; ++t) {
    int* c = a.g_cnt + ((size_t)b * a.row_tiles + t) * g.NB + j;
    const int v = *c;
    *c = run;
    run += v;
  }
  a.g_total[f] = run;
}

// Work items of the key-block gradient (one workgroup): the gather's list
// offsets first, then the rows of every (b, c, j) and the item prefix. Each
// thread takes a contiguous segment; the segment totals are scanned in LDS.
__global__ __launch_bounds__(256) void bwd_plan_kernel(BwdArgs a, int op) {
  __shared__ int seg[256];
  const Geom& g = a.g;
  const int tid = threadIdx.x;
  auto seg_scan = [&](int v) -> int {  // exclusive prefix of v over threads
    seg[tid] = v;
    __syncthreads();
    if (tid == 0) {
      int r = 0;
      for (int t = 0; t < 256; ++t) {
        const int x = seg[t];
        seg[t] = r;
        r += x;
      }
    }
    __syncthreads();
    const int out = seg[tid];
    __syncthreads();
    return out;
  };
  if (op == kGather) {
    const int FB = g.B * g.NB, per = (FB + 255) / 256;
    const int f0 = min(FB, tid * per), f1 = min(FB, f0 + per);
    int sum = 0;
    for (int f = f0; f < f1; ++f) sum += a.g_total[f];
    int run = seg_scan(sum);
    for (int f = f0; f < f1; ++f) {
      a.g_off[f] = run;
      run += a.g_total[f];
    }
    __syncthreads();
  }
  const int C = a.n_chunks;
  const int F = g.B * C * g.NB, per = (F + 255) / 256;
  const int f0 = min(F, tid * per), f1 = min(F, f0 + per);
  int cnt = 0;
  for (int f = f0; f < f1; ++f) {
    const int j = f % g.NB, c = (f / g.NB) % C, b = f / (g.NB * C);
    int first;
    const int n = item_rows(g, op, b, c, j, a.window, a.chunk_rows, a.row_tiles, a.g_cnt,
                            a.g_total, a.g_off, &first);
    a.plan_first[f] = first;
    a.plan_nrows[f] = n;
    cnt += items_of(n, a.split_rows);
  }
  int run = seg_scan(cnt);
  for (int f = f0; f < f1; ++f) {
    a.plan_pre[f] = min(run, a.items);
    run += items_of(a.plan_nrows[f], a.split_rows);
  }
  if (tid == 255) a.plan_pre[F] = min(run, a.items);
}

// Gather: row lists, each block's rows in ascending order. One wave walks
// the tile's rows in order; a row's entries are distinct blocks, and the
// LDS counter makes repeated entries land in distinct slots regardless.
__global__ __launch_bounds__(256) void bwd_gfill_kernel(BwdArgs a) {
  __shared__ int next[4096];
  const Geom& g = a.g;
  const int T = a.row_tiles;
  const int b = blockIdx.x / T, tile = blockIdx.x % T;
  const int* cnt = a.g_cnt + ((size_t)b * T + tile) * g.NB;
  for (int j = threadIdx.x; j < g.NB; j += 256) next[j] = a.g_off[b * g.NB + j] + cnt[j];
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const int nb_b = nb_of_entry(g, b);
  for (int rl = 0; rl < 64; ++rl) {
    const int r = tile * 64 + rl;
    if (r >= g.Sq) break;
    if (lane < a.top_k) {
      const int j = a.block_idx[((size_t)b * g.Sq + r) * a.top_k + lane];
      const RowRange rr = row_range(g, kGather, b, r, 0);
      if (gather_hit(g, b, nb_b, rr, j)) {
        const int at = atomicAdd(&next[j], 1);
        a.g_rows[at] = r;
        if (a.g_pos != nullptr) a.g_pos[at] = lane;  // the row's stored tile
      }
    }
  }
}

// First stored tile of row (b, r).
__device__ inline long long ds_row_base(const BwdArgs& a, int b, int r) {
  if (a.ds_stride > 0) return ((long long)b * a.g.Sq + r) * a.ds_stride;
  return a.ds_entry[b] + causal_tiles_before(a.g, b, r);
}

// First stored tile of each entry (exclusive prefix of the entries' causal
// block counts) and the total.
__global__ __launch_bounds__(256) void bwd_ds_entry_kernel(BwdArgs a) {
  __shared__ long long tot[kMaxBatch];
  const Geom& g = a.g;
  if ((int)threadIdx.x < g.B) tot[threadIdx.x] = causal_tiles_before(g, threadIdx.x, g.Sq);
  __syncthreads();
  if (threadIdx.x == 0) {
    long long run = 0;
    for (int b = 0; b < g.B; ++b) {
      a.ds_entry[b] = run;
      run += tot[b];
    }
    a.ds_entry[g.B] = run;
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernels.
// ---------------------------------------------------------------------------
// Copy 32 head rows of Q (576 wide) and of dout (512 wide) into a stage
// buffer: wave w fills rows 8w .. 8w+7 of every column group.
__device__ __forceinline__ void stage_half_rows(char* st, const bf16* qrows, const bf16* drows,
                                                int wave, int lane) {
  using namespace bw;
  const int hr = 8 * wave + (lane >> 3);
  const int c8 = (lane & 7) ^ swz(hr);
  const char* sq = (const char*)(qrows + (size_t)hr * DK) + 16 * c8;
  const char* sd = (const char*)(drows + (size_t)hr * DV) + 16 * c8;
  char* dst = st + wave * 1024;
#pragma unroll
  for (int G = 0; G < 9; ++G) dma16(sq + 128 * G, dst + G * HGR);
#pragma unroll
  for (int G = 0; G < 8; ++G) dma16(sd + 128 * G, dst + QH + G * HGR);
}

// A fragment rows 16 rb + l16, k-step ks, from a tile with group stride gs.
__device__ __forceinline__ bf16x8 frag(const char* base, int gs, int ks, int rb, int l16, int grp) {
  const int slot = (4 * (ks & 1) + grp) ^ swz(l16);
  return *(const HS_LDS bf16x8*)(const HS_LDS char*)(base + (ks >> 1) * gs + (16 * rb + l16) * 128 +
                                                     16 * slot);
}

// Transposed A fragment: A[m = column 16 db + l16][k-slot 8 grp + e] =
// tile[row 32 kk + 16 (e >> 2) + 4 grp + (e & 3)][column], by two transpose
// reads (rows 4 grp .. +3 and 16 + 4 grp .. +3 of the 32-row k-step).
__device__ __forceinline__ bf16x8 frag_t(const char* base, int gs, int kk, int db, int l16, int grp) {
  const int kloc = 4 * grp + (l16 >> 2);
  const int tv = ((l16 >> 1) & 1) ^ swz(kloc);
  const char* p = base + kloc * 128 + 8 * (l16 & 1) + 16 * ((2 * (db & 3)) ^ tv) + (db >> 2) * gs +
                  (32 * kk) * 128;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((HS_LDS bf16x4*)(HS_LDS char*)p);
  const bf16x4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4bf16((HS_LDS bf16x4*)(HS_LDS char*)(p + 16 * 128));
  bf16x8 v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  return v;
}

// dq from the stored score gradients: one workgroup per pair of consecutive
// query rows (heaviest first), 8 waves, two per SIMD: wave w owns heads
// 16 (w & 3) .. +15 of row r_hi - (w >> 2). Per tile only dQ^T += K^T . dS^T
// remains, with dS^T read from the stored tile in operand order (16 B per
// lane and k-step, the next tile's prefetched during the current one). Both
// rows walk one tile sequence and each copied K tile serves both; a row takes
// zero dS on a tile it does not have. Causal and window: the union of the two
// rows' block ranges. Gather: the union of their selections (the first row's
// usable entries in list order, then the second row's other ones), built by
// every wave in its own LDS list; a row's stored tile is its selection entry.
template <int OP>
__global__ __launch_bounds__(2 * bw::NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_ds_bf16_kernel(BwdArgs a) {
  using namespace bw;
  __shared__ __attribute__((aligned(16))) char buf[2][TILE];
  // gather: per wave, the union's blocks and each row's entry (-1: none)
  __shared__ int ulist[OP == kGather ? 2 * NT / 64 : 1][128];
  __shared__ int upos[OP == kGather ? 2 * NT / 64 : 1][2][128];

  const Geom& g = a.g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // 0 .. 7
  const int grp = lane >> 4, l16 = lane & 15;
  const int hw = wave & 3, rsel = wave >> 2;
  const int head = 16 * hw + l16;
  const int npair = (g.Sq + 1) / 2;
  const int b = blockIdx.x / npair;
  const int r_hi = g.Sq - 1 - 2 * (blockIdx.x % npair);
  const int r_lo = r_hi - 1;                       // -1: no second row
  const RowRange ra = row_range(g, OP, b, r_hi, a.window);
  const RowRange rb = r_lo >= 0 ? row_range(g, OP, b, r_lo, a.window) : ra;
  int jf = min(ra.j_first, rb.j_first), jl = max(ra.j_last, rb.j_last);
  int ntiles = jl - jf + 1;
  if constexpr (OP == kGather) {
    const int K = a.top_k;
    const int nb_b = nb_of_entry(g, b);
    int ja = -1, jb = -1;
    if (lane < K) {
      ja = a.block_idx[((size_t)b * g.Sq + r_hi) * K + lane];
      if (r_lo >= 0) jb = a.block_idx[((size_t)b * g.Sq + r_lo) * K + lane];
    }
    const bool oka = lane < K && gather_hit(g, b, nb_b, ra, ja);
    const bool okb = lane < K && r_lo >= 0 && gather_hit(g, b, nb_b, rb, jb);
    const unsigned long long lt = (1ull << lane) - 1ull;
    const unsigned long long ma = __ballot(oka);
    const int na = __popcll(ma);
    if (oka) {
      const int at = __popcll(ma & lt);
      ulist[wave][at] = ja;
      upos[wave][0][at] = lane;
      upos[wave][1][at] = -1;
    }
    // the second row's entry that the first row also selected
    const int jam = oka ? ja : -2;
    int found = -1;
    for (int k = 0; k < K; ++k)
      if (okb && jb == __builtin_amdgcn_readlane(jam, k)) found = k;
    // (LDS operations of one wave complete in order)
    if (found >= 0) upos[wave][1][__popcll(ma & ((1ull << found) - 1ull))] = lane;
    const bool only_b = okb && found < 0;
    const unsigned long long mb = __ballot(only_b);
    if (only_b) {
      const int at = na + __popcll(mb & lt);
      ulist[wave][at] = jb;
      upos[wave][0][at] = -1;
      upos[wave][1][at] = lane;
    }
    ntiles = na + __popcll(mb);
    __builtin_amdgcn_wave_barrier();
  }
  auto tile_block = [&](int t) -> int { return OP == kGather ? ulist[wave][t] : jf + t; };
  // this wave's row
  const int r = rsel ? r_lo : r_hi;
  const bool has_row = r >= 0;
  const RowRange rr = rsel ? rb : ra;
  const size_t row = (size_t)b * g.Sq + (has_row ? r : 0);

  const bf16* kv_entry = static_cast<const bf16*>(a.kv) + (size_t)b * g.Skv * DK;
  // copy: wave w fills keys 8w .. 8w+7 of every column group
  const int cp_c8 = (lane & 7) ^ swz(8 * wave + (lane >> 3));
  auto copy_tile = [&](char* dst, const Blk& bk, auto&& issue) __attribute__((always_inline)) {
    const int k = min(8 * wave + (lane >> 3), bk.len - 1);
    const char* src = (const char*)(kv_entry + (size_t)(bk.start + k) * DK) + 16 * cp_c8;
    issue(src, dst + wave * 1024);
  };
  if (ntiles > 0)
    copy_tile(buf[0], block_rows(g, b, tile_block(0)), [&](const char* src, char* dst) __attribute__((always_inline)) {
#pragma unroll
      for (int G = 0; G < 9; ++G) dma16(src + 128 * G, dst + G * GR);
    });
  const long long base = has_row ? ds_row_base(a, b, r) : 0;
  const bf16* dsp = a.ds_tiles + (base * 4 + hw) * 2 * 512 + lane * 8;  // row tile t: + 4096 t
  const bf16x8 zero8 = {};
  // dS of tile t of the walk for this wave's row; false: the row has no
  // entry for the tile (its dS is zero)
  auto ds_load = [&](int t, bf16x8* d) __attribute__((always_inline)) -> bool {
    int e = -1;
    if (OP == kGather) {
      e = has_row ? upos[wave][rsel][t] : -1;
    } else {
      const int j = jf + t;
      if (has_row && j >= rr.j_first && j <= rr.j_last) e = j - rr.j_first;
    }
    if (e >= 0) {
      const bf16* q = dsp + (size_t)e * 4096;
      d[0] = *(const bf16x8*)q;
      d[1] = *(const bf16x8*)(q + 512);
    } else {
      d[0] = zero8;
      d[1] = zero8;
    }
    return e >= 0;
  };
  bf16x8 dnext[2], dcur[2];
  bool mine_next = ntiles > 0 && ds_load(0, dnext);

  f32x4 acc[DBK];
#pragma unroll
  for (int db = 0; db < DBK; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int t = 0; t < ntiles; ++t) {
    char* cur = buf[t & 1];
    const int tn = min(t + 1, ntiles - 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // tile t and its dS resident; tile t-1 consumed by every wave
    dcur[0] = dnext[0];
    dcur[1] = dnext[1];
    const bool mine = mine_next;
    mine_next = ds_load(tn, dnext);
    // The copy of the next tile (on the last tile the current one again, into
    // the idle buffer) is spread over the stream.
    const Blk nbk = block_rows(g, b, tile_block(tn));
    const int ck = min(8 * wave + (lane >> 3), nbk.len - 1);
    const char* cp_src = (const char*)(kv_entry + (size_t)(nbk.start + ck) * DK) + 16 * cp_c8;
    char* cp_dst = buf[(t + 1) & 1] + wave * 1024;

    // 72 K^T fragments, k-step kk major, column block db.
    constexpr int NF = 2 * DBK;
    auto load = [&](auto F) __attribute__((always_inline)) -> bf16x8 {
      constexpr int f = decltype(F)::value;
      return frag_t(cur, GR, f / DBK, f % DBK, l16, grp);
    };
    auto use = [&](auto I, bf16x8 fr) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      acc[i % DBK] = mfma(fr, dcur[i / DBK], acc[i % DBK]);
    };
    auto pre = [&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      if constexpr ((i & 7) == 7) {
        constexpr int G = i >> 3;
        dma16(cp_src + 128 * G, cp_dst + G * GR);
      }
    };
    // A wave whose row has no entry for this tile (a block that only the
    // other row of the pair selected or reaches, or a pair without a second
    // row) has dS = 0 here: it skips the MFMAs and issues only its share of
    // the copy, which leaves its SIMD to the other row's wave.
    if (!__builtin_amdgcn_readfirstlane((int)mine)) {
#pragma unroll
      for (int G = 0; G < 9; ++G) dma16(cp_src + 128 * G, cp_dst + G * GR);
      continue;
    }
    operand_stream<NF, 8>(load, use, pre);
  }
  __builtin_amdgcn_s_waitcnt(0);

  // acc[db][i] = dq[head][16 db + 4 grp + i]
  if (has_row) {
    float* out = a.dq + (row * H + head) * DK + 4 * grp;
#pragma unroll
    for (int db = 0; db < DBK; ++db) *(f32x4*)(out + 16 * db) = acc[db];
  }
}

template <int OP>
__global__ __launch_bounds__(bw::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dq_bf16_kernel(BwdArgs a) {
  using namespace bw;
  __shared__ __attribute__((aligned(16))) char buf[2][TILE];
  __shared__ int tile_list[64];
  __shared__ int tile_count;

  const Geom& g = a.g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 4, l16 = lane & 15;
  const int head = 16 * wave + l16;
  const int w = blockIdx.x;
  const int b = w / g.Sq;
  const int r = g.Sq - 1 - (w % g.Sq);  // heaviest rows first
  const size_t row = (size_t)b * g.Sq + r;
  const RowRange rr = row_range(g, OP, b, r, a.window);
  const int nb_b = nb_of_entry(g, b);

  int ntiles;
  if (OP == kGather) {
    if (wave == 0) {
      int j = -1;
      bool ok = false;
      if (lane < a.top_k) {
        j = a.block_idx[row * a.top_k + lane];
        ok = gather_hit(g, b, nb_b, rr, j);
      }
      const unsigned long long m = __ballot(ok);
      if (ok) tile_list[__popcll(m & ((1ull << lane) - 1ull))] = j;
      if (lane == 0) tile_count = __popcll(m);
    }
    __syncthreads();
    ntiles = tile_count;
  } else {
    ntiles = rr.j_last - rr.j_first + 1;
  }
  auto tile_block = [&](int t) -> int { return OP == kGather ? tile_list[t] : rr.j_first + t; };

  const bf16* kv_entry = static_cast<const bf16*>(a.kv) + (size_t)b * g.Skv * DK;
  if (ntiles > 0) {
    const Blk b0 = block_rows(g, b, tile_block(0));
    stage_tile(buf[0], kv_entry, b0.start, b0.len, wave, lane);
  }

  bf16x8 qreg[KSTEPS], dreg[VSTEPS];
  {
    const bf16* qp = static_cast<const bf16*>(a.q) + (row * H + head) * DK + 8 * grp;
    const bf16* dp = static_cast<const bf16*>(a.dout) + (row * H + head) * DV + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qreg[ks] = *(const bf16x8*)(qp + 32 * ks);
#pragma unroll
    for (int ks = 0; ks < VSTEPS; ++ks) dreg[ks] = *(const bf16x8*)(dp + 32 * ks);
  }
  const float lse2 = a.lse[row * H + head] * kLog2e;
  const float dsum = a.dsum[row * H + head];
  const int cp_c8 = (lane & 7) ^ swz(8 * wave + (lane >> 3));  // copy: chunk of this lane
  const float sl2 = g.scale_log2;
  const float scale = g.scale_log2 * kLn2;

  f32x4 acc[DBK];
#pragma unroll
  for (int db = 0; db < DBK; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int t = 0; t < ntiles; ++t) {
    char* cur = buf[t & 1];
    const int j = tile_block(t);
    const Blk blk = block_rows(g, b, j);
    const int klo = rr.lo - blk.start, khi = min(rr.hi - blk.start, blk.len - 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // tile t resident; tile t-1 consumed by every wave
    // The copy of the next tile is spread over the first 36 MFMAs of the
    // stream. On the last tile the current block is copied again into the
    // idle buffer, which keeps the stream free of branches; nothing reads it.
    const Blk nbk = t + 1 < ntiles ? block_rows(g, b, tile_block(t + 1)) : blk;
    const int cka = min(8 * wave + (lane >> 3), nbk.len - 1);
    const int ckb = min(8 * (wave + 4) + (lane >> 3), nbk.len - 1);
    const char* cp_a = (const char*)(kv_entry + (size_t)(nbk.start + cka) * DK) + 16 * cp_c8;
    const char* cp_b = (const char*)(kv_entry + (size_t)(nbk.start + ckb) * DK) + 16 * cp_c8;
    char* cp_dst = buf[(t + 1) & 1] + wave * 1024;

    // Stream: 72 K fragments (k-step ks, key block kb), each feeding the
    // score MFMA and, for ks < 16, the dP MFMA; then 72 K^T fragments (k-step
    // kk major, column block db) for dQ. P and dS are formed between the two.
    constexpr int NP1 = 4 * KSTEPS, NF = NP1 + 2 * DBK;
    f32x4 s[4], dp[4];
    bf16x8 dsb[2];
    auto load = [&](auto F) __attribute__((always_inline)) -> bf16x8 {
      constexpr int f = decltype(F)::value;
      if constexpr (f < NP1) return frag(cur, GR, f / 4, f % 4, l16, grp);
      else return frag_t(cur, GR, (f - NP1) / DBK, (f - NP1) % DBK, l16, grp);
    };
    auto use = [&](auto I, bf16x8 fr) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      if constexpr (i < NP1) {
        constexpr int ks = i / 4, kb = i % 4;
        s[kb] = mfma(fr, qreg[ks], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[kb]);
        if constexpr (ks < VSTEPS)
          dp[kb] = mfma(fr, dreg[ks], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : dp[kb]);
      } else {
        constexpr int kk = (i - NP1) / DBK, db = (i - NP1) % DBK;
        acc[db] = mfma(fr, dsb[kk], acc[db]);
      }
    };
    auto pre = [&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      if constexpr (i < 36 && (i & 3) == 3) {
        constexpr int G = i >> 2;
        dma16(cp_a + 128 * G, cp_dst + G * GR);
        dma16(cp_b + 128 * G, cp_dst + G * GR + 4096);
      }
      if constexpr (i == NP1) {
        // s[kb][i], dp[kb][i]: key 16 kb + 4 grp + i of the tile, head l16.
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int k = 16 * kb + 4 * grp + e;
            const float p =
                (k >= klo && k <= khi) ? __builtin_amdgcn_exp2f(s[kb][e] * sl2 - lse2) : 0.f;
            dsb[kb >> 1][4 * (kb & 1) + e] = (bf16)(p * (dp[kb][e] - dsum) * scale);
          }
        }
      }
    };
    operand_stream<NF, 8>(load, use, pre);
  }
  __builtin_amdgcn_s_waitcnt(0);

  // acc[db][i] = dq[head][16 db + 4 grp + i]
  float* out = a.dq + (row * H + head) * DK + 4 * grp;
#pragma unroll
  for (int db = 0; db < DBK; ++db) *(f32x4*)(out + 16 * db) = acc[db];
}

// STORE (causal and window): also write each stage's dS to the stored tiles. The
// lanes hold dS for one key and eight heads; the dq kernel wants one head and
// eight keys, so a stage's 64 x 32 dS tile goes through LDS ([key][head], 64 B
// rows, written a few MFMAs into phase 2) and read back during phase 1 of
// the next stage, after its barrier, with transpose reads: wave w then writes
// head block 2 (s & 1) + (w >> 1), k-step w & 1 of the row's tile, 16 B per
// lane. (Issued right after the barrier instead, the transpose reads delay
// the stream's first fragments: 3.5 ms more at S = 32768.)
template <int OP, bool STORE>
__global__ __launch_bounds__(bw::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkv_bf16_kernel(BwdArgs a) {
  using namespace bw;
  __shared__ __attribute__((aligned(16))) char stg[2][STAGE];
  __shared__ __attribute__((aligned(16))) char dsl[STORE ? 2 : 1][STORE ? 64 * 64 : 16];

  const Geom& g = a.g;
  const int C = a.n_chunks;
  const int F = g.B * C * g.NB;
  const int item = blockIdx.x;
  if (item >= a.plan_pre[F]) return;
  int lo = 0, hi = F - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.plan_pre[mid] <= item) lo = mid; else hi = mid - 1;
  }
  const int f = lo;
  const int j = f % g.NB, b = f / (g.NB * C);
  // the item's share of (b, c, j)'s rows: all of them, or split_rows from
  // sub-item (item - plan_pre[f]) onwards
  const int sub = item - a.plan_pre[f];
  const int n = a.split_rows > 0 ? min(a.split_rows, a.plan_nrows[f] - sub * a.split_rows)
                                 : a.plan_nrows[f];
  const int base_i = a.plan_first[f] + sub * a.split_rows;
  auto row_at = [&](int i) -> int {
    const int rr = OP == kGather ? a.g_rows[base_i + i] : base_i + i;
    return min(max(rr, 0), g.Sq - 1);
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 4, l16 = lane & 15;
  const int kloc = 16 * wave + l16;  // this lane's key inside the block
  const Blk blk = block_rows(g, b, j);
  const int key = blk.start + kloc;

  const bf16* q = static_cast<const bf16*>(a.q);
  const bf16* dout = static_cast<const bf16*>(a.dout);
  auto stage = [&](int s) {
    const size_t rw = (size_t)b * g.Sq + row_at(s >> 1);
    const int h0 = 32 * (s & 1);
    stage_half_rows(stg[s & 1], q + (rw * H + h0) * DK, dout + (rw * H + h0) * DV, wave, lane);
  };
  if (n > 0) stage(0);

  bf16x8 kreg[KSTEPS];
  {
    const int kr = blk.start + min(kloc, blk.len - 1);
    const bf16* kp = static_cast<const bf16*>(a.kv) + ((size_t)b * g.Skv + kr) * DK + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) kreg[ks] = *(const bf16x8*)(kp + 32 * ks);
  }
  const float sl2 = g.scale_log2;
  const float scale = g.scale_log2 * kLn2;
  const int cp_hr = 8 * wave + (lane >> 3);       // copy: head row of this lane
  const int cp_c8 = (lane & 7) ^ swz(cp_hr);      // and its chunk

  f32x4 acc[DBK];
#pragma unroll
  for (int db = 0; db < DBK; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // STORE: first stored tile of the current row (rows of a causal or window
  // item are consecutive), the previous stage's target and its transposed dS.
  long long rbase = 0;
  int prev_nt = 0;
  bf16* st_prev = nullptr;
  const int tr_off = (32 * (wave & 1) + 4 * grp + (l16 >> 2)) * 64 + 32 * (wave >> 1) + 8 * (l16 & 3);
  if (STORE) {
    if (OP != kGather) rbase = ds_row_base(a, b, row_at(0));
    st_prev = a.ds_dummy + wave * 512 + lane * 8;
  }

  for (int s = 0; s < 2 * n; ++s) {
    const char* cur = stg[s & 1];
    const int r = row_at(s >> 1);
    const size_t rw = (size_t)b * g.Sq + r;
    const int h0 = 32 * (s & 1);
    const RowRange rr = row_range(g, OP, b, r, a.window);
    bf16* st_cur = nullptr;
    if (STORE) {
      long long slot;
      if (OP == kGather) {
        // the row's tile of this selection entry
        slot = ((long long)b * g.Sq + r) * a.ds_stride + a.g_pos[base_i + (s >> 1)];
      } else {
        if (s > 0 && (s & 1) == 0) rbase += a.ds_stride > 0 ? a.ds_stride : prev_nt;
        prev_nt = rr.j_last - rr.j_first + 1;
        slot = rbase + (j - rr.j_first);
      }
      st_cur = a.ds_tiles + ((slot * 4 + 2 * (s & 1) + (wave >> 1)) * 2 + (wave & 1)) * 512 + lane * 8;
    }
    const bool valid = kloc < blk.len && key >= rr.lo && key <= rr.hi;
    // heads h0 + 16 hb + 4 grp + i of this lane
    float lse2[2][4], ds[2][4];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = h0 + 16 * hb + 4 * grp + i;
        lse2[hb][i] = a.lse[rw * H + h] * kLog2e;
        ds[hb][i] = a.dsum[rw * H + h];
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // stage s resident; stage s-1 consumed by every wave
    bf16x4 tlo, thi;
    const HS_LDS char* tp = (const HS_LDS char*)(dsl[(s + 1) & 1] + tr_off);
    // The copy of the next stage is spread over the 68 MFMAs of phase 1: Q
    // groups at positions 3, 7, .., 35, dout groups at 39, .., 67. The last
    // stage copies itself again into the idle buffer (nothing reads it).
    const int sn = s + 1 < 2 * n ? s + 1 : s;
    const size_t rwn = (size_t)b * g.Sq + row_at(sn >> 1);
    const int hn = 32 * (sn & 1) + cp_hr;
    const char* cq = (const char*)(q + (rwn * H + hn) * DK) + 16 * cp_c8;
    const char* cd = (const char*)(dout + (rwn * H + hn) * DV) + 16 * cp_c8;
    char* cp_dst = stg[(s + 1) & 1] + wave * 1024;

    // Stream: 68 fragments of the staged rows for S and dP (per k-step: Q of
    // head blocks 0 and 1, then dout of both while ks < 16), then 36 Q^T and
    // 32 dout^T fragments for dKV. P and dS are formed between the two.
    constexpr int NP1 = 2 * KSTEPS + 2 * VSTEPS, NF = NP1 + DBK + DBV;
    f32x4 sc[2], dp[2];
    bf16x8 pb, dsb;
    // phase-1 fragment f: k-step, operand (0 = Q, 1 = dout) and head block
    auto p1_ks = [](int f) constexpr { return f < 64 ? f >> 2 : 16 + ((f - 64) >> 1); };
    auto p1_kind = [](int f) constexpr { return f < 64 ? (f & 3) >> 1 : 0; };
    auto load = [&](auto F) __attribute__((always_inline)) -> bf16x8 {
      constexpr int f = decltype(F)::value;
      if constexpr (f < NP1) return frag(cur + (p1_kind(f) ? QH : 0), HGR, p1_ks(f), f & 1, l16, grp);
      else if constexpr (f - NP1 < DBK) return frag_t(cur, HGR, 0, f - NP1, l16, grp);
      else return frag_t(cur + QH, HGR, 0, f - NP1 - DBK, l16, grp);
    };
    auto use = [&](auto I, bf16x8 fr) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      if constexpr (i < NP1) {
        constexpr int ks = p1_ks(i), hb = i & 1;
        if constexpr (p1_kind(i) == 0)
          sc[hb] = mfma(fr, kreg[ks], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sc[hb]);
        else
          dp[hb] = mfma(fr, kreg[ks], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : dp[hb]);
      } else if constexpr (i - NP1 < DBK) {
        acc[i - NP1] = mfma(fr, dsb, acc[i - NP1]);
      } else {
        acc[i - NP1 - DBK] = mfma(fr, pb, acc[i - NP1 - DBK]);
      }
    };
    auto pre = [&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      if constexpr (i == NP1 + 4) {
        if constexpr (STORE) {
          // this stage's dS as [key][head of the stage], heads 16 hb + 4 grp ..
          char* wp = dsl[s & 1] + kloc * 64 + 8 * grp;
          bf16x4 lo4, hi4;
          lo4[0] = dsb[0]; lo4[1] = dsb[1]; lo4[2] = dsb[2]; lo4[3] = dsb[3];
          hi4[0] = dsb[4]; hi4[1] = dsb[5]; hi4[2] = dsb[6]; hi4[3] = dsb[7];
          *(HS_LDS bf16x4*)(HS_LDS char*)wp = lo4;
          *(HS_LDS bf16x4*)(HS_LDS char*)(wp + 32) = hi4;
        }
      }
      if constexpr (i < NP1 && (i & 3) == 3) {
        constexpr int G = i >> 2;
        if constexpr (G < 9) dma16(cq + 128 * G, cp_dst + G * HGR);
        else dma16(cd + 128 * (G - 9), cp_dst + QH + (G - 9) * HGR);
      }
      if constexpr (STORE && i == 30) {
        // the previous stage's dS, transposed (stage 0: unused contents,
        // written to the dummy target)
        tlo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((HS_LDS bf16x4*)tp);
        thi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((HS_LDS bf16x4*)(tp + 16 * 64));
      }
      if constexpr (STORE && i == 44) {
        bf16x8 v;
        v[0] = tlo[0]; v[1] = tlo[1]; v[2] = tlo[2]; v[3] = tlo[3];
        v[4] = thi[0]; v[5] = thi[1]; v[6] = thi[2]; v[7] = thi[3];
        *(bf16x8*)st_prev = v;
      }
      if constexpr (i == NP1) {
        // sc[hb][e], dp[hb][e]: head h0 + 16 hb + 4 grp + e, key kloc.
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = valid ? __builtin_amdgcn_exp2f(sc[hb][e] * sl2 - lse2[hb][e]) : 0.f;
            pb[4 * hb + e] = (bf16)p;
            dsb[4 * hb + e] = (bf16)(p * (dp[hb][e] - ds[hb][e]) * scale);
          }
        }
      }
    };
    operand_stream<NF, 8>(load, use, pre);
    if (STORE) st_prev = st_cur;
  }
  __builtin_amdgcn_s_waitcnt(0);
  if (STORE) {
    // the last stage's dS
    __syncthreads();
    const HS_LDS char* tp = (const HS_LDS char*)(dsl[(2 * n + 1) & 1] + tr_off);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((HS_LDS bf16x4*)tp);
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((HS_LDS bf16x4*)(tp + 16 * 64));
    bf16x8 v;
    v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
    v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
    *(bf16x8*)st_prev = v;
  }

  // acc[db][i] = dkv[key kloc][16 db + 4 grp + i]
  float* out = a.part + ((size_t)item * BS + kloc) * DK + 4 * grp;
#pragma unroll
  for (int db = 0; db < DBK; ++db) *(f32x4*)(out + 16 * db) = acc[db];
}

// dkv rows of entry b, 64 at a time: each row sums its block's partials in
// chunk order; rows past the entry's valid length are zero. Without documents
// the 64 rows are exactly one block (key k of block c is row 64 c + k), so a
// thread keeps its 36 elements in registers and walks the block's items once:
// per item 36 independent loads, and the workgroup reads each item's partial
// as one contiguous 147 KB run. With documents each row looks up its own
// block, four threads per row. Both add the partials in the same order.
__global__ __launch_bounds__(256) void bwd_reduce_bf16_kernel(BwdArgs a) {
  using namespace bw;
  const Geom& g = a.g;
  const int chunks = (g.Skv + 63) / 64;
  const int b = blockIdx.x / chunks, c = blockIdx.x % chunks;
  const int L = kv_len_of(g, b);
  constexpr int V4 = DK / 4;           // 144 float4 per row
  constexpr int PT = 64 * V4 / 256;    // 36 float4 per thread
  if (g.n_docs == 0) {
    f32x4 v[PT];
#pragma unroll
    for (int n = 0; n < PT; ++n) v[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (64 * c < L) {
      for (int cc = 0; cc < a.n_chunks; ++cc) {
        const int f = (b * a.n_chunks + cc) * g.NB + c;
        const int it1 = a.plan_pre[f + 1];
        for (int it = a.plan_pre[f]; it < it1; ++it) {
          const f32x4* src = (const f32x4*)(a.part + (size_t)it * BS * DK) + threadIdx.x;
          // all of the item's loads in flight before the first add
          f32x4 t[PT];
#pragma unroll
          for (int n = 0; n < PT; ++n) t[n] = __builtin_nontemporal_load(src + 256 * n);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int n = 0; n < PT; ++n) v[n] += t[n];
        }
      }
    }
#pragma unroll
    for (int n = 0; n < PT; ++n) {
      const int e = threadIdx.x + 256 * n;
      const int i = 64 * c + e / V4;
      if (i < g.Skv)
        *(f32x4*)(a.dkv + ((size_t)b * g.Skv + i) * DK + 4 * (e % V4)) =
            i < L ? v[n] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  // With documents: four threads per row (row 64 c + t / 4), thread q of a
  // row taking float4 columns q, q + 4, ..; each row finds its own block.
  const int i = 64 * c + (threadIdx.x >> 2), q = threadIdx.x & 3;
  if (i >= g.Skv) return;
  f32x4 v[PT];
#pragma unroll
  for (int n = 0; n < PT; ++n) v[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (i < L) {
    const Doc d = doc_of_pos(g, b, i);
    const int j = block_of_pos(g, d, i);
    const int k = i - (d.start + (j - d.blk0) * g.BS);
    for (int cc = 0; cc < a.n_chunks; ++cc) {
      const int f = (b * a.n_chunks + cc) * g.NB + j;
      const int it1 = a.plan_pre[f + 1];
      for (int it = a.plan_pre[f]; it < it1; ++it) {
        const f32x4* src = (const f32x4*)(a.part + ((size_t)it * BS + k) * DK) + q;
        f32x4 t[PT];
#pragma unroll
        for (int n = 0; n < PT; ++n) t[n] = __builtin_nontemporal_load(src + 4 * n);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int n = 0; n < PT; ++n) v[n] += t[n];
      }
    }
  }
  f32x4* dst = (f32x4*)(a.dkv + ((size_t)b * g.Skv + i) * DK) + q;
#pragma unroll
  for (int n = 0; n < PT; ++n) dst[4 * n] = v[n];
}

// ---------------------------------------------------------------------------
// fp32 kernels (H <= 16, Dk <= 128): plain FMAs over LDS-staged rows.
// ---------------------------------------------------------------------------
namespace f32b {
constexpr int MAXH = 16, MAXD = 128, BS = 64, NT = 256, KS = MAXD + 1;
constexpr int MAXQ = (MAXH * MAXD + NT - 1) / NT;  // dq elements per thread
constexpr int MAXK = (BS * MAXD + NT - 1) / NT;    // dkv elements per thread
}  // namespace f32b

template <int OP>
__global__ __launch_bounds__(f32b::NT) void bwd_dq_f32_kernel(BwdArgs a) {
  using namespace f32b;
  __shared__ float qs[MAXH * MAXD], dos[MAXH * MAXD], ks[BS * KS], dss[MAXH * BS];
  __shared__ float lse2[MAXH], dsum[MAXH];
  __shared__ int tile_list[64];
  __shared__ int tile_count;
  const Geom& g = a.g;
  const int H = g.H, Dk = g.Dk, Dv = g.Dv, tid = threadIdx.x;
  const int w = blockIdx.x;
  const int b = w / g.Sq, r = g.Sq - 1 - (w % g.Sq);
  const size_t row = (size_t)b * g.Sq + r;
  const RowRange rr = row_range(g, OP, b, r, a.window);
  const int nb_b = nb_of_entry(g, b);
  const float* q = static_cast<const float*>(a.q);
  const float* kv = static_cast<const float*>(a.kv);
  const float* dout = static_cast<const float*>(a.dout);
  if (tid == 0) {
    int n = 0;
    if (OP == kGather) {
      for (int k = 0; k < a.top_k; ++k) {
        const int j = a.block_idx[row * a.top_k + k];
        if (gather_hit(g, b, nb_b, rr, j)) tile_list[n++] = j;
      }
    } else {
      n = rr.j_last - rr.j_first + 1;
    }
    tile_count = n;
  }
  for (int i = tid; i < H * Dk; i += NT) qs[(i / Dk) * MAXD + i % Dk] = q[row * H * Dk + i];
  for (int i = tid; i < H * Dv; i += NT) dos[(i / Dv) * MAXD + i % Dv] = dout[row * H * Dv + i];
  if (tid < H) {
    lse2[tid] = a.lse[row * H + tid] * kLog2e;
    dsum[tid] = a.dsum[row * H + tid];
  }
  __syncthreads();
  const int ntiles = tile_count;
  const float sl2 = g.scale_log2, scale = g.scale_log2 * kLn2;
  float acc[MAXQ];
#pragma unroll
  for (int m = 0; m < MAXQ; ++m) acc[m] = 0.f;
  const float* kv_entry = kv + (size_t)b * g.Skv * Dk;
  for (int t = 0; t < ntiles; ++t) {
    const int j = OP == kGather ? tile_list[t] : rr.j_first + t;
    const Blk blk = block_rows(g, b, j);
    for (int i = tid; i < BS * Dk; i += NT) {
      const int k = i / Dk, d = i % Dk;
      ks[k * KS + d] = kv_entry[(size_t)(blk.start + min(k, blk.len - 1)) * Dk + d];
    }
    __syncthreads();
    for (int i = tid; i < H * BS; i += NT) {
      const int h = i / BS, k = i % BS;
      float s = 0.f, dp = 0.f;
      for (int d = 0; d < Dk; ++d) s = fmaf(qs[h * MAXD + d], ks[k * KS + d], s);
      for (int d = 0; d < Dv; ++d) dp = fmaf(dos[h * MAXD + d], ks[k * KS + d], dp);
      const int key = blk.start + k;
      const bool ok = k < blk.len && key >= rr.lo && key <= rr.hi;
      const float p = ok ? exp2f(s * sl2 - lse2[h]) : 0.f;
      dss[i] = p * (dp - dsum[h]) * scale;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MAXQ; ++m) {
      const int e = tid + NT * m;
      if (e < H * Dk) {
        const int h = e / Dk, d = e % Dk;
        float v = acc[m];
        for (int k = 0; k < BS; ++k) v = fmaf(dss[h * BS + k], ks[k * KS + d], v);
        acc[m] = v;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int m = 0; m < MAXQ; ++m) {
    const int e = tid + NT * m;
    if (e < H * Dk) a.dq[row * H * Dk + e] = acc[m];
  }
}

// One workgroup per work item (rows of one key block, as for bf16): the item's
// rows in turn, the next row's q, dout, lse and D fetched into registers while
// the current one is processed; partial dkv of the block's 64 keys.
template <int OP>
__global__ __launch_bounds__(f32b::NT) void bwd_dkv_f32_kernel(BwdArgs a) {
  using namespace f32b;
  __shared__ float ks[BS * KS], qs[2][MAXH * MAXD], dos[2][MAXH * MAXD], ps[MAXH * BS],
      dss[MAXH * BS];
  __shared__ float lse2[2][MAXH], dsum[2][MAXH];
  const Geom& g = a.g;
  const int H = g.H, Dk = g.Dk, Dv = g.Dv, tid = threadIdx.x;
  const int C = a.n_chunks;
  const int F = g.B * C * g.NB;
  const int item = blockIdx.x;
  if (item >= a.plan_pre[F]) return;
  int lo = 0, hi = F - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.plan_pre[mid] <= item) lo = mid; else hi = mid - 1;
  }
  const int f = lo;
  const int j = f % g.NB, b = f / (g.NB * C);
  // the item's share of (b, c, j)'s rows: all of them, or split_rows from
  // sub-item (item - plan_pre[f]) onwards
  const int sub = item - a.plan_pre[f];
  const int n = a.split_rows > 0 ? min(a.split_rows, a.plan_nrows[f] - sub * a.split_rows)
                                 : a.plan_nrows[f];
  const int base_i = a.plan_first[f] + sub * a.split_rows;
  auto row_at = [&](int i) -> int {
    const int rr = OP == kGather ? a.g_rows[base_i + i] : base_i + i;
    return min(max(rr, 0), g.Sq - 1);
  };
  const float* q = static_cast<const float*>(a.q);
  const float* kv = static_cast<const float*>(a.kv);
  const float* dout = static_cast<const float*>(a.dout);
  const Blk blk = block_rows(g, b, j);
  const float* kv_entry = kv + (size_t)b * g.Skv * Dk;
  for (int i = tid; i < BS * Dk; i += NT) {
    const int k = i / Dk, d = i % Dk;
    ks[k * KS + d] = kv_entry[(size_t)(blk.start + min(k, blk.len - 1)) * Dk + d];
  }
  // Row data of this thread: q and dout elements tid + NT m, lse and D of head tid.
  float rq[MAXQ], rd[MAXQ], rl = 0.f, rs = 0.f;
  auto fetch = [&](int ri) {
    const size_t row = (size_t)b * g.Sq + row_at(ri);
#pragma unroll
    for (int m = 0; m < MAXQ; ++m) {
      const int e = tid + NT * m;
      rq[m] = e < H * Dk ? q[row * H * Dk + e] : 0.f;
      rd[m] = e < H * Dv ? dout[row * H * Dv + e] : 0.f;
    }
    if (tid < H) {
      rl = a.lse[row * H + tid] * kLog2e;
      rs = a.dsum[row * H + tid];
    }
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int m = 0; m < MAXQ; ++m) {
      const int e = tid + NT * m;
      if (e < H * Dk) qs[buf][(e / Dk) * MAXD + e % Dk] = rq[m];
      if (e < H * Dv) dos[buf][(e / Dv) * MAXD + e % Dv] = rd[m];
    }
    if (tid < H) {
      lse2[buf][tid] = rl;
      dsum[buf][tid] = rs;
    }
  };
  if (n > 0) {
    fetch(0);
    put(0);
  }
  const float sl2 = g.scale_log2, scale = g.scale_log2 * kLn2;
  float acc[MAXK];
#pragma unroll
  for (int m = 0; m < MAXK; ++m) acc[m] = 0.f;
  __syncthreads();
  for (int ri = 0; ri < n; ++ri) {
    const int cb = ri & 1;
    if (ri + 1 < n) fetch(ri + 1);
    const RowRange rr = row_range(g, OP, b, row_at(ri), a.window);
    for (int i = tid; i < H * BS; i += NT) {
      const int h = i / BS, k = i % BS;
      float sv = 0.f, dp = 0.f;
      for (int d = 0; d < Dk; ++d) sv = fmaf(qs[cb][h * MAXD + d], ks[k * KS + d], sv);
      for (int d = 0; d < Dv; ++d) dp = fmaf(dos[cb][h * MAXD + d], ks[k * KS + d], dp);
      const int key = blk.start + k;
      const bool ok = k < blk.len && key >= rr.lo && key <= rr.hi;
      const float p = ok ? exp2f(sv * sl2 - lse2[cb][h]) : 0.f;
      ps[i] = p;
      dss[i] = p * (dp - dsum[cb][h]) * scale;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MAXK; ++m) {
      const int e = tid + NT * m;
      if (e < BS * Dk) {
        const int k = e / Dk, d = e % Dk;
        float v = acc[m];
        for (int h = 0; h < H; ++h) v = fmaf(dss[h * BS + k], qs[cb][h * MAXD + d], v);
        if (d < Dv)
          for (int h = 0; h < H; ++h) v = fmaf(ps[h * BS + k], dos[cb][h * MAXD + d], v);
        acc[m] = v;
      }
    }
    if (ri + 1 < n) put(cb ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int m = 0; m < MAXK; ++m) {
    const int e = tid + NT * m;
    if (e < BS * Dk) a.part[(size_t)item * BS * Dk + e] = acc[m];
  }
}

// dkv rows of entry b, 64 at a time, any width: each row sums its block's
// partials in chunk order; rows past the entry's valid length are zero.
__global__ __launch_bounds__(256) void bwd_reduce_f32_kernel(BwdArgs a) {
  const Geom& g = a.g;
  const int Dk = g.Dk;
  const int chunks = (g.Skv + 63) / 64;
  const int b = blockIdx.x / chunks, c = blockIdx.x % chunks;
  const int L = kv_len_of(g, b);
  for (int e = threadIdx.x; e < 64 * Dk; e += 256) {
    const int i = 64 * c + e / Dk, d = e % Dk;
    if (i >= g.Skv) break;
    float v = 0.f;
    if (i < L) {
      const Doc dc = doc_of_pos(g, b, i);
      const int j = block_of_pos(g, dc, i);
      const int k = i - (dc.start + (j - dc.blk0) * g.BS);
      for (int cc = 0; cc < a.n_chunks; ++cc) {
        const int f = (b * a.n_chunks + cc) * g.NB + j;
        for (int it = a.plan_pre[f]; it < a.plan_pre[f + 1]; ++it)
          v += a.part[((size_t)it * 64 + k) * Dk + d];
      }
    }
    a.dkv[((size_t)b * g.Skv + i) * Dk + d] = v;
  }
}

template <int OP>
void launch_bf16(const BwdArgs& a, hipStream_t s) {
  const Geom& g = a.g;
  const unsigned F = (unsigned)(g.B * g.NB);
  if (OP == kGather) {
    hipLaunchKernelGGL(bwd_gcount_kernel, dim3(g.B * a.row_tiles), dim3(256), 0, s, a);
    hipLaunchKernelGGL(bwd_gscan_kernel, dim3((F + 255) / 256), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL(bwd_plan_kernel, dim3(1), dim3(256), 0, s, a, OP);
  if (OP == kGather)
    hipLaunchKernelGGL(bwd_gfill_kernel, dim3(g.B * a.row_tiles), dim3(256), 0, s, a);
  if (a.ds_tiles != nullptr) {
    // stored score gradients: the key-block pass writes dS, dq reads it
    if (a.ds_stride == 0) hipLaunchKernelGGL(bwd_ds_entry_kernel, dim3(1), dim3(256), 0, s, a);
    if (a.items > 0)
      hipLaunchKernelGGL((bwd_dkv_bf16_kernel<OP, true>), dim3(a.items), dim3(bw::NT), 0, s, a);
    hipLaunchKernelGGL(bwd_dq_ds_bf16_kernel<OP>, dim3(g.B * ((g.Sq + 1) / 2)), dim3(2 * bw::NT),
                       0, s, a);
  } else {
    hipLaunchKernelGGL(bwd_dq_bf16_kernel<OP>, dim3(g.B * g.Sq), dim3(bw::NT), 0, s, a);
    if (a.items > 0)
      hipLaunchKernelGGL((bwd_dkv_bf16_kernel<OP, false>), dim3(a.items), dim3(bw::NT), 0, s, a);
  }
  hipLaunchKernelGGL(bwd_reduce_bf16_kernel, dim3(g.B * ((g.Skv + 63) / 64)), dim3(256), 0, s, a);
}

template <int OP>
void launch_f32(const BwdArgs& a, hipStream_t s) {
  const Geom& g = a.g;
  const unsigned F = (unsigned)(g.B * g.NB);  // blocks of all entries
  if (OP == kGather) {
    hipLaunchKernelGGL(bwd_gcount_kernel, dim3(g.B * a.row_tiles), dim3(256), 0, s, a);
    hipLaunchKernelGGL(bwd_gscan_kernel, dim3((F + 255) / 256), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL(bwd_plan_kernel, dim3(1), dim3(256), 0, s, a, OP);
  if (OP == kGather)
    hipLaunchKernelGGL(bwd_gfill_kernel, dim3(g.B * a.row_tiles), dim3(256), 0, s, a);
  hipLaunchKernelGGL(bwd_dq_f32_kernel<OP>, dim3(g.B * g.Sq), dim3(f32b::NT), 0, s, a);
  if (a.items > 0)
    hipLaunchKernelGGL(bwd_dkv_f32_kernel<OP>, dim3(a.items), dim3(f32b::NT), 0, s, a);
  hipLaunchKernelGGL(bwd_reduce_f32_kernel, dim3(g.B * ((g.Skv + 63) / 64)), dim3(256), 0, s, a);
}

}  // namespace

int bwd_launch(int op, const BwdArgs& a, bool is_bf16, hipStream_t s) {
  if (is_bf16) hipLaunchKernelGGL(bwd_pre_kernel<bf16>, dim3(a.n_pre), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(bwd_pre_kernel<float>, dim3(a.n_pre), dim3(256), 0, s, a);
  if (a.dsink != nullptr) hipLaunchKernelGGL(bwd_sink_kernel, dim3(a.g.H), dim3(256), 0, s, a);
  if (is_bf16) {
    if (op == kScore) launch_bf16<kScore>(a, s);
    else if (op == kGather) launch_bf16<kGather>(a, s);
    else launch_bf16<kSwa>(a, s);
  } else {
    if (op == kScore) launch_f32<kScore>(a, s);
    else if (op == kGather) launch_f32<kGather>(a, s);
    else launch_f32<kSwa>(a, s);
  }
  return (int)hipGetLastError();
}

}  // namespace hs
