// bf16 MFMA attention engine for the HySparse MQA forward path on gfx950.
//
// One kernel template serves the three attention operations of the method
// (page "HySparse MQA sparse attention (FA4 block scoring + SWA MQA +
// block-sparse DSA gather)", section "Core"): causal attention fused with
// per-block scores, block-sparse gather attention, and sliding-window
// attention, all with the optional learnable per-head sink. The shapes are the
// absorbed-MLA MQA layout of the same page, section "FlashMLA sparse kernel
// constraints": 64 query heads share one latent KV head with Dk = 576 columns,
// and the value is its leading Dv = 512 columns.
//
// Work decomposition
//   A workgroup owns one query token: its 64 heads are 64 rows. It walks a
//   sequence of 64-key tiles; every tile is exactly one key block, so a row's
//   reduction over a tile is that block's log-sum-exp. Four waves split the
//   heads (wave w owns heads 16w .. 16w+15) and share each KV tile, which is
//   staged once in LDS (the one KV head serves every query head). One
//   workgroup per CU, one wave per SIMD with the whole register file: the O
//   accumulator takes 128 VGPRs and the scores 16; Q (72 registers) is held
//   for the whole row in AGPRs, which the score MFMA reads directly. Tiles are
//   double-buffered so the copy of tile t+1 overlaps the MFMAs of tile t.
//
// Contractions (v_mfma_f32_16x16x32_bf16)
//   S^T[key, row] = K_tile[key, :] . Q[row, :]     A = K (LDS), B = Q (AGPRs)
//   Lane l then holds 16 scores of ONE row (head l%16): the softmax row
//   statistics are in-register reductions plus two exchanges across the four
//   16-lane groups.
//   O^T[dim, row] += V^T[dim, key] . P^T[key, row]
//   A = V^T comes from the LDS transpose read ds_read_b64_tr_b16; B = P^T is
//   taken straight from the S^T registers: inside each 32-key k-step the key
//   order is permuted the same way on both operands, so P never moves.
//
// LDS tile layout: 9 groups of 64 columns; group G holds, for each key k, the
//   128 B of columns 64G .. 64G+63 at [G * 8192 + k * 128]. Inside those
//   128 B, 16-byte chunk c8 (8 columns) sits in slot c8 ^ sw(k), with
//   sw(k) = 3 * bit2(k) + 4 * bit1(k): both the score-fragment ds_read_b128
//   reads (lanes {0-7, 32-39}, {8-15, 40-47}, ... share an LDS cycle) and the
//   transpose reads (lanes 0-31, 32-63) are free of bank conflicts. Tiles are
//   filled with global_load_lds_dwordx4 (lane l of a wave instruction writes
//   16 B at base + 16 l): one instruction covers 8 keys x one full 128 B line
//   each.
//
// Issue: with one wave per SIMD, the wave issues at most one instruction per
//   four cycles, and a 16x16x32 MFMA lasts 16. The tile is therefore written
//   as one straight-line stream of 136 MFMAs in which every other instruction
//   counts: each MFMA is followed by the LDS read of the operand six places
//   ahead and preceded by a wait for its own operand only (LDS reads complete
//   in order), the score MFMA takes Q from AGPRs without copies, and the tile
//   copy has no branches.
//
// Softmax: scores live in the log2 domain (scale * log2 e folded in). Per
//   tile, p = exp2(x - m_tile): the tile max is the stabiliser of the block
//   log-sum-exp, so a block far below the running max cannot underflow to
//   -inf. The running reference max is raised only when a tile max exceeds it
//   by more than 8 (factor 256), so O is rescaled rarely; the result is the
//   same up to rounding. The sink enters as the initial reference max
//   sigma * log2 e with weight 1, counted once per row.
#include <hip/hip_runtime.h>

#include <utility>

#include "hs_common.h"
#include "hs_gfx950.h"
#include "hs_kernels.h"
#include "hs_topk_row.h"

namespace hs {

namespace mla {
constexpr int H = 64, DK = 576, DV = 512, BS = 64;
constexpr int NW = 4;                        // waves per workgroup
constexpr int RW = 16;                       // rows (heads) per wave
constexpr int NTHREADS = 64 * NW;
constexpr int NCH = DK / 8;                  // 72 chunks of 8 columns (16 B)
constexpr int NGR = NCH / 8;                 // 9 groups of 8 chunks (64 columns)
constexpr int GR_BYTES = BS * 128;           // one group: 64 keys x 128 B
constexpr int TILE_BYTES = NGR * GR_BYTES;   // 73728
constexpr int KSTEPS = DK / 32;              // 18 k-steps of the score MFMA
constexpr int DBLK = DV / 16;                // 32 column blocks of O
constexpr float TAU = 8.0f;                  // lazy-rescale threshold (log2 units)
}  // namespace mla

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Cross-lane reductions without LDS round trips. A row (head) of the score
// tile lives in lanes {l, l^16, l^32, l^48}; the heads of one wave are the
// 16 lanes of a DPP row.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Max over the 16 lanes of a DPP row: xor 1, xor 2, half-row mirror, row mirror.
__device__ __forceinline__ float max_row16(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  return v;
}

// Wait until at most N LDS operations are outstanding (vmcnt and expcnt left
// at their maxima).
template <int N>
__device__ __forceinline__ void wait_lgkm() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));
}
// LDS operations issued after fragment i of the tile's operand stream that
// may still be pending when MFMA i issues: the fragments requested up to LA - 1
// places ahead (score fragments are one read, V^T fragments two), plus the
// block-score slot write issued at stream position iw.
__host__ __device__ constexpr int stream_pending(int i, int la, int nsf, int nf, int iw) {
  int n = 0;
  for (int f = i + 1; f <= i + la - 1 && f < nf; ++f) n += f < nsf ? 1 : 2;
  if (iw >= 0 && i > iw && i <= iw + la) n += 1;
  return n;
}
// Score MFMA with the Q operand read straight from AGPRs (the builtin in the
// VGPR-accumulator form copies it to VGPRs first: 72 extra instructions per
// tile). Dependent MFMAs on one accumulator are interlocked by the hardware,
// but the compiler inserts no wait states for VALU instructions around inline
// assembly: the score stream below reads these results with VALU code only
// after at least three further MFMAs.
__device__ __forceinline__ f32x4 mfma_q0(bf16x8 k, bf16x8 q) {
  f32x4 d;
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=v"(d) : "v"(k), "a"(q));
  return d;
}
__device__ __forceinline__ f32x4 mfma_q(bf16x8 k, bf16x8 q, f32x4 c) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(k), "a"(q));
  return c;
}
template <int OP, bool SPLIT, bool PAGED>
__global__ __launch_bounds__(mla::NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bf16_kernel(AttnArgs a) {
  using namespace mla;
  // Two separate buffers (not one array with a computed offset): each of the
  // two unrolled step instances reads its tile at compile-time addresses (one
  // array indexed at run time measured about 3 % slower).
  __shared__ __attribute__((aligned(16))) char buf_a[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char buf_b[TILE_BYTES];
  __shared__ float bl_slot[2][NW];
  __shared__ int tile_list[NW][64];

  const Geom& g = a.g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int grp = lane >> 4;     // 16-lane group: k-offset 8*grp inside a k-step
  const int l16 = lane & 15;
  const int head = wave * RW + l16;

  // Work item: heaviest query rows first (causal cost grows with position).
  int w = blockIdx.x;
  const int split = SPLIT ? (w % a.nsplit) : 0;
  if (SPLIT) w /= a.nsplit;
  const int b = w / g.Sq;
  const int r = g.Sq - 1 - (w % g.Sq);
  const size_t row = (size_t)b * g.Sq + r;

  const RowRange rr = row_range<true>(g, OP == kSwaSparse ? kGather : OP, b, r, a.window);
  const int nb_b = nb_of_entry<true>(g, b);
  const Doc rdoc = rr.doc;   // every tile of the row lies in its document
  // window-and-sparse: the window branch's range; its n_w tiles come first
  const RowRange rw = OP == kSwaSparse ? row_range<true>(g, kSwa, b, r, a.window) : rr;
  const int n_w = OP == kSwaSparse ? rw.j_last - rw.j_first + 1 : 0;

  // Tile sequence: a block range, or the listed blocks that intersect the
  // allowed key range (compacted in order of the list).
  // The selection's load first, then the Q loads, so that the Q loads are
  // in flight while the tile list waits for the selection.
  int jsel = -1;
  if (OP == kGather || OP == kSwaSparse) {
    if (lane < a.top_k) jsel = a.block_idx[row * a.top_k + lane];
  }
  // Q rows of this wave as MFMA B operands: lane holds q[row, head, 32ks + 8grp .. +8].
  bf16x8 qreg[KSTEPS];
  {
    const bf16* qp = a.q + (row * H + head) * DK + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qreg[ks] = *(const bf16x8*)(qp + 32 * ks);
  }

  int ntiles;
  if (OP == kGather || OP == kSwaSparse) {
    // Every wave builds its own copy of the list (same indices, same result),
    // so no workgroup barrier separates it from the first copy.
    const int j = jsel;
    bool ok = false;
    if (lane < a.top_k) {
      if (j >= 0 && j < nb_b && block_in_doc(g, rdoc, j)) {
        const Blk bk = block_rows_in(g, rdoc, j);
        ok = !(bk.start > rr.hi || bk.start + bk.len - 1 < rr.lo);
      }
    }
    const unsigned long long m = __ballot(ok);
    const int pos = __popcll(m & ((1ull << lane) - 1ull));
    if (ok) tile_list[wave][pos] = j;
    ntiles = n_w + __popcll(m);
    // LDS operations of one wave complete in order: the reads below see these writes
    __builtin_amdgcn_wave_barrier();
  } else {
    ntiles = rr.j_last - rr.j_first + 1;
  }
  int t_begin = 0, t_end = ntiles;
  if (SPLIT) {
    t_begin = min(ntiles, split * a.split_tiles);
    t_end = min(ntiles, t_begin + a.split_tiles);
    if (split > 0 && t_begin == t_end) {
      // chunk past the end of this row: an empty partial, skipped by the merge
      if (lane < RW) {
        const size_t slot = (size_t)w * a.nsplit + split;
        a.ws_ml[(slot * H + wave * RW + lane) * 2 + 0] = -INFINITY;
        a.ws_ml[(slot * H + wave * RW + lane) * 2 + 1] = 0.f;
      }
      return;
    }
  }
  auto tile_block = [&](int t) -> int {
    if (OP == kSwaSparse) return t < n_w ? rw.j_first + t : tile_list[wave][t - n_w];
    return OP == kGather ? tile_list[wave][t] : rr.j_first + t;
  };

  // Block-score columns this row never visits are -inf.
  if (OP == kScore && split == 0) {
    float* blr = a.block_logit + row * g.NB;
    for (int j = threadIdx.x; j < g.NB; j += NTHREADS)
      if (j < rr.j_first || j > rr.j_last) blr[j] = -INFINITY;
  }

  const bf16* kv_entry = a.kv + (size_t)b * g.Skv * DK;
  // Key block j's rows are base + start .. : the entry's rows in place, or row 0
  // onwards of the block's page in the pool.
  auto block_base = [&](int j) -> const bf16* {
    if (PAGED) return a.kv + (size_t)a.page_table[(size_t)b * a.max_pages + j] * (BS * DK);
    return kv_entry;
  };
  if (t_begin < t_end) {
    const int j0 = tile_block(t_begin);
    const Blk b0 = block_rows_in(g, rdoc, j0);
    stage_tile(buf_a, block_base(j0), PAGED ? 0 : b0.start, b0.len, wave, lane);
  }

  const float sk = (a.sink != nullptr && split == 0) ? a.sink[head] * kLog2e : -INFINITY;
  float m_run = sk;
  float l_run = (sk > -INFINITY && grp == 0) ? 1.0f : 0.0f;  // lane-partial denominator
  f32x4 oacc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  const float sl2 = g.scale_log2;
  int j_prev = -1;  // block whose score partials wait in bl_slot
  int par = 0;

  // Per-lane LDS bases of the score fragments: key 16kb + l16, chunk 4ks +
  // grp (group ks/2, chunk-in-group 4 (ks & 1) + grp) in slot c8 ^ sw(key),
  // where sw depends only on l16 here.
  const int swk = swz(l16);
  const int koff_e = l16 * 128 + 16 * (grp ^ swk);
  const int koff_o = l16 * 128 + 16 * ((4 + grp) ^ swk);
  // Transpose reads: lane i of group grp reads key 32kk (+16) + 4grp + i/4,
  // chunk 2db + ((i >> 1) & 1), byte 8 (i & 1); one base per db & 3.
  const int kloc = 4 * grp + (l16 >> 2);
  const int swv = swz(kloc);
  const int tv = ((l16 >> 1) & 1) ^ swv;
  const int voff = kloc * 128 + 8 * (l16 & 1);
  // Tile copy: lane l of instruction (G, kq) takes key 8kq + l/8 and stores
  // chunk (l%8) ^ sw(key) in slot l%8; wave w issues kq = w and w + 4.
  const int cp_c8 = (lane & 7) ^ swz(8 * wave + (lane >> 3));

  // Window-and-sparse: normalise and store one branch's output, then restart
  // the online softmax (the sink again as the initial reference) for the next.
  auto finalize_to = [&](bf16* outp, float* lsep) __attribute__((always_inline)) {
    const float l_tot = sum_xor32(sum_xor16(l_run));
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    bf16* op = outp + (row * H + head) * DV + 4 * grp;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      bf16x4 v;
      v[0] = (bf16)(oacc[db][0] * inv);
      v[1] = (bf16)(oacc[db][1] * inv);
      v[2] = (bf16)(oacc[db][2] * inv);
      v[3] = (bf16)(oacc[db][3] * inv);
      *(bf16x4*)(op + 16 * db) = v;
    }
    if (grp == 0) lsep[row * H + head] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
  };
  auto restart = [&]() __attribute__((always_inline)) {
    m_run = sk;
    l_run = (sk > -INFINITY && grp == 0) ? 1.0f : 0.0f;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // One tile, processed as two 32-key halves so that in-order issue can
  // overlap VALU with MFMA: the softmax of half 0 runs between the score
  // MFMAs of half 1, the softmax of half 1 between the PV MFMAs of half 0,
  // and the block score between those of half 1. The copy of the next tile
  // is spread over the score MFMAs of half 0.
  auto step = [&](char* cur, char* nxt, int t) __attribute__((always_inline)) {
    if constexpr (OP == kSwaSparse) {
      if (t == n_w) {  // first selected block: the window branch is complete
        finalize_to(a.out2, a.lse2);
        restart();
      }
    }
    const int j = tile_block(t);
    const Blk blk = block_rows_in(g, rdoc, j);
    const int rlo = (OP == kSwaSparse && t < n_w) ? rw.lo : rr.lo;
    const int rhi = (OP == kSwaSparse && t < n_w) ? rw.hi : rr.hi;
    const int klo = rlo - blk.start, khi = min(rhi - blk.start, blk.len - 1);

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // tile t resident; tile t-1 fully consumed; partials visible
    if (OP == kScore && j_prev >= 0 && threadIdx.x == 0) {
      float v = bl_slot[par ^ 1][0];
#pragma unroll
      for (int k = 1; k < NW; ++k) v = fmaxf(v, bl_slot[par ^ 1][k]);
      a.block_logit[row * g.NB + j_prev] = v * kLn2;
    }
    // Copy source: the next tile's block, or on the last tile the current
    // block again into the idle buffer (harmless, and it keeps the copy free
    // of branches inside the MFMA stream).
    const bool has_next = t + 1 < t_end;
    char* cp_dst = nxt + wave * 1024;
    const int jn = has_next ? tile_block(t + 1) : j;
    const Blk nb = has_next ? block_rows_in(g, rdoc, jn) : blk;
    const bf16* nbase = block_base(jn);
    const int nst = PAGED ? 0 : nb.start;
    const int ka = min(8 * wave + (lane >> 3), nb.len - 1);
    const int kb2 = min(8 * (wave + 4) + (lane >> 3), nb.len - 1);
    const char* cp_a = (const char*)(nbase + (size_t)(nst + ka) * DK) + 16 * cp_c8;
    const char* cp_b = (const char*)(nbase + (size_t)(nst + kb2) * DK) + 16 * cp_c8;

    const HS_LDS char* kbe = (const HS_LDS char*)(cur + koff_e);
    const HS_LDS char* kbo = (const HS_LDS char*)(cur + koff_o);
    auto kfrag = [&](int ks, int kb) -> bf16x8 {
      const HS_LDS char* base = (ks & 1) ? kbo : kbe;
      return *(const HS_LDS bf16x8*)(base + (ks >> 1) * GR_BYTES + kb * 2048);
    };
    const HS_LDS char* vb0 = (const HS_LDS char*)(cur + voff);
    auto vfrag = [&](int kk, int db) -> bf16x8 {
      const HS_LDS char* vb =
          vb0 + 16 * ((2 * (db & 3)) ^ tv) + (db >> 2) * GR_BYTES + (32 * kk) * 128;
      const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((HS_LDS bf16x4*)(vb));
      const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((HS_LDS bf16x4*)(vb + 16 * 128));
      bf16x8 va;
      va[0] = lo4[0]; va[1] = lo4[1]; va[2] = lo4[2]; va[3] = lo4[3];
      va[4] = hi4[0]; va[5] = hi4[1]; va[6] = hi4[2]; va[7] = hi4[3];
      return va;
    };

    // Softmax of one half in nine small pieces, issued between MFMAs.
    // x: the 8 scores of this lane (key blocks 2h, 2h+1), then p.
    float xh[2][8];
    float mh[2], sh[2], ph_lane[2];
    auto soft_piece = [&](int h, int piece, const f32x4* sp) __attribute__((always_inline)) {
      float* x = xh[h];
      switch (piece) {
        case 0:
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = sp[2 * h][i] * sl2;
          break;
        case 1:
#pragma unroll
          for (int i = 0; i < 4; ++i) x[4 + i] = sp[2 * h + 1][i] * sl2;
          if (klo > 32 * h || khi < 32 * h + 31) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int m = 32 * h + 16 * (e >> 2) + 4 * grp + (e & 3);
              if (m < klo || m > khi) x[e] = -INFINITY;
            }
          }
          break;
        case 2: {
          float m = x[0];
#pragma unroll
          for (int e = 1; e < 8; ++e) m = fmaxf(m, x[e]);
          mh[h] = max_xor16(m);
          break;
        }
        case 3:
          mh[h] = max_xor32(mh[h]);
          break;
        case 4: {
          const float ms = (mh[h] == -INFINITY) ? 0.f : mh[h];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = fast_exp2(x[e] - ms);
          break;
        }
        case 5: {
          const float ms = (mh[h] == -INFINITY) ? 0.f : mh[h];
#pragma unroll
          for (int e = 4; e < 8; ++e) x[e] = fast_exp2(x[e] - ms);
          break;
        }
        case 6: {
          float ps = x[0];
#pragma unroll
          for (int e = 1; e < 8; ++e) ps += x[e];
          ph_lane[h] = ps;
          break;
        }
        case 7:
          sh[h] = sum_xor16(ph_lane[h]);
          break;
        default:
          sh[h] = sum_xor32(sh[h]);
          break;
      }
    };
    // Online-softmax update for half h and its bf16 P^T operand, in two
    // parts: prepare() assumes the reference max stays (the common case) and
    // can run in an MFMA shadow; commit() raises the reference when the half's
    // max exceeds it by more than TAU (rare), which rescales O and redoes P.
    bf16x8 pbh[2];
    float lph[2];
    auto prepare_half = [&](int h) __attribute__((always_inline)) {
      const float f = (mh[h] == -INFINITY) ? 0.f : fast_exp2(mh[h] - m_run);
      lph[h] = ph_lane[h] * f;
#pragma unroll
      for (int e = 0; e < 8; ++e) pbh[h][e] = (bf16)(xh[h][e] * f);
    };
    auto commit_half = [&](int h) __attribute__((always_inline)) {
      if (mh[h] > m_run + TAU) {
        const float alpha = fast_exp2(m_run - mh[h]);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) oacc[db] *= alpha;
        m_run = mh[h];
        prepare_half(h);
      }
      l_run += lph[h];
    };

    // Operand stream of one tile: 72 score fragments (half h, k-step ks, key
    // block 2h + k), one ds_read_b128 each, then 64 V^T fragments (k-step kk,
    // column block db), two transpose reads each. The fragment LA places ahead
    // is requested right after each MFMA, so LA fragments stay in flight, and
    // each MFMA waits only for its own operand (LDS reads complete in order).
    f32x4 s[4];
    constexpr int NSF = 2 * KSTEPS * 2;  // 72 score fragments
    constexpr int NF = NSF + 2 * DBLK;   // + 64 V^T fragments
    constexpr int LA = 6;
    constexpr int R = LA + 1;
    bf16x8 fr[R];
    auto load_frag = [&](int f) __attribute__((always_inline)) -> bf16x8 {
      if (f < NSF) return kfrag((f % (2 * KSTEPS)) / 2, 2 * (f / (2 * KSTEPS)) + (f & 1));
      return vfrag((f - NSF) / DBLK, (f - NSF) % DBLK);
    };
    wait_lgkm<0>();
    static_for<LA>([&](auto F) __attribute__((always_inline)) {
      constexpr int f = decltype(F)::value;
      fr[f % R] = load_frag(f);
      __builtin_amdgcn_sched_barrier(0);
    });
    __builtin_amdgcn_sched_barrier(0);

    static_for<NF>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      if constexpr (i == NSF + DBLK) commit_half(1);
      wait_lgkm<stream_pending(i, LA, NSF, NF, OP == kScore ? NSF + DBLK + 7 : -1)>();
      if constexpr (i < NSF) {
        constexpr int h = i / (2 * KSTEPS), ks = (i % (2 * KSTEPS)) / 2, k = i & 1;
        if constexpr (ks == 0)
          s[2 * h + k] = mfma_q0(fr[i % R], qreg[ks]);
        else
          s[2 * h + k] = mfma_q(fr[i % R], qreg[ks], s[2 * h + k]);
      } else {
        constexpr int kk = (i - NSF) / DBLK, db = (i - NSF) % DBLK;
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[i % R], pbh[kk], oacc[db], 0, 0, 0);
      }
      if constexpr (i + LA < NF) fr[(i + LA) % R] = load_frag(i + LA);
      if constexpr (i < NSF / 2) {
        // copy column group G of the next tile in the shadow of the half-0 score MFMAs
        if ((i & 3) == 3) {
          const int G = i >> 2;
          dma16(cp_a + 128 * G, cp_dst + G * GR_BYTES);
          dma16(cp_b + 128 * G, cp_dst + G * GR_BYTES + 4096);
        }
      } else if constexpr (i < NSF) {
        // softmax of half 0 in the shadow of the half-1 score MFMAs
        if ((i & 3) == 3) {
          const int gi = (i - NSF / 2) >> 2;
          soft_piece(0, gi, s);
          if (gi == 8) {
            prepare_half(0);
            commit_half(0);
          }
        }
      } else if constexpr (i < NSF + DBLK) {
        // softmax of half 1 in the shadow of the half-0 PV MFMAs
        const int v = i - NSF;
        if (v % 3 == 2 && v / 3 < 9) soft_piece(1, v / 3, s);
        if (v == 29) prepare_half(1);
      } else if constexpr (OP == kScore && i == NSF + DBLK + 7) {
        // block log-sum-exp over both halves, then max over the wave's heads
        const float M = fmaxf(mh[0], mh[1]);
        float bl = -INFINITY;
        if (M > -INFINITY)
          bl = M + fast_log2(sh[0] * fast_exp2(mh[0] - M) + sh[1] * fast_exp2(mh[1] - M));
        bl = max_row16(bl);
        bl_slot[par][wave] = bl;  // every lane holds the same value
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    if (OP == kScore) {
      j_prev = j;
      par ^= 1;
    }
  };

  for (int t = t_begin; t < t_end; t += 2) {
    step(buf_a, buf_b, t);
    if (t + 1 < t_end) step(buf_b, buf_a, t + 1);
  }
  __builtin_amdgcn_s_waitcnt(0);  // the last tile's spare copy has landed
  if constexpr (OP == kSwaSparse) {
    if (t_end <= n_w) {  // no selected block met the row: the sparse branch is empty
      finalize_to(a.out2, a.lse2);
      restart();
    }
  }

  // every wave is past the last tile and every copy has landed: the tile
  // buffers are free for the output transpose below
  __syncthreads();
  if (OP == kScore && j_prev >= 0 && threadIdx.x == 0) {
    float v = bl_slot[par ^ 1][0];
#pragma unroll
    for (int k = 1; k < NW; ++k) v = fmaxf(v, bl_slot[par ^ 1][k]);
    a.block_logit[row * g.NB + j_prev] = v * kLn2;
  }

  const float l_tot = sum_xor32(sum_xor16(l_run));
  // oacc[db][i] is O[row l16][dim 16db + 4grp + i].
  if (!SPLIT && (OP != kSwaSparse || a.out_mix == nullptr)) {
    // The wave's 16 x 512 bf16 outputs go through LDS (its own 16.25 KB of
    // the free tile buffer, head rows 1040 B apart against bank conflicts)
    // so that each store writes one head's whole 1 KB row: a lane's own
    // values are 8 B pieces of 16 different rows, which stored directly cost
    // 16 memory segments per store instruction.
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    constexpr int OROW = 2 * DV + 16;
    HS_LDS char* ob = (HS_LDS char*)buf_a + wave * (RW * OROW);
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      bf16x4 v;
      v[0] = (bf16)(oacc[db][0] * inv);
      v[1] = (bf16)(oacc[db][1] * inv);
      v[2] = (bf16)(oacc[db][2] * inv);
      v[3] = (bf16)(oacc[db][3] * inv);
      *(HS_LDS bf16x4*)(ob + l16 * OROW + 2 * (16 * db + 4 * grp)) = v;
    }
    // (LDS operations of one wave complete in order)
    bf16* orow = a.out + (row * H + wave * RW) * DV + 8 * lane;
#pragma unroll
    for (int h = 0; h < RW; ++h)
      *(bf16x8*)(orow + h * DV) = *(const HS_LDS bf16x8*)(ob + h * OROW + 16 * lane);
    if (grp == 0)
      a.lse[row * H + head] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
  } else if (!SPLIT) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    bf16* op = a.out + (row * H + head) * DV + 4 * grp;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      bf16x4 v;
      v[0] = (bf16)(oacc[db][0] * inv);
      v[1] = (bf16)(oacc[db][1] * inv);
      v[2] = (bf16)(oacc[db][2] * inv);
      v[3] = (bf16)(oacc[db][3] * inv);
      *(bf16x4*)(op + 16 * db) = v;
    }
    if (grp == 0)
      a.lse[row * H + head] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
    if constexpr (OP == kSwaSparse) {
      // Gated sum of the two branches from their stored bf16 values (this lane
      // wrote both rows of columns it now reads).
      if (a.out_mix != nullptr) {
        const float ga = a.gate_a[row * H + head], gb = a.gate_b[row * H + head];
        const bf16* sw = a.out2 + (row * H + head) * DV + 4 * grp;
        const bf16* sp = a.out + (row * H + head) * DV + 4 * grp;
        bf16* mp = a.out_mix + (row * H + head) * DV + 4 * grp;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
          const bf16x4 x = *(const bf16x4*)(sw + 16 * db);
          const bf16x4 y = *(const bf16x4*)(sp + 16 * db);
          bf16x4 m;
#pragma unroll
          for (int e = 0; e < 4; ++e) m[e] = (bf16)gated_mix(ga, (float)x[e], gb, (float)y[e]);
          *(bf16x4*)(mp + 16 * db) = m;
        }
      }
    }
  } else {
    // Unnormalised partial: O (fp32), reference max (log2) and denominator.
    const size_t slot = (size_t)w * a.nsplit + split;
    float* op = a.ws_o + (slot * H + head) * DV + 4 * grp;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) *(f32x4*)(op + 16 * db) = oacc[db];
    if (grp == 0) {
      a.ws_ml[(slot * H + head) * 2 + 0] = m_run;
      a.ws_ml[(slot * H + head) * 2 + 1] = l_tot;
    }
  }
}

// Merge split partials: one wave per (item, head); lane owns 8 columns. With
// PER > 0 the launch has one more wave per row that selects the row's top-k
// blocks from the complete block scores (PER = ceil(NB / 64)).
template <int PER>
__global__ __launch_bounds__(64) void merge_bf16_kernel(AttnArgs a) {
  using namespace mla;
  if constexpr (PER > 0) {
    if ((int)blockIdx.x >= a.g.B * a.g.Sq * H) {
      const int rowi = blockIdx.x - a.g.B * a.g.Sq * H;
      float lmax2 = 0.f;
      if (a.topk_prob != nullptr) {
        // the row's per-head lse in log2 units, formed from the partials as
        // the merge waves of this launch form it (lane = head)
        const int bb = rowi / a.g.Sq, rq = rowi % a.g.Sq;
        const int item = bb * a.g.Sq + (a.g.Sq - 1 - rq);
        const int head = threadIdx.x;
        float M = -INFINITY;
        for (int s = 0; s < a.nsplit; ++s) {
          const size_t slot = (size_t)item * a.nsplit + s;
          if (a.ws_ml[(slot * H + head) * 2 + 1] > 0.f) M = fmaxf(M, a.ws_ml[(slot * H + head) * 2]);
        }
        float L = 0.f;
        if (M > -INFINITY)
          for (int s = 0; s < a.nsplit; ++s) {
            const size_t slot = (size_t)item * a.nsplit + s;
            const float l = a.ws_ml[(slot * H + head) * 2 + 1];
            if (l > 0.f) L += l * fast_exp2(a.ws_ml[(slot * H + head) * 2] - M);
          }
        lmax2 = wave_max_f(L > 0.f ? M + fast_log2(L) : -INFINITY);
      }
      __shared__ unsigned pack[192];
      topk_row<PER>(a.g, a.block_logit, a.topk_idx, a.topk_k, rowi, threadIdx.x, pack,
                    a.topk_prob, lmax2);
      return;
    }
  }
  const int item = blockIdx.x / H;
  const int head = blockIdx.x % H;
  const int lane = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) {
    const size_t slot = (size_t)item * a.nsplit + s;
    const float m = a.ws_ml[(slot * H + head) * 2 + 0];
    const float l = a.ws_ml[(slot * H + head) * 2 + 1];
    if (l > 0.f) M = fmaxf(M, m);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (M > -INFINITY) {
    for (int s = 0; s < a.nsplit; ++s) {
      const size_t slot = (size_t)item * a.nsplit + s;
      const float m = a.ws_ml[(slot * H + head) * 2 + 0];
      const float l = a.ws_ml[(slot * H + head) * 2 + 1];
      if (!(l > 0.f)) continue;
      const float wgt = fast_exp2(m - M);
      L += l * wgt;
      const float* op = a.ws_o + (slot * H + head) * DV + 8 * lane;
      const f32x4 v0 = *(const f32x4*)op;
      const f32x4 v1 = *(const f32x4*)(op + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += v0[e] * wgt;
        acc[4 + e] += v1[e] * wgt;
      }
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (bf16)(acc[e] * inv);
  // Items follow the launch order of the attention kernel: item = b*Sq + (Sq-1-r).
  const int b = item / a.g.Sq;
  const int r = a.g.Sq - 1 - (item % a.g.Sq);
  const size_t row = (size_t)b * a.g.Sq + r;
  *(bf16x8*)(a.out + (row * H + head) * DV + 8 * lane) = o;
  if (lane == 0) a.lse[row * H + head] = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
}

template <bool PAGED>
void launch_attn_kernels(int op, const AttnArgs& a, dim3 grid, dim3 block, hipStream_t stream) {
  if (a.nsplit == 1) {
    if (op == kScore) hipLaunchKernelGGL((attn_bf16_kernel<kScore, false, PAGED>), grid, block, 0, stream, a);
    else if (op == kGather) hipLaunchKernelGGL((attn_bf16_kernel<kGather, false, PAGED>), grid, block, 0, stream, a);
    else if (op == kSwa) hipLaunchKernelGGL((attn_bf16_kernel<kSwa, false, PAGED>), grid, block, 0, stream, a);
    else if constexpr (!PAGED) hipLaunchKernelGGL((attn_bf16_kernel<kSwaSparse, false, false>), grid, block, 0, stream, a);
  } else {
    if (op == kScore) hipLaunchKernelGGL((attn_bf16_kernel<kScore, true, PAGED>), grid, block, 0, stream, a);
    else if (op == kGather) hipLaunchKernelGGL((attn_bf16_kernel<kGather, true, PAGED>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<kSwa, true, PAGED>), grid, block, 0, stream, a);
  }
}

int attn_bf16_launch(int op, const AttnArgs& a, hipStream_t stream) {
  const int items = a.g.B * a.g.Sq;
  const dim3 block(mla::NTHREADS);
  const dim3 grid((unsigned)(items * a.nsplit));
  // Paged KV is a separate instantiation, so the in-place path carries no
  // page-table code at all.
  if (a.page_table != nullptr) launch_attn_kernels<true>(op, a, grid, block, stream);
  else launch_attn_kernels<false>(op, a, grid, block, stream);
  if (a.nsplit > 1) {
    const unsigned waves = (unsigned)(items * mla::H);
    if (a.topk_idx == nullptr) {
      hipLaunchKernelGGL(merge_bf16_kernel<0>, dim3(waves), dim3(64), 0, stream, a);
    } else {
      // the block scores are complete once the split kernel has finished: the
      // top-k runs as extra waves of the merge launch
      const dim3 grid(waves + (unsigned)items);
      const int NB = a.g.NB;
      if (NB <= 64) hipLaunchKernelGGL(merge_bf16_kernel<1>, grid, dim3(64), 0, stream, a);
      else if (NB <= 128) hipLaunchKernelGGL(merge_bf16_kernel<2>, grid, dim3(64), 0, stream, a);
      else if (NB <= 256) hipLaunchKernelGGL(merge_bf16_kernel<4>, grid, dim3(64), 0, stream, a);
      else if (NB <= 512) hipLaunchKernelGGL(merge_bf16_kernel<8>, grid, dim3(64), 0, stream, a);
      else if (NB <= 1024) hipLaunchKernelGGL(merge_bf16_kernel<16>, grid, dim3(64), 0, stream, a);
      else if (NB <= 2048) hipLaunchKernelGGL(merge_bf16_kernel<32>, grid, dim3(64), 0, stream, a);
      else hipLaunchKernelGGL(merge_bf16_kernel<64>, grid, dim3(64), 0, stream, a);
    }
  } else if (a.topk_idx != nullptr) {
    // One row per workgroup: the standalone top-k kernel, whose many waves per
    // CU hide the per-row search latency that an epilogue would expose.
    TopkArgs t;
    t.block_logit = a.block_logit;
    t.block_idx = a.topk_idx;
    t.top_k = a.topk_k;
    t.lse = a.lse;
    t.block_prob = a.topk_prob;
    t.g = a.g;
    const int err = (int)hipGetLastError();
    if (err != 0) return err;
    return topk_launch(t, stream);
  }
  return (int)hipGetLastError();
}

}  // namespace hs
