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
//   workgroup per CU, one wave per SIMD: Q stays in 72 VGPRs, the O
//   accumulator takes 128, the scores 16. Tiles are double-buffered so the
//   copy of tile t+1 overlaps the MFMAs of tile t.
//
// Contractions (v_mfma_f32_16x16x32_bf16)
//   S^T[key, row] = K_tile[key, :] . Q[row, :]     A = K (LDS), B = Q (VGPRs)
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
//   sw(k) = 2 * ((k >> 1) & 3) + ((k >> 3) & 1). The swizzle makes the 16
//   keys of a score-fragment read, and the 8 keys x 2 chunks of a
//   transpose-read half-wave, land on distinct banks. Tiles are filled with
//   global_load_lds_dwordx4 (lane l of a wave instruction writes 16 B at base
//   + 16 l): one instruction covers 8 keys x one full 128 B line each.
//
// Softmax: scores live in the log2 domain (scale * log2 e folded in). Per
//   tile, p = exp2(x - m_tile): the tile max is the stabiliser of the block
//   log-sum-exp, so a block far below the running max cannot underflow to
//   -inf. The running reference max is raised only when a tile max exceeds it
//   by more than 8 (factor 256), so O is rescaled rarely; the result is the
//   same up to rounding. The sink enters as the initial reference max
//   sigma * log2 e with weight 1, counted once per row.
#include <hip/hip_runtime.h>

#include "hs_common.h"
#include "hs_kernels.h"

namespace hs {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define HS_LDS __attribute__((address_space(3)))
#define HS_GLB __attribute__((address_space(1)))

namespace mla {
constexpr int H = 64, DK = 576, DV = 512, BS = 64;
constexpr int NW = 4;                        // waves per workgroup
constexpr int NTHREADS = 64 * NW;
constexpr int NCH = DK / 8;                  // 72 chunks of 8 columns (16 B)
constexpr int NGR = NCH / 8;                 // 9 groups of 8 chunks (64 columns)
constexpr int GR_BYTES = BS * 128;           // one group: 64 keys x 128 B
constexpr int TILE_BYTES = NGR * GR_BYTES;   // 73728
constexpr int KSTEPS = DK / 32;              // 18 k-steps of the score MFMA
constexpr int DBLK = DV / 16;                // 32 column blocks of O
constexpr float TAU = 8.0f;                  // lazy-rescale threshold (log2 units)
constexpr int SG = 2;                        // k-steps per score prefetch group
constexpr int PG = 8;                        // column blocks per PV prefetch group
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

// Wait for outstanding LDS reads only (lgkmcnt(0); vmcnt and expcnt left at
// their maxima so in-flight tile copies keep running).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Copy one 64-key tile (rows [start, start+len), clamped) into an LDS buffer.
// Instruction n = (G, kq) = (n / 8, n % 8) fills keys 8kq .. 8kq+7 of column
// group G; lane l takes key 8kq + l/8 and stores slot l%8, i.e. chunk
// (l%8) ^ sw(key). Wave w issues n = w + 4i, so kq alternates between w and
// w + 4 and G = i / 2: two source rows per lane, immediate offsets otherwise.
__device__ __forceinline__ void stage_tile(char* buf, const bf16* kv_entry, const Blk& blk,
                                           int wave_u, int lane) {
  using namespace mla;
  const int kl = lane >> 3;                                    // key inside the octet
  const int c8 = (lane & 7) ^ (2 * ((lane >> 4) & 3) + (wave_u & 1));
  const int ka = min(8 * wave_u + kl, blk.len - 1);           // kq = w
  const int kb = min(8 * (wave_u + 4) + kl, blk.len - 1);     // kq = w + 4
  const char* src_a = (const char*)(kv_entry + (size_t)(blk.start + ka) * DK) + 16 * c8;
  const char* src_b = (const char*)(kv_entry + (size_t)(blk.start + kb) * DK) + 16 * c8;
  char* dst = buf + wave_u * 1024;
#pragma unroll
  for (int G = 0; G < NGR; ++G) {
    __builtin_amdgcn_global_load_lds((const HS_GLB void*)(src_a + 128 * G),
                                     (HS_LDS void*)(dst + G * GR_BYTES), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const HS_GLB void*)(src_b + 128 * G),
                                     (HS_LDS void*)(dst + G * GR_BYTES + 4096), 16, 0, 0);
  }
}

template <int OP, bool SPLIT>
__global__ __launch_bounds__(mla::NTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bf16_kernel(AttnArgs a) {
  using namespace mla;
  // Two separate buffers (not one array with a computed offset) so that the
  // compiler can prove a tile copy in flight never aliases the tile being read.
  __shared__ __attribute__((aligned(16))) char buf_a[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char buf_b[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) bf16x8 px[NW][2][64];  // P^T operands per wave
  __shared__ float mx_x[NW][2][16];                               // half-tile row max / l
  __shared__ float ps_x[NW][2][16];                               // half-tile row sums
  __shared__ float bl_slot[2][2];
  __shared__ int tile_list[64];
  __shared__ int tile_count;

  const Geom& g = a.g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int rh = wave >> 1;      // head half: heads 32rh .. 32rh+31 (two 16-row blocks)
  const int dh = wave & 1;       // key half of the scores / column half of O
  const int grp = lane >> 4;     // 16-lane group: k-offset 8*grp inside a k-step
  const int l16 = lane & 15;

  // Work item: heaviest query rows first (causal cost grows with position).
  int w = blockIdx.x;
  const int split = SPLIT ? (w % a.nsplit) : 0;
  if (SPLIT) w /= a.nsplit;
  const int b = w / g.Sq;
  const int r = g.Sq - 1 - (w % g.Sq);
  const size_t row = (size_t)b * g.Sq + r;

  const RowRange rr = row_range(g, OP, b, r, a.window);
  const int nb_b = nb_of_entry(g, b);

  // Tile sequence: a block range, or the listed blocks that intersect the
  // allowed key range (compacted in order of the list).
  int ntiles;
  if (OP == kGather) {
    if (wave == 0) {
      int j = -1;
      bool ok = false;
      if (lane < a.top_k) {
        j = a.block_idx[row * a.top_k + lane];
        if (j >= 0 && j < nb_b) {
          const Blk bk = block_rows(g, b, j);
          ok = !(bk.start > rr.hi || bk.start + bk.len - 1 < rr.lo);
        }
      }
      const unsigned long long m = __ballot(ok);
      const int pos = __popcll(m & ((1ull << lane) - 1ull));
      if (ok) tile_list[pos] = j;
      if (lane == 0) tile_count = __popcll(m);
    }
    __syncthreads();
    ntiles = tile_count;
  } else {
    ntiles = rr.j_last - rr.j_first + 1;
  }
  int t_begin = 0, t_end = ntiles;
  if (SPLIT) {
    const int per = (ntiles + a.nsplit - 1) / a.nsplit;
    t_begin = min(ntiles, split * per);
    t_end = min(ntiles, t_begin + per);
  }
  auto tile_block = [&](int t) -> int { return OP == kGather ? tile_list[t] : rr.j_first + t; };

  // Block-score columns this row never visits are -inf.
  if (OP == kScore && split == 0) {
    float* blr = a.block_logit + row * g.NB;
    for (int j = threadIdx.x; j < g.NB; j += NTHREADS)
      if (j < rr.j_first || j > rr.j_last) blr[j] = -INFINITY;
  }

  const bf16* kv_entry = a.kv + (size_t)b * g.Skv * DK;
  if (t_begin < t_end) stage_tile(buf_a, kv_entry, block_rows(g, b, tile_block(t_begin)), wave, lane);

  // Q of the two head blocks as MFMA B operands: lane holds
  // q[row, 32rh + 16hb + l16, 32ks + 8grp .. +8].
  bf16x8 qreg[2][KSTEPS];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const bf16* qp = a.q + (row * H + 32 * rh + 16 * hb + l16) * DK + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qreg[hb][ks] = *(const bf16x8*)(qp + 32 * ks);
  }

  // Running state per head block. The sink enters once per row: on the
  // column-half-0 wave, as the initial reference with weight 1.
  float m_run[2], l_run[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const float sk = (a.sink != nullptr && split == 0) ? a.sink[32 * rh + 16 * hb + l16] * kLog2e
                                                       : -INFINITY;
    m_run[hb] = sk;
    l_run[hb] = (sk > -INFINITY && dh == 0 && grp == 0) ? 1.0f : 0.0f;
  }
  f32x4 oacc[2][DBLK / 2];  // O^T[dims 256dh + 16dbl + 4grp + i][head 32rh + 16hb + l16]
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int d = 0; d < DBLK / 2; ++d) oacc[hb][d] = f32x4{0.f, 0.f, 0.f, 0.f};

  const float sl2 = g.scale_log2;
  int j_prev = -1;  // block whose score partials wait in bl_slot
  int par = 0;

  // Per-lane LDS bases. Score fragments: key 16kb + l16, chunk 4ks + grp
  // (group ks/2, chunk-in-group 4 (ks & 1) + grp) in slot c8 ^ sw(key).
  const int swk = 2 * ((l16 >> 1) & 3) + ((l16 >> 3) & 1);
  const int koff_e = l16 * 128 + 16 * (grp ^ swk);
  const int koff_o = l16 * 128 + 16 * ((4 + grp) ^ swk);
  // Transpose reads: lane i of group grp reads key 32kk (+16) + 4grp + i/4,
  // chunk 2db + ((i >> 1) & 1), byte 8 (i & 1); four bases for db & 3.
  const int kloc = 4 * grp + (l16 >> 2);
  const int swv = 2 * ((kloc >> 1) & 3) + ((kloc >> 3) & 1);
  const int tv = ((l16 >> 1) & 1) ^ swv;
  const int voff = kloc * 128 + 8 * (l16 & 1);

  // One tile: half-tile scores, max exchange, P exchange, PV on own columns,
  // while the next tile streams into `nxt`.
  auto step = [&](char* cur, char* nxt, int t) __attribute__((always_inline)) {
    const int j = tile_block(t);
    const Blk blk = block_rows(g, b, j);

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // tile t resident; tile t-1 fully consumed; partials visible
    if (OP == kScore && j_prev >= 0 && threadIdx.x == 0) {
      const float v = fmaxf(bl_slot[par ^ 1][0], bl_slot[par ^ 1][1]);
      a.block_logit[row * g.NB + j_prev] = v * kLn2;
    }
    if (t + 1 < t_end) stage_tile(nxt, kv_entry, block_rows(g, b, tile_block(t + 1)), wave, lane);

    // S^T for keys 32dh .. 32dh+31 (local key blocks kbl = 0, 1) of both head
    // blocks; each K fragment feeds two MFMAs.
    f32x4 s[2][2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int kbl = 0; kbl < 2; ++kbl) s[hb][kbl] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      const HS_LDS char* kbe = (const HS_LDS char*)(cur + koff_e + dh * 4096);
      const HS_LDS char* kbo = (const HS_LDS char*)(cur + koff_o + dh * 4096);
      auto kfrag = [&](int ks, int kbl) -> bf16x8 {
        const HS_LDS char* base = (ks & 1) ? kbo : kbe;
        return *(const HS_LDS bf16x8*)(base + (ks >> 1) * GR_BYTES + kbl * 2048);
      };
      bf16x8 fa[2 * SG], fb[2 * SG];
#pragma unroll
      for (int u = 0; u < SG; ++u)
#pragma unroll
        for (int kbl = 0; kbl < 2; ++kbl) fa[2 * u + kbl] = kfrag(u, kbl);
#pragma unroll
      for (int gi = 0; gi < KSTEPS / SG; ++gi) {
        bf16x8* fc = (gi & 1) ? fb : fa;
        bf16x8* fn = (gi & 1) ? fa : fb;
        wait_lds();
        if (gi + 1 < KSTEPS / SG) {
#pragma unroll
          for (int u = 0; u < SG; ++u)
#pragma unroll
            for (int kbl = 0; kbl < 2; ++kbl) fn[2 * u + kbl] = kfrag((gi + 1) * SG + u, kbl);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < SG; ++u)
#pragma unroll
          for (int kbl = 0; kbl < 2; ++kbl)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
              s[hb][kbl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  fc[2 * u + kbl], qreg[hb][gi * SG + u], s[hb][kbl], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // Log2 domain; s[hb][kbl][i] is key 32dh + 16kbl + 4grp + i of head block
    // hb, row l16. Keys outside [lo, hi] or past the block end are masked.
    float x[2][8];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int kbl = 0; kbl < 2; ++kbl)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[hb][4 * kbl + i] = s[hb][kbl][i] * sl2;
    {
      const int klo = rr.lo - blk.start, khi = min(rr.hi - blk.start, blk.len - 1);
      if (klo > 32 * dh || khi < 32 * dh + 31) {
#pragma unroll
        for (int kbl = 0; kbl < 2; ++kbl)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = 32 * dh + 16 * kbl + 4 * grp + i;
            if (m < klo || m > khi) {
              x[0][4 * kbl + i] = -INFINITY;
              x[1][4 * kbl + i] = -INFINITY;
            }
          }
      }
    }
    float mh[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float m = x[hb][0];
#pragma unroll
      for (int i = 1; i < 8; ++i) m = fmaxf(m, x[hb][i]);
      mh[hb] = max_xor32(max_xor16(m));
    }
    if (grp == 0) {
      mx_x[wave][0][l16] = mh[0];
      mx_x[wave][1][l16] = mh[1];
    }
    __syncthreads();  // half-tile maxima visible
    float mt[2], f[2], psum[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      mt[hb] = fmaxf(mh[hb], mx_x[wave ^ 1][hb][l16]);
      const float msafe = (mt[hb] == -INFINITY) ? 0.f : mt[hb];
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[hb][i] = fast_exp2(x[hb][i] - msafe);  // now p
        ps += x[hb][i];
      }
      psum[hb] = sum_xor32(sum_xor16(ps));
      // Online softmax with a lazily raised reference max; both waves of the
      // pair see the same tile max, so they take the same decisions.
      if (mt[hb] > m_run[hb] + TAU) {
        const float alpha = fast_exp2(m_run[hb] - mt[hb]);
        l_run[hb] *= alpha;
#pragma unroll
        for (int d = 0; d < DBLK / 2; ++d) oacc[hb][d] *= alpha;
        m_run[hb] = mt[hb];
      }
      f[hb] = (mt[hb] == -INFINITY) ? 0.f : fast_exp2(mt[hb] - m_run[hb]);
      if (grp == 0) l_run[hb] += psum[hb] * f[hb];
    }

    // P^T B operands of the own 32-key half, shared with the partner wave,
    // which owns the other half.
    bf16x8 p_own[2], p_oth[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int e = 0; e < 8; ++e) p_own[hb][e] = (bf16)(x[hb][e] * f[hb]);
      px[wave][hb][lane] = p_own[hb];
    }
    if (grp == 0) {
      ps_x[wave][0][l16] = psum[0];
      ps_x[wave][1][l16] = psum[1];
    }
    __syncthreads();  // P halves and half sums visible
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) p_oth[hb] = px[wave ^ 1][hb][lane];

    if (OP == kScore) {
      // Block log-sum-exp of each head over all 64 keys; max over the heads.
      float bl = -INFINITY;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const float tot = psum[hb] + ps_x[wave ^ 1][hb][l16];
        const float v = (mt[hb] == -INFINITY) ? -INFINITY : mt[hb] + fast_log2(tot);
        bl = fmaxf(bl, v);
      }
      bl = max_row16(bl);
      if (dh == 0 && lane == 0) bl_slot[par][rh] = bl;
      j_prev = j;
      par ^= 1;
    }

    // O^T[own 256 columns] += V^T . P^T over both 32-key k-steps (k-step 0 =
    // the own key half, 1 = the partner's). Each V^T fragment feeds both head
    // blocks.
    {
      const HS_LDS char* vb_own =
          (const HS_LDS char*)(cur + voff + (4 * dh) * GR_BYTES + (32 * dh) * 128);
      const HS_LDS char* vb_oth =
          (const HS_LDS char*)(cur + voff + (4 * dh) * GR_BYTES + (32 * (dh ^ 1)) * 128);
      auto vfrag = [&](int kk, int dbl) -> bf16x8 {
        // global column block 16dh + dbl: group 4dh + dbl/4, chunk pair dbl & 3
        const HS_LDS char* vb = (kk ? vb_oth : vb_own) + 16 * ((2 * (dbl & 3)) ^ tv) +
                                (dbl >> 2) * GR_BYTES;
        const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((HS_LDS bf16x4*)(vb));
        const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((HS_LDS bf16x4*)(vb + 16 * 128));
        bf16x8 va;
        va[0] = lo4[0]; va[1] = lo4[1]; va[2] = lo4[2]; va[3] = lo4[3];
        va[4] = hi4[0]; va[5] = hi4[1]; va[6] = hi4[2]; va[7] = hi4[3];
        return va;
      };
      constexpr int NV = 2 * (DBLK / 2);  // (kk, dbl) fragments
      constexpr int NGRP = NV / PG;
      bf16x8 va[PG], vb2[PG];
#pragma unroll
      for (int u = 0; u < PG; ++u) va[u] = vfrag(u / (DBLK / 2), u % (DBLK / 2));
#pragma unroll
      for (int gi = 0; gi < NGRP; ++gi) {
        bf16x8* vc = (gi & 1) ? vb2 : va;
        bf16x8* vn = (gi & 1) ? va : vb2;
        wait_lds();
        if (gi + 1 < NGRP) {
#pragma unroll
          for (int u = 0; u < PG; ++u) {
            const int n = (gi + 1) * PG + u;
            vn[u] = vfrag(n / (DBLK / 2), n % (DBLK / 2));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < PG; ++u) {
          const int n = gi * PG + u;
          const int kk = n / (DBLK / 2), dbl = n % (DBLK / 2);
#pragma unroll
          for (int hb = 0; hb < 2; ++hb)
            oacc[hb][dbl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                vc[u], kk ? p_oth[hb] : p_own[hb], oacc[hb][dbl], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  for (int t = t_begin; t < t_end; t += 2) {
    step(buf_a, buf_b, t);
    if (t + 1 < t_end) step(buf_b, buf_a, t + 1);
  }

  // Row denominators: each wave holds the partial of its own key halves.
  float l_part[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) l_part[hb] = sum_xor32(sum_xor16(l_run[hb]));
  __syncthreads();
  if (OP == kScore && j_prev >= 0 && threadIdx.x == 0) {
    const float v = fmaxf(bl_slot[par ^ 1][0], bl_slot[par ^ 1][1]);
    a.block_logit[row * g.NB + j_prev] = v * kLn2;
  }
  if (grp == 0) {
    mx_x[wave][0][l16] = l_part[0];
    mx_x[wave][1][l16] = l_part[1];
  }
  __syncthreads();
  float l_tot[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) l_tot[hb] = l_part[hb] + mx_x[wave ^ 1][hb][l16];

  // oacc[hb][dbl][i] is O[head 32rh + 16hb + l16][column 256dh + 16dbl + 4grp + i].
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int head = 32 * rh + 16 * hb + l16;
    if (!SPLIT) {
      const float inv = l_tot[hb] > 0.f ? 1.0f / l_tot[hb] : 0.f;
      bf16* op = a.out + (row * H + head) * DV + 256 * dh + 4 * grp;
#pragma unroll
      for (int d = 0; d < DBLK / 2; ++d) {
        bf16x4 v;
        v[0] = (bf16)(oacc[hb][d][0] * inv);
        v[1] = (bf16)(oacc[hb][d][1] * inv);
        v[2] = (bf16)(oacc[hb][d][2] * inv);
        v[3] = (bf16)(oacc[hb][d][3] * inv);
        *(bf16x4*)(op + 16 * d) = v;
      }
      if (dh == 0 && grp == 0)
        a.lse[row * H + head] =
            l_tot[hb] > 0.f ? (m_run[hb] + fast_log2(l_tot[hb])) * kLn2 : -INFINITY;
    } else {
      // Unnormalised partial: O (fp32), reference max (log2) and denominator.
      const size_t slot = (size_t)w * a.nsplit + split;
      float* op = a.ws_o + (slot * H + head) * DV + 256 * dh + 4 * grp;
#pragma unroll
      for (int d = 0; d < DBLK / 2; ++d) *(f32x4*)(op + 16 * d) = oacc[hb][d];
      if (dh == 0 && grp == 0) {
        a.ws_ml[(slot * H + head) * 2 + 0] = m_run[hb];
        a.ws_ml[(slot * H + head) * 2 + 1] = l_tot[hb];
      }
    }
  }
}

// Merge split partials: one wave per (item, head); lane owns 8 columns.
__global__ __launch_bounds__(64) void merge_bf16_kernel(AttnArgs a) {
  using namespace mla;
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

int attn_bf16_launch(int op, const AttnArgs& a, hipStream_t stream) {
  const int items = a.g.B * a.g.Sq;
  const dim3 block(mla::NTHREADS);
  const dim3 grid((unsigned)(items * a.nsplit));
  if (a.nsplit == 1) {
    if (op == kScore) hipLaunchKernelGGL((attn_bf16_kernel<kScore, false>), grid, block, 0, stream, a);
    else if (op == kGather) hipLaunchKernelGGL((attn_bf16_kernel<kGather, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<kSwa, false>), grid, block, 0, stream, a);
  } else {
    if (op == kScore) hipLaunchKernelGGL((attn_bf16_kernel<kScore, true>), grid, block, 0, stream, a);
    else if (op == kGather) hipLaunchKernelGGL((attn_bf16_kernel<kGather, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<kSwa, true>), grid, block, 0, stream, a);
    hipLaunchKernelGGL(merge_bf16_kernel, dim3((unsigned)(items * mla::H)), dim3(64), 0, stream, a);
  }
  return (int)hipGetLastError();
}

}  // namespace hs
