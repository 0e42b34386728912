/*
 * hs.h -- C ABI of the HySparse MQA sparse-attention forward path on MI355X
 * (gfx950).
 *
 * The method (page "HySparse MQA sparse attention (FA4 block scoring + SWA MQA
 * + block-sparse DSA gather)", sections "What" and "Core") is three
 * cooperating structures over one shared latent KV head: a causal full
 * attention that also emits a scaled score per key block, a per-token top-k
 * selection of key blocks, and an attention that gathers only the selected
 * blocks; a sliding-window MQA branch runs beside them. Every attention call
 * takes an optional learnable per-head sink (same page, "Core", the learnable
 * per-head attn_sink bullet).
 *
 * Shapes follow the absorbed-MLA layout of the same page, section "FlashMLA
 * sparse kernel constraints": one KV head whose rows hold Dk = kv_lora_rank +
 * rope columns; the value of key i is the leading Dv columns of that row.
 *
 * Supported instantiations (anything else returns HS_ERR_UNSUPPORTED):
 *   HS_BF16: H = 64, Dk = 576, Dv = 512, block_size = 64
 *   HS_F32 : 1 <= H <= 16, 1 <= Dk <= 128, 1 <= Dv <= Dk, block_size = 64
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layouts (row-major, innermost stride 1, all device pointers 16-byte
 * aligned):
 *   q           [B, Sq, H, Dk]   dtype
 *   kv          [B, Skv, Dk]     dtype   (value = kv[..., :Dv])
 *   sink        [H]              float32, or NULL (= no sink, i.e. -inf)
 *   out         [B, Sq, H, Dv]   dtype
 *   lse         [B, Sq, H]       float32, natural log, sink included
 *   block_logit [B, Sq, NB]      float32, NB = hs_num_blocks()
 *   block_idx   [B, Sq, top_k]   int32
 * Positions: query row r of batch b sits at absolute position
 *   p = L_b - Sq + r, where L_b = kv_lens[b] (or Skv when kv_lens is NULL);
 * a decode token is the last row of its cache (blog page on the unified
 * sparse-attention dispatcher, decode paragraph: key length = cache +
 * current token). The allowed keys of p are doc_start(p) <= i <= p.
 * Documents: optional packed-document bounds (B == 1, Sq == Skv, doc_start /
 * doc_end tile [0, Sq) in ascending contiguous order). Blocks restart at each
 * document's first row and never cross a document (review of PaddleFleet PR
 * 1453, block-score PyLayer comments: the block_bos input). Block ids are
 * global, numbered in document order.
 * Ownership: every tensor pointer is caller-owned device memory; the library
 * allocates nothing, keeps no pointer after return, and copies the small host
 * arrays of hs_problem (kv_lens, doc_start, doc_end) by value into kernel
 * arguments before returning.
 * Paged KV (serving-style decode; the blog page on the unified sparse-attention
 * dispatcher, the paragraph on batched and paged serving; page "Support attn
 * sink in fa3", the KV-cache decode review): when page_table is set, kv is a
 * pool of pages [n_pages, block_size, Dk] and key block j of entry b (its rows
 * block_size*j .. +block_size-1) is page page_table[b * max_pages + j]. One
 * page holds exactly one key block. Block ids, top-k indices and masks stay
 * logical. Paged KV needs HS_BF16, no documents, and
 * L_b <= max_pages * block_size for every entry (checked); the page ids must
 * lie in the pool (device data, not checked).
 * Device-resident lengths (bf16, in-place or paged KV, no documents): with
 * kv_lens_device set, L_b is read from device memory when the kernels run,
 * so one recorded launch (for instance a captured HIP graph) serves changing
 * cache lengths. The host then plans with the capacity seqlen_kv (the row
 * stride of an in-place kv; <= max_pages * block_size when paged, checked):
 * hs_num_blocks and hs_workspace_size use it, block_logit has
 * ceil(seqlen_kv / block_size) columns (-inf past each entry's blocks), and
 * seqlen_q <= L_b <= seqlen_kv must hold (device data, not checked).
 * Device-resident document bounds (bf16 forward calls; same pages, packed
 * prefill replayed from a recorded launch): with doc_bounds_device set, the
 * packing is read from device memory when the kernels run, as cumulative
 * starts cu[0..n_docs] (document d is rows [cu[d], cu[d+1])), and n_docs is
 * the capacity: a packing of fewer documents pads cu with empty documents
 * (equal consecutive bounds; anywhere). cu[0] = 0, cu[n_docs] = seqlen_q and
 * cu non-decreasing must hold (device data, not checked; kernels clamp every
 * bound into [0, seqlen_q], so a bad table gives wrong results, not stray
 * reads). The host plans with the capacity: hs_num_blocks returns
 * ceil(seqlen / block_size) + n_docs - 1, the most blocks any such packing
 * has; block ids are numbered in document order and block_logit columns past
 * the packing's last block are -inf. Needs B == 1, seqlen_q == seqlen_kv, no
 * kv_lens, kv_lens_device or page_table, and doc_start/doc_end NULL. Such
 * launches never split the key range. The gradient calls reject it.
 * Streams: `stream` is a hipStream_t passed as void* (NULL = default stream).
 * Calls enqueue work and return without synchronising; a fault inside a
 * kernel surfaces at the caller's next synchronisation.
 * Errors: every check runs on the host before any launch; on failure nothing
 * is launched, the status is returned and hs_last_error() holds a message
 * (thread-local). Unsupported inputs are rejected, never silently ignored or
 * routed to another implementation (page "Support attn sink in fa3": a path
 * that cannot honour the sink must reject rather than drop it).
 * Reentrancy: stateless apart from the thread-local error string.
 */
#ifndef HS_H_
#define HS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HS_OK = 0,
  HS_ERR_INVALID_ARG = -1,   /* NULL pointer, bad size, inconsistent documents */
  HS_ERR_UNSUPPORTED = -2,   /* valid but not an instantiation built here      */
  HS_ERR_HIP = -3,           /* the HIP runtime reported an error at launch    */
  HS_ERR_WORKSPACE = -4      /* workspace missing or smaller than required     */
} hs_status;

typedef enum { HS_BF16 = 0, HS_F32 = 1 } hs_dtype;

typedef enum {
  HS_OP_BLOCK_SCORE = 0,
  HS_OP_SPARSE_GATHER = 1,
  HS_OP_SWA = 2,
  HS_OP_BLOCK_SCORE_BWD = 3,    /* workspace of hs_block_score_bwd   */
  HS_OP_SPARSE_GATHER_BWD = 4,  /* workspace of hs_sparse_gather_bwd */
  HS_OP_SWA_BWD = 5,            /* workspace of hs_swa_bwd           */
  HS_OP_BLOCK_SCORE_BWD_STORE_DS = 6, /* larger workspace of hs_block_score_bwd
                                         that also holds the score gradients */
  HS_OP_SWA_BWD_STORE_DS = 7,   /* the same for hs_swa_bwd           */
  HS_OP_SWA_SPARSE = 8,         /* workspace of hs_swa_sparse_fwd    */
  HS_OP_SPARSE_GATHER_BWD_STORE_DS = 9 /* the same for hs_sparse_gather_bwd */
} hs_op;

typedef struct {
  int32_t batch;          /* B                                                   */
  int32_t seqlen_q;       /* Sq: query rows per batch entry                     */
  int32_t seqlen_kv;      /* Skv: KV row stride per batch entry                 */
  int32_t num_heads;      /* H: query heads sharing the one KV head             */
  int32_t head_dim_qk;    /* Dk                                                 */
  int32_t head_dim_v;     /* Dv <= Dk: value = leading Dv columns of kv         */
  int32_t block_size;     /* key-block size (64)                                */
  float scale;            /* softmax scale; <= 0 selects 1/sqrt(Dk)             */
  int32_t dtype;          /* hs_dtype of q, kv and out                          */
  const int32_t* kv_lens; /* HOST [B] valid KV length per entry, or NULL (=Skv) */
  int32_t n_kv_lens;      /* must equal B when kv_lens is set (B <= 256)        */
  const int32_t* doc_start; /* HOST [n_docs] packed documents, or NULL          */
  const int32_t* doc_end;   /* HOST [n_docs]                                     */
  int32_t n_docs;         /* 0, or 1..64 with B == 1 and kv_lens == NULL (with  */
                          /* doc_bounds_device: the capacity)                   */
  const int32_t* page_table; /* DEVICE [B, max_pages] int32, or NULL: paged KV  */
  int32_t max_pages;      /* pages per entry in page_table (paged KV only)      */
  const int32_t* kv_lens_device; /* DEVICE [B] int32 valid KV lengths, read at  */
                          /* run time (bf16; kv_lens must be NULL)              */
  const int32_t* doc_bounds_device; /* DEVICE [n_docs + 1] int32 cumulative    */
                          /* document starts, read at run time (bf16 forward;  */
                          /* n_docs = capacity; doc_start/doc_end NULL)         */
} hs_problem;

/* Number of key blocks NB = columns of block_logit: the largest, over the
 * batch, of sum over documents of ceil(L_d / block_size) (with
 * doc_bounds_device, the capacity ceil(seqlen / block_size) + n_docs - 1).
 * Returns NB >= 1, or a negative hs_status if the problem is invalid. */
int32_t hs_num_blocks(const hs_problem* p);

/* Workspace bytes the given operation needs for this problem (0 when it
 * needs none; single-token decode splits the key range across workgroups and
 * merges partial results through the workspace; the gradient operations
 * always need one; HS_OP_BLOCK_SCORE_BWD_STORE_DS, HS_OP_SWA_BWD_STORE_DS and
 * HS_OP_SPARSE_GATHER_BWD_STORE_DS give the larger causal, window and gather
 * gradient workspaces that also hold the score gradients). top_k and window
 * are the values the operation will be called with (ignored where
 * irrelevant). */
hs_status hs_workspace_size(const hs_problem* p, int32_t op, int32_t top_k, int32_t window,
                            size_t* bytes);

/* Fused causal attention and block scores (page "HySparse MQA sparse
 * attention ...", section "Core", first bullet; per-file table row for
 * block_score_fa4.py: causal attention fused with a scaled block_logit).
 *   out[b,r,h,:] = attention of q[b,r,h] over the allowed keys, with sink;
 *   lse[b,r,h]   = natural-log normaliser, sink included;
 *   block_logit[b,r,j] = max over heads h of ln sum over the allowed keys i
 *                  of block j of exp(scale * q[b,r,h] . kv[b,i]); the sink is
 *                  never part of it; -inf where block j has no allowed key
 *                  (blocks of other documents, past the causal limit, or
 *                  beyond this entry's block count). Every column is written.
 * q, kv, out: dtype; sink may be NULL; ws/ws_bytes per hs_workspace_size. */
hs_status hs_block_score_fwd(const hs_problem* p, const void* q, const void* kv,
                             const float* sink, void* out, float* lse, float* block_logit,
                             void* ws, size_t ws_bytes, void* stream);

/* Per-token top-k block selection (same page, per-file table row for
 * pipeline.py: top-k block selection on the block scores before the gather).
 * For each row, C = {j : block_logit[j] > -inf}. If |C| <= top_k all of C is
 * kept; otherwise the row's own block (the block holding its position) plus
 * the top_k-1 best other blocks of C ordered by (score descending, index
 * ascending). Indices are written ascending, padded with -1 to top_k entries.
 * Comparisons are exact on the float32 inputs. 1 <= top_k <= 64. */
hs_status hs_topk_blocks(const hs_problem* p, const float* block_logit, int32_t top_k,
                         int32_t* block_idx, void* stream);

/* Block scores and the per-token top-k in one call: writes exactly what
 * hs_block_score_fwd followed by hs_topk_blocks writes (out, lse, block_logit
 * and block_idx [B, Sq, top_k] int32, 4-byte aligned). The selection is fused
 * into the attention launch sequence, as the page "TileLang CSA compressed
 * indexer for DSv4" (description, item 2) fuses its indexer's top-k into the
 * forward: when decode splits the key range, the top-k runs inside the launch
 * that merges the partial results, once every block score of the row is
 * final, so the call costs no separate launch; otherwise the top-k kernel
 * follows the attention kernel on the stream. 1 <= top_k <= 64, at most 4096
 * blocks; ws/ws_bytes as for hs_block_score_fwd.
 * block_prob (optional, NULL = not written) [B, Sq, NB] float32, 4-byte
 * aligned: the normalised block scores (same page, per-file row for
 * pipeline.py: the probabilities are recovered as exp(block_logit - lse)).
 * With one lse per head, the row's normaliser is its largest per-head lse:
 *   block_prob[b,r,j] = exp(block_logit[b,r,j] - max_h lse[b,r,h]),
 * 0 where block_logit is -inf. Every value lies in [0, 1]; with one head the
 * row sums to the mass the attention puts on keys (1 - exp(sink - lse)). */
hs_status hs_block_score_topk_fwd(const hs_problem* p, const void* q, const void* kv,
                                  const float* sink, int32_t top_k, void* out, float* lse,
                                  float* block_logit, int32_t* block_idx, float* block_prob,
                                  void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * outputs as hs_block_score_topk_fwd, but the partial results of a split key
 * range (single-token decode) live in a library-owned device array of 64 MiB
 * per GPU instead of a caller workspace, and the call allocates nothing.
 * The split is planned to fit that array (rows then take fewer, longer
 * chunks), so results agree with hs_block_score_topk_fwd up to the rounding
 * of the partial merge; HS_ERR_UNSUPPORTED if the partials could not fit.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (each call writes every partial it later reads, so nothing needs
 * clearing): calls that overlap on one GPU (concurrent streams) race. */
hs_status hs_block_score_topk_fwd_noalloc(const hs_problem* p, const void* q, const void* kv,
                                          const float* sink, int32_t top_k, void* out, float* lse,
                                          float* block_logit, int32_t* block_idx,
                                          float* block_prob, void* stream);

/* Block-sparse gather attention (same page, "Core", block-sparse DSA gather
 * bullet; per-file table row for block_sparse_mqa_dsa.py): attention with
 * sink over the union of the listed blocks intersected with the allowed keys.
 * Entries < 0 or >= the entry's block count are skipped; the entries of a row
 * must be distinct (not checked: device data). */
hs_status hs_sparse_gather_fwd(const hs_problem* p, const void* q, const void* kv,
                               const float* sink, const int32_t* block_idx, int32_t top_k,
                               void* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Sliding-window MQA attention (same page, "Core", SWA bullet; per-file table
 * rows for swa_attn.py and windowed_mqa_attn*.py): attention with sink over
 * the allowed keys i with i >= p - window + 1 (window keys including the
 * token itself). window >= 1. */
hs_status hs_swa_fwd(const hs_problem* p, const void* q, const void* kv, const float* sink,
                     int32_t window, void* out, float* lse, void* ws, size_t ws_bytes,
                     void* stream);

/* Both attention branches of a sliding-window layer that reuses a full
 * layer's shared latent KV and block selection (same page, Changes list: the
 * full layer emits the shared KV and block indices, and the window kernel
 * serves the sliding-window layer's main branch; per-file table row for
 * transformer_layer.py: KV shared across layers). One call returns the two
 * branch outputs separately, exactly as hs_swa_fwd (out_swa, lse_swa) and
 * hs_sparse_gather_fwd (out_sparse, lse_sparse) would for the same
 * arguments. On the bf16 path with an in-place cache, whenever neither
 * branch splits its key range across workgroups (few rows with long ranges
 * do, e.g. single-token decode or a short chunk over a long cache), one
 * launch walks each row's window blocks and then its selected blocks,
 * loading the row's queries once; otherwise the two operations run one after
 * the other. top_k < 1 and window < 1 are HS_ERR_INVALID_ARG, top_k > 64 is
 * HS_ERR_UNSUPPORTED (as for hs_sparse_gather_fwd). Workspace:
 * hs_workspace_size with HS_OP_SWA_SPARSE.
 * Branch combination (optional; all three pointers or none): the pages do
 * not state how a layer combines its branches; the method is NSA-style
 * (same page, section "What"), and NSA combines its branches by a gated sum
 * with gates the model computes per token and head. With gate_swa and
 * gate_sparse ([B, Sq, H] float32, 4-byte aligned) the call also writes
 *   out_mix[b,r,h,:] = gate_swa[b,r,h] * out_swa[b,r,h,:]
 *                    + gate_sparse[b,r,h] * out_sparse[b,r,h,:]
 * ([B, Sq, H, Dv], dtype, 16-byte aligned), formed in float32 from the two
 * stored outputs and rounded to dtype; the one-pass launch forms it in its
 * epilogue, otherwise a small elementwise launch follows (same values). */
hs_status hs_swa_sparse_fwd(const hs_problem* p, const void* q, const void* kv, const float* sink,
                            int32_t window, const int32_t* block_idx, int32_t top_k, void* out_swa,
                            float* lse_swa, void* out_sparse, float* lse_sparse,
                            const float* gate_swa, const float* gate_sparse, void* out_mix,
                            void* ws, size_t ws_bytes, void* stream);

/* Gradients (page "HySparse MQA sparse attention ...", section "Core": block
 * scoring trained through its autograd layer and the analytic gradient of
 * the learnable per-head sink; per-file table rows for windowed_mqa_attn*.py
 * and block_sparse_mqa_dsa.py, forward and backward kernels). For the loss
 * L = sum(dout * out) of the forward output out:
 *   dq  [B, Sq, H, Dk]  float32 = dL/dq;
 *   dkv [B, Skv, Dk]    float32 = dL/dkv, the key and value gradients added
 *                       (the latent row is both); rows past an entry's valid
 *                       length are zero; every row is written;
 *   dsink [H] float32   = dL/dsink = -sum over rows of exp(sink - lse) *
 *                       (dout . out); NULL skips it; needs a sink.
 * out and lse are the forward's outputs for the same inputs (out: dtype,
 * [B, Sq, H, Dv]; lse: [B, Sq, H]); dout has out's layout and dtype. dlse
 * (optional, NULL = zero) [B, Sq, H] float32 is an incoming gradient of lse,
 * for losses that use it (for instance a combination of branches weighted by
 * their log-sum-exp): the loss is then L = sum(dout * out) + sum(dlse * lse),
 * and since d lse / d s_i is the probability P_i, every formula above holds
 * with dout . out replaced by dout . out - dlse. The block scores take none
 * (review of PaddleFleet PR 1453, block-score PyLayer comments: the backward
 * returns gradients for q, k and v only). The workspace is mandatory:
 * hs_workspace_size with HS_OP_*_BWD and the same top_k / window, 16-byte
 * aligned. Results are deterministic (fixed summation order). Paged KV and
 * device-resident lengths are rejected (HS_ERR_UNSUPPORTED).
 * hs_block_score_bwd: the causal attention of hs_block_score_fwd. Given at
 * least the HS_OP_BLOCK_SCORE_BWD_STORE_DS workspace (bf16 only; 8 KB per
 * causal (row, key block) pair, 69 GB at one 32768-token sequence), the
 * key-block pass stores the bf16 score gradients dS (softmax scale included)
 * and dq is computed from them instead of recomputing the scores; with the
 * smaller HS_OP_BLOCK_SCORE_BWD workspace dq recomputes them. Both give the
 * same gradients up to the rounding of dS. */
hs_status hs_block_score_bwd(const hs_problem* p, const void* q, const void* kv, const float* sink,
                             const void* out, const float* lse, const void* dout,
                             const float* dlse, float* dq, float* dkv, float* dsink, void* ws,
                             size_t ws_bytes, void* stream);

/* Gradients of hs_sparse_gather_fwd for the given selection (block_idx and
 * top_k as in the forward; the selection itself takes no gradient). At most
 * 4096 blocks. Given at least the HS_OP_SPARSE_GATHER_BWD_STORE_DS workspace
 * (bf16 only; 8 KB per row and per selection entry, 8.6 GB at one
 * 32768-token sequence with top_k 32), the key-block pass stores the score
 * gradients of every (row, selected block) pair and dq is computed from them,
 * for two consecutive rows at a time over the union of their selections, as
 * for hs_block_score_bwd; with the smaller HS_OP_SPARSE_GATHER_BWD workspace
 * dq recomputes them. */
hs_status hs_sparse_gather_bwd(const hs_problem* p, const void* q, const void* kv,
                               const float* sink, const int32_t* block_idx, int32_t top_k,
                               const void* out, const float* lse, const void* dout,
                               const float* dlse, float* dq, float* dkv, float* dsink, void* ws,
                               size_t ws_bytes, void* stream);

/* Gradients of hs_swa_fwd (review of PaddleFleet PR 1453, the windowed
 * backward comments: a sequence length that is not a multiple of the tile
 * must read no row past its end; here every row index is bounded by Sq).
 * Given at least the HS_OP_SWA_BWD_STORE_DS workspace (bf16 only; 8 KB per
 * row and per block a window of that size can meet, ceil((window - 1) / 64)
 * + 1, at most the block count), dq is computed from the score gradients the
 * key-block pass stores, as for hs_block_score_bwd. */
hs_status hs_swa_bwd(const hs_problem* p, const void* q, const void* kv, const float* sink,
                     int32_t window, const void* out, const float* lse, const void* dout,
                     const float* dlse, float* dq, float* dkv, float* dsink, void* ws,
                     size_t ws_bytes, void* stream);

/* Static description of a status code. */
const char* hs_status_string(int32_t status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* hs_last_error(void);

/* ABI version of this library (major * 100 + minor). */
int32_t hs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HS_H_ */
