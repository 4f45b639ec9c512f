/*
 * flashcache.h -- C ABI of libflashcache.so: the Flash-Cache denoising step of
 * Flash-dLLM (arXiv 2609.26796) as hand-written HIP kernels for AMD CDNA4
 * (gfx950, MI355X).
 *
 * Method sources (web pages about Flash-dLLM):
 *   [FIG]    signal-papers page on arXiv 2609.26796, figure captions, Fig. 2:
 *            each step a fixed-size query of beta_m tokens (tracked positions +
 *            the current masked window) attends bidirectionally to the full KV
 *            cache through the fused kernel; tracked positions are the top-k
 *            decoded tokens by attention importance.
 *   [NEWS]   infernews post "Flash-dLLM 讓擴散式語言模型解碼更快、更省記憶體",
 *            paragraph 2: one fused kernel does the QKV projection, RoPE and the
 *            cache writes; block-scheduled attention serves different query
 *            lengths in one batch; only new tokens and a few positions chosen by
 *            attention importance are refreshed. Paragraph 3: Flash-Verify checks
 *            drafts and [MASK] tokens through two views and accepts together
 *            the predictions that meet a confidence threshold.
 *   [README] zhichai.net forum post quoting the project README, section 4:
 *            defaults block length 16, confidence threshold 0.9.
 *
 * Conventions for every entry point
 *   - Pointers are device pointers owned by the caller (for example torch
 *     tensors). The library keeps no pointer after the call returns, never
 *     frees caller memory, and allocates no device memory.
 *   - Work is enqueued on `stream` (NULL = the default stream) and the call
 *     returns without waiting; inputs must stay valid and unchanged until the
 *     stream has run the work. Faults inside a kernel show up at the caller's
 *     next synchronisation, as with any HIP launch.
 *   - Arguments are checked on the host before anything is enqueued; a failed
 *     check returns an error status and enqueues nothing. fc_last_error()
 *     gives a readable message for the calling thread's last failure.
 *   - Arrays are row-major and densely packed. Indices are int32.
 *   - Calls keep no state between them; calls on different streams with
 *     disjoint outputs may run concurrently.
 *   - dtype: FC_DTYPE_BF16 (bf16 storage, fp32 accumulation) or FC_DTYPE_F32.
 *   - Index inputs (positions, cu_seqlens_*, block_table) are trusted: the
 *     kernels index memory with them. With the environment variable FC_DEBUG
 *     set to a non-zero value, fc_qkv_rope_cache_write,
 *     fc_varlen_bidir_attention, fc_importance_topk, fv_verify_accept and
 *     fc_assemble_query first wait for the stream, copy these inputs to the
 *     host and check the preconditions each call can see (offsets start at 0
 *     and never decrease, totals match; positions >= 0 and distinct per
 *     sequence when the cache is written; every page a sequence uses has an
 *     entry >= 0 within max_pages_per_seq; Q_b <= max_seqlen_q), returning
 *     FC_ERR_INVALID_VALUE with a message before anything is enqueued.
 *     fc_validate_step_inputs checks all of them, page-id upper bounds
 *     included, on request.
 *
 * Notation: B sequences; sequence b has query length Q_b (its rows are packed
 * by cu_seqlens_q) and cache length L_b (cu_seqlens_k); H heads of size D;
 * d = H * D; T_q = sum Q_b, T_k = sum L_b. cu_seqlens_* are [B+1] exclusive
 * prefix sums starting at 0.
 *
 * Paged KV cache: k_cache and v_cache are [num_pages, H, page_size, D]. Cache
 * position p of sequence b lives in page block_table[b * max_pages_per_seq +
 * p / page_size] at offset p % page_size; its slot id is
 * page * page_size + offset.
 */
#ifndef FLASHCACHE_H
#define FLASHCACHE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* fc_stream_t;   /* a hipStream_t */

typedef enum {
  FC_OK = 0,
  FC_ERR_INVALID_VALUE = 1,   /* null pointer, negative or inconsistent size    */
  FC_ERR_UNSUPPORTED = 2,     /* valid request outside the built shapes/dtypes */
  FC_ERR_WORKSPACE = 3,       /* workspace missing or smaller than required     */
  FC_ERR_HIP = 4              /* a HIP runtime call failed (message has detail) */
} fc_status_t;

enum { FC_DTYPE_F32 = 0, FC_DTYPE_BF16 = 1 };

/* Static description of a status code. Never NULL. */
const char* fc_status_string(fc_status_t status);

/* Message for the calling thread's most recent failed call ("" if none).
 * Valid until the thread's next call into the library. Never NULL. */
const char* fc_last_error(void);

/* Library version string, e.g. "flashcache-gfx950 0.1". */
const char* fc_version(void);

/*
 * Fused QKV projection + RoPE + paged cache write ([NEWS] paragraph 2; the
 * query and its tokens: [FIG] Fig. 2).
 *
 * For every query token t (row t of hidden, sequence b, position positions[t]):
 *   [q k v] = hidden[t] . w_qkv^T            (fp32 accumulation)
 *   q, k   <- rotate-half RoPE at positions[t]: for e < D/2, the pair
 *             (x_e, x_{e+D/2}) turns by angle positions[t] * rope_base^(-2e/D):
 *             x_e' = x_e cos - x_{e+D/2} sin,  x_{e+D/2}' = x_{e+D/2} cos + x_e sin
 *   q_out[t]               = q (rounded to dtype)
 *   k_cache/v_cache at the slot of (b, positions[t]) = k / v (rounded to dtype)
 *   slot_mapping[t]        = that slot id
 *
 * hidden        [T_q, d]            dtype
 * positions     [T_q]               cache position of each token, 0 <= p < L_b;
 *                                   distinct within a sequence when the cache is
 *                                   written (two tokens on one slot would race)
 * cu_seqlens_q  [B+1]               token rows per sequence
 * T_q                               total query tokens (= cu_seqlens_q[B])
 * w_qkv         [3d, d]             dtype; rows are the Q, K, V blocks, each
 *                                   head-major (row h*D + e of a block); no bias
 * k_cache, v_cache                  dtype, written in place; both NULL for a
 *                                   projection that writes no cache (the verify
 *                                   pass, where two views share positions)
 * block_table   [B, max_pages_per_seq]   page ids (entries past the last page
 *                                   of a sequence are never read)
 * q_out         [T_q, H, D]         dtype
 * slot_mapping  [T_q] or NULL
 * row_scale     [T_q] fp32 or NULL: when set, token t's q, k and v are
 *               multiplied by row_scale[t] before RoPE, i.e. the projection of
 *               hidden[t] * row_scale[t] (an input normalisation computed by
 *               fc_rms_row_scale)
 * workspace     device memory of at least fc_qkv_workspace_size() bytes (the
 *               per-token rotation table and cache slots, and for bf16 calls
 *               with few row tiles the fp32 partial products of a K-split
 *               projection; overwritten; NULL allowed when that size is 0;
 *               calls that overlap on one workspace race)
 * Supported: bf16 with D = 128 and d a multiple of 256 (other head sizes:
 * FC_ERR_UNSUPPORTED; every bf16 workload here has D = 128, and the bf16
 * kernels give a wave whole 128-wide heads); f32 with D in {64,128}.
 * page_size must be a power of two in [1, 256]. bf16: hidden, w_qkv, q_out,
 * k_cache, v_cache and workspace must be 16-byte aligned (FC_ERR_INVALID_VALUE
 * otherwise).
 */
fc_status_t fc_qkv_rope_cache_write(
    const void* hidden, const int32_t* positions, const int32_t* cu_seqlens_q, int32_t B,
    int32_t T_q, const void* w_qkv, int32_t d_model, int32_t n_heads, int32_t head_dim,
    float rope_base, void* k_cache, void* v_cache, const int32_t* block_table,
    int32_t max_pages_per_seq, int32_t page_size, void* q_out, int32_t* slot_mapping,
    const float* row_scale, void* workspace, size_t workspace_bytes, int32_t dtype,
    fc_stream_t stream);

/* Bytes of device workspace fc_qkv_rope_cache_write needs (0 when none). The
 * K-split decision depends on the compute-unit count of the device current at
 * the time of the query (counted per device), so query it with the device
 * current that the call will run on. */
size_t fc_qkv_workspace_size(int32_t T_q, int32_t d_model, int32_t head_dim, int32_t dtype);

/* Bytes of device workspace fc_varlen_bidir_attention needs for these sizes
 * (0 when none). max_seqlen_q: the largest query length of any sequence in the
 * calls the workspace serves (with importance, sequences of more than 128 query
 * rows need (ceil(max_seqlen_q / 128) - 1) * n_heads * T_k floats more). A
 * workspace sized for the largest B, T_k and max_seqlen_q serves smaller calls. */
size_t fc_attention_workspace_size(int32_t B, int32_t T_q, int32_t T_k, int32_t n_heads,
                                   int32_t head_dim, int32_t with_importance,
                                   int32_t max_seqlen_q);

/*
 * Bidirectional varlen attention over each sequence's whole paged cache, with
 * the per-key attention importance fused in ([FIG] Fig. 2: no causal mask,
 * every cached key; [NEWS] paragraph 2: block-scheduled attention across
 * sequences of different query lengths, importance picks refreshed positions).
 *
 * For sequence b, head h and query row i of b:
 *   s_ij = softmax_scale * <q[i, h], k_j>      over all keys j < L_b of b
 *   P_ij = exp(s_ij - max_j s_ij) / sum_j exp(s_ij - max_j s_ij)
 *   out[i, h] = sum_j P_ij v_j
 * and, when importance != NULL, for every key j of b:
 *   importance[h, cu_seqlens_k[b] + j]  (=, or += when accumulate) sum_i P_ij
 * The importance path computes exact normalised P in two passes over the keys
 * (row max and normaliser first), so it reads K twice. With importance == NULL
 * a single online-softmax pass is used.
 *
 * q             [T_q, H, D]  dtype (post-RoPE queries)
 * k_cache, v_cache, block_table, page_size   the paged cache (see above)
 * max_seqlen_q                max Q_b (sizes the grid; rows beyond Q_b idle)
 * out           [T_q, H, D]  dtype
 * importance    [H, T_k] fp32 or NULL
 * workspace     device memory of at least fc_attention_workspace_size() bytes
 *               (scratch for the longest-first sequence order, the key split's
 *               partials and the column sums of row tiles past the first;
 *               contents need no initialisation and are overwritten; calls that
 *               overlap on one workspace race)
 * A sequence with L_b = 0 gets out = 0. Supported: bf16 with D = 128; f32 with
 * D in {64, 128}.
 */
fc_status_t fc_varlen_bidir_attention(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
    int32_t max_pages_per_seq, int32_t page_size, const int32_t* cu_seqlens_q,
    const int32_t* cu_seqlens_k, int32_t B, int32_t max_seqlen_q, int32_t T_k, int32_t n_heads,
    int32_t head_dim, float softmax_scale, void* out, float* importance, int32_t accumulate,
    void* workspace, size_t workspace_bytes, int32_t dtype, fc_stream_t stream);

/*
 * fc_varlen_bidir_attention without a workspace argument, for callers that
 * cannot allocate device memory (code under stream capture, tight serving
 * loops, harnesses that forbid hipMalloc). The arguments and results are
 * those of fc_varlen_bidir_attention; the workspace is instead a static
 * device array of FC_ATTN_NOALLOC_SCRATCH_BYTES inside the library, one per
 * device, held until the process ends. The call allocates nothing.
 * Sizes whose fc_attention_workspace_size exceeds that array are rejected
 * with FC_ERR_WORKSPACE before anything is enqueued. Every call on one device
 * shares that device's array: calls that may overlap in time on one device
 * (different streams, host threads) race and must be serialised by the
 * caller. The array needs no clearing between calls.
 */
#define FC_ATTN_NOALLOC_SCRATCH_BYTES ((size_t)24 << 20)
fc_status_t fc_varlen_bidir_attention_noalloc(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
    int32_t max_pages_per_seq, int32_t page_size, const int32_t* cu_seqlens_q,
    const int32_t* cu_seqlens_k, int32_t B, int32_t max_seqlen_q, int32_t T_k, int32_t n_heads,
    int32_t head_dim, float softmax_scale, void* out, float* importance, int32_t accumulate,
    int32_t dtype, fc_stream_t stream);

/*
 * Top-k reselection of the tracked positions ([FIG] Fig. 2: tracked positions
 * are the top-k decoded tokens by attention importance).
 *
 * score_j = sum over h = 0..H-1, in that order, of importance[h, j] (fp32).
 * For each sequence b, among its candidate positions (candidate_mask != 0, or
 * all positions when candidate_mask is NULL) keep min(k, #candidates) of them:
 * larger score first, equal scores -> lower position.
 *
 * importance      [H, T_k] fp32
 * candidate_mask  [T_k] uint8 or NULL
 * topk_pos        [B, k] chosen positions (within the sequence) in ascending
 *                 order, -1 after the last one
 * topk_count      [B] number chosen: min(k, candidates of the sequence)
 * topk_score      [B, k] fp32 scores in the same order (NaN padded) or NULL
 * Sequences of up to FC_TOPK_MAX_LEN keys keep their scores in LDS; longer ones
 * are served too, recomputing the head sums from `importance` in each of the
 * selection's passes (the same sums, several times the reads).
 */
#define FC_TOPK_MAX_LEN 16384
fc_status_t fc_importance_topk(
    const float* importance, const int32_t* cu_seqlens_k, int32_t B, int32_t T_k,
    int32_t n_heads, const uint8_t* candidate_mask, int32_t k, int32_t* topk_pos,
    int32_t* topk_count, float* topk_score, fc_stream_t stream);

/*
 * Flash-Verify accept test over the draft and [MASK] views ([NEWS] paragraph 3;
 * threshold default 0.9 from [README] section 4).
 *
 * Rows: sequence b owns n_b = cu_positions[b+1] - cu_positions[b] verified
 * positions and 2 n_b logit rows starting at row 2*cu_positions[b]: first the
 * n_b draft-view rows, then the n_b mask-view rows, both in position order.
 * For row r of verified position p:
 *   argmax[r]     = lowest token id among the row's maxima
 *   conf[r]       = 1 / sum_v exp(logits[r, v] - logits[r, argmax[r]])
 *                   (the largest softmax probability), fp32
 *   accept_row[r] = argmax[r] == draft_tokens[p]  and  conf[r] >= tau
 *   accept_pos[p] = accept_row[draft-view row] and accept_row[mask-view row]
 *
 * logits        [R, vocab] bf16, R = 2 * cu_positions[B]
 * cu_positions  [B+1]
 * draft_tokens  [cu_positions[B]] int32
 * tau           confidence threshold in (0, 1], compared as fp32, inclusive
 * argmax [R] int32, conf [R] fp32, accept_row [R] uint8; accept_pos
 * [cu_positions[B]] uint8 or NULL.
 */
fc_status_t fv_verify_accept(
    const void* logits, int32_t vocab, const int32_t* cu_positions, int32_t B, int32_t R,
    const int32_t* draft_tokens, float tau, int32_t* argmax, float* conf, uint8_t* accept_row,
    uint8_t* accept_pos, fc_stream_t stream);

/*
 * The LM head with the Flash-Verify accept test fused in ([NEWS] paragraph 3:
 * predictions of the two views meeting the confidence threshold are
 * accepted; the predictions come from the model's logits over the
 * vocabulary). For every row r of hidden:
 *   logit[r, v] = hidden[r] . w_lm[v]              (fp32 accumulation, never stored)
 *   argmax[r]   = lowest v among the row's maxima
 *   conf[r]     = 1 / sum_v exp(logit[r, v] - logit[r, argmax[r]])
 * then accept_row / accept_pos exactly as fv_verify_accept (rows of sequence
 * b: its draft-view rows, then its mask-view rows).
 * hidden [R, d_model] bf16, w_lm [vocab, d_model] bf16 (16-byte aligned);
 * workspace of at least fv_lmhead_workspace_size(R, vocab) bytes (per-row
 * partial maxima and sums; overwritten). Supported: vocab % 256 == 0,
 * d_model % 64 == 0, vocab * d_model < 2^30.
 */
size_t fv_lmhead_workspace_size(int32_t R, int32_t vocab);
fc_status_t fv_lmhead_verify_accept(const void* hidden, const void* w_lm, int32_t d_model,
                                    int32_t vocab, const int32_t* cu_positions, int32_t B,
                                    int32_t R, const int32_t* draft_tokens, float tau,
                                    void* workspace, size_t workspace_bytes, int32_t* argmax,
                                    float* conf, uint8_t* accept_row, uint8_t* accept_pos,
                                    fc_stream_t stream);

/*
 * Confidence-aware acceptance: threshold unmasking without drafts, the
 * decoding that Flash-Verify is compared with ([README] section 1: the
 * confidence-aware Flash-Cache configuration; [FIG] Fig. 6: tokens per
 * iteration against confidence-aware decoding).
 *
 * One logit row per masked position; sequence b owns rows cu_positions[b] ..
 * cu_positions[b+1]-1. For row r:
 *   argmax[r] = lowest token id among the row's maxima
 *   conf[r]   = 1 / sum_v exp(logits[r, v] - logits[r, argmax[r]])   (fp32)
 *   accept[r] = conf[r] >= tau   (fp32, inclusive)
 * With at_least_one != 0, a sequence none of whose rows passed accepts its
 * row of largest conf (equal conf: the lower row; NaN conf, from non-finite
 * logits, never counts as largest, and a sequence whose rows are all NaN
 * accepts its first row), so each step unmasks at least one token per
 * sequence.
 * logits [R, vocab] bf16, R = cu_positions[B]; argmax [R] int32, conf [R]
 * fp32, accept [R] uint8.
 */
fc_status_t fv_confidence_accept(const void* logits, int32_t vocab, const int32_t* cu_positions,
                                 int32_t B, int32_t R, float tau, int32_t at_least_one,
                                 int32_t* argmax, float* conf, uint8_t* accept,
                                 fc_stream_t stream);

/*
 * Flash-Verify's two views with view-private K/V ([NEWS] paragraph 3: drafts
 * and [MASK] tokens are verified through two views of the same positions; the
 * fugumt abstract page: KV-cache-driven draft-and-verify).
 *
 * Sequence b (cache length L_b = cu_seqlens_k[b+1] - cu_seqlens_k[b]) verifies
 * positions verify_start[b] .. L_b - 1. Each view v (0 = draft, 1 = [MASK])
 * attends with its own fresh K/V at those positions and the shared cache at
 * every earlier one. fv_fork_view_pages makes that a paged cache of its own:
 * virtual sequence 2b + v gets row 2b + v of view_block_table
 * [2B, max_pages_per_seq], equal to row b of block_table for the pages before
 * the one holding verify_start[b], then private page ids
 * view_page_base + (2b + v) * pages_per_view + i (i = 0, 1, ...) up to the last
 * page of the sequence, then -1. The private pages are pages of k_cache and
 * v_cache themselves (the caller reserves 2 B pages_per_view of them from
 * view_page_base on); the shared positions of the first private page are
 * copied into it. Then:
 *   - fc_qkv_rope_cache_write over the 2B virtual sequences (rows of sequence
 *     b: its draft-view rows, then its [MASK]-view rows, at positions
 *     verify_start[b] + i; block_table = view_block_table) writes each view's
 *     fresh K/V into its private pages;
 *   - fc_varlen_bidir_attention (no importance) over the 2B virtual sequences
 *     (cu_seqlens_k repeating L_b for both views) attends each view to its own
 *     cache;
 *   - fv_commit_accepted copies, for every position p of cu_positions with
 *     accept_pos[p] != 0, the draft view's K and V rows (all heads) into the
 *     sequence's shared slot; other slots keep their bytes.
 * Preconditions (checked under FC_DEBUG): 0 <= verify_start[b] <= L_b, the
 * sequence's pages from the one holding verify_start[b] to its last number at
 * most pages_per_view, the reserved pages exist. bf16, head_dim 128; k_cache
 * and v_cache 16-byte aligned. cu_positions [B+1] counts L_b - verify_start[b]
 * per sequence; n_positions = cu_positions[B].
 */
fc_status_t fv_fork_view_pages(void* k_cache, void* v_cache, const int32_t* block_table,
                               int32_t max_pages_per_seq, int32_t page_size,
                               const int32_t* cu_seqlens_k, const int32_t* verify_start,
                               int32_t B, int32_t n_heads, int32_t head_dim,
                               int32_t view_page_base, int32_t pages_per_view,
                               int32_t* view_block_table, fc_stream_t stream);
fc_status_t fv_commit_accepted(void* k_cache, void* v_cache, const int32_t* block_table,
                               const int32_t* view_block_table, int32_t max_pages_per_seq,
                               int32_t page_size, const int32_t* cu_positions,
                               const int32_t* verify_start, int32_t B, int32_t n_positions,
                               const uint8_t* accept_pos, int32_t n_heads, int32_t head_dim,
                               fc_stream_t stream);

/*
 * Per-row RMS normalisation factor for a layer's input in the layer stack:
 * scale[m] = 1 / sqrt(mean_n x[m, n]^2 + eps) (fp32 accumulation, no learned
 * weight). Feeds row_scale of fc_qkv_rope_cache_write. Not part of the pages'
 * single-step description: a stack of residual layers with random weights needs
 * it to keep the hidden state bounded, as pre-normalised transformer layers do.
 * x [M, N] dtype, scale [M] fp32.
 */
fc_status_t fc_rms_row_scale(const void* x, int32_t M, int32_t N, float eps, float* scale,
                             int32_t dtype, fc_stream_t stream);

/*
 * Output projection with residual for the layer stack: h_inout += x . w^T
 * (fp32 accumulation, one rounding to dtype).
 * x [M, K], w [N, K], h_inout [M, N], all dtype. Supported: bf16 with N a
 * multiple of 128 and K a multiple of 64; f32 any size.
 */
fc_status_t fc_linear_residual(const void* x, const void* w, void* h_inout, int32_t M,
                               int32_t N, int32_t K, int32_t dtype, fc_stream_t stream);

/*
 * Query assembly for the next denoising step ([FIG] Fig. 2: the query is the
 * tracked positions plus the current masked window).
 * For sequence b, rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of positions get
 * the first topk_count[b] entries of topk_pos[b] followed by window_start[b],
 * window_start[b]+1, ... (up to the sequence's query length). topk_pos/count
 * may be NULL (window only). topk_pos is [B, k].
 */
fc_status_t fc_assemble_query(const int32_t* topk_pos, const int32_t* topk_count, int32_t k,
                              const int32_t* window_start, const int32_t* cu_seqlens_q,
                              int32_t B, int32_t* positions, fc_stream_t stream);

/*
 * Debug check of a step's index inputs (the preconditions of
 * fc_qkv_rope_cache_write and fc_varlen_bidir_attention): cu_seqlens_q and
 * cu_seqlens_k start at 0, never decrease and end at T_q and T_k; sequence b
 * uses pages 0 .. ceil(L_b / page_size) - 1 of its block-table row, at most
 * max_pages_per_seq of them, each entry in [0, num_pages); when positions is
 * not NULL, the rows of sequence b hold distinct positions in [0, L_b).
 * Waits for the stream and reads the inputs back to the host; returns FC_OK,
 * or FC_ERR_INVALID_VALUE with a message naming the first violation. All
 * pointers are device memory; positions [T_q] may be NULL.
 */
fc_status_t fc_validate_step_inputs(const int32_t* positions, const int32_t* cu_seqlens_q,
                                    const int32_t* cu_seqlens_k, int32_t B, int32_t T_q,
                                    int32_t T_k, const int32_t* block_table,
                                    int32_t max_pages_per_seq, int32_t page_size,
                                    int32_t num_pages, fc_stream_t stream);

/*
 * Measurement probes (diagnostics for benchmarks; not part of the step).
 *
 * fc_probe_kv_stream: streams the paged bf16 cache of B sequences with the
 * attention kernel's own access pattern (one workgroup per (sequence, head),
 * 64-key tiles through registers into LDS, nontemporal loads) and computes
 * nothing. k_passes = 1 reads K and V once; k_passes = 2 reads K, then K and V
 * (the two passes of the importance path). The elapsed time is the floor of
 * that pattern's memory traffic on the device. k_policy is the cache policy of
 * the K-only pass when k_passes = 2 (0 nontemporal, as the attention kernel;
 * 1 default; 2 sc1; 3 sc0; pages of 16 keys or more for 1..3, else
 * FC_ERR_UNSUPPORTED); with k_passes = 1 it must be 0. The K and V pass is
 * always nontemporal. head_dim must be 128. sink [B * n_heads] fp32 is a dummy
 * output (left unchanged in practice).
 *
 * fc_probe_mfma_bf16: n_blocks workgroups of 4 waves, each wave running
 * iters x 8 independent v_mfma_f32_32x32x16_bf16 (32768 flops each) on
 * register operands: the sustained dense bf16 matrix rate, in flops
 * n_blocks * 4 * iters * 8 * 32768 over the elapsed time. sink [n_blocks].
 */
fc_status_t fc_probe_kv_stream(const void* k_cache, const void* v_cache,
                               const int32_t* block_table, int32_t max_pages_per_seq,
                               int32_t page_size, const int32_t* cu_seqlens_k, int32_t B,
                               int32_t n_heads, int32_t head_dim, int32_t k_passes,
                               int32_t k_policy, float* sink, fc_stream_t stream);
fc_status_t fc_probe_mfma_bf16(int32_t n_blocks, int32_t iters, float* sink, fc_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FLASHCACHE_H */
