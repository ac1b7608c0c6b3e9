/*
 * qsa.h - C ABI of the MI355X (gfx950) Qwen Sparse Attention (QSA) library.
 *
 * QSA compresses the key cache into small blocks, scores those compressed
 * blocks against each query, keeps the best contiguous token blocks and runs
 * exact softmax attention over only those blocks
 * ("Qwen4 architecture: QSA, GatedResidual, PLE", codebridge-ai.com,
 * section 1 "QSA: not looking at every token equally").
 * The split into a selector that returns cache addresses and an attention
 * step that reads only those addresses follows
 * "Qwen4 in llama.cpp: Dissecting PR #27742" (ramgpt.org), section
 * "QSA Is an Address-Selection Problem, Not a New Attention Equation".
 *
 * Notation: b = batch, Hq / Hkv = query / KV heads, G = Hq / Hkv, d = head
 * dim, Bs = block size, k = top_k, N = kv_len. Query head h reads KV head
 * h / G. A query at absolute position p has own block i = p / Bs.
 *
 * Semantics (the library's reading of the pages where they are silent):
 *   compressed key   kc[b][g][c] = mean of K[b][g][c*Bs .. c*Bs+Bs-1]
 *   score            s(c) = scale * sum_{j<G} <q_{g*G+j}, kc[c]>
 *   frame            which blocks compete and which one is always kept:
 *                    keep_tail = 0: candidates 0 .. i-1, block i always kept
 *                    keep_tail = 1 (the released budget of "Qwen4 in
 *                    llama.cpp: Dissecting PR #27742", section "QSA Is an
 *                    Address-Selection Problem...", whose visible width is
 *                    at most budget + ratio - 1): candidates are all
 *                    n = (p+1)/Bs complete blocks, the own block included
 *                    once complete; block n (the positions past the last
 *                    complete block) is always kept when (p+1) % Bs != 0
 *   selection        the kept block (if any) counts in k; the other
 *                    min(k-1, #candidates) slots take the best scores, equal
 *                    scores going to the smaller block id; written ascending
 *                    and padded with -1
 *   attention        softmax(scale * <q_h, K_t>) weighted sum of V_t over
 *                    the positions of the kept blocks that are <= p
 *   scale            1/sqrt(d) when qsa_shape.scale == 0
 *
 * Layouts (all contiguous, row-major, 16-byte aligned base pointers):
 *   Q, out    [b][q_len][Hq][d]            dtype of qsa_shape
 *   K, V      [b][Hkv][kv_cap][d]          dtype of qsa_shape
 *   k_comp    [b][Hkv][kv_cap / Bs][d]     float32
 *   sel       [b][q_len][Hkv][k]           int32
 *   sel_scores[b][q_len][Hkv][k]           float32 (optional)
 *
 * Ownership: the caller allocates and frees every buffer (device memory for
 * all tensors and the workspace; `shape` is host memory read during the
 * call). The library never allocates, frees, synchronises, or keeps a
 * pointer after returning (qsa_decode_step_noalloc alone uses device memory
 * of the library's own: a fixed array, see there). All work is enqueued on `stream` (a hipStream_t;
 * NULL = the null stream), in order; results are ready when the stream
 * reaches that point.
 *
 * Errors: every argument is validated on the host before any HIP call.
 *   QSA_ERR_INVALID      null required pointer, non-positive size, Hq not a
 *                        multiple of Hkv, kv_len > kv_cap, inconsistent
 *                        positions, misaligned pointer, unknown op/dtype,
 *                        keep_tail not 0/1, keep_tail with k < 2
 *   QSA_ERR_UNSUPPORTED  valid but not implemented: d not in {64,128},
 *                        Bs not a power of two in [4,128], k > 513,
 *                        G not in {1,2,4,8,16}; selection with k > 64 and
 *                        more than 65536 candidates per row; too many
 *                        blocks or rows for a launch
 *   QSA_ERR_WORKSPACE    ws_bytes below qsa_workspace_bytes(...) or ws NULL
 *                        while bytes are needed
 *   QSA_ERR_HIP          a kernel launch was rejected by the runtime
 * On error nothing is enqueued (QSA_ERR_HIP: launches before the failing
 * one may have been enqueued). Faults during execution surface at the
 * caller's next synchronisation. Kernels trust that sel holds valid ids for
 * the given positions and that inputs are finite.
 *
 * Determinism: identical inputs and shapes give bitwise identical outputs
 * (no floating-point atomics, fixed reduction orders).
 * Thread safety: calls may come from several host threads; calls that
 * share output or workspace buffers must be ordered by the caller.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_ABI_VERSION 12

enum { QSA_F32 = 0, QSA_BF16 = 1 };

enum {
  QSA_OP_COMPRESS = 0,
  QSA_OP_SELECT = 1,
  QSA_OP_DECODE = 2,
  QSA_OP_PREFILL = 3,
  QSA_OP_DECODE_STEP = 4,
  QSA_OP_DECODE_STEP_RAGGED = 5,
  QSA_OP_INDEXER_SELECT = 6,
  QSA_OP_PREFILL_Q8 = 7,
  QSA_OP_SELECT_RAGGED = 8
};

typedef enum {
  QSA_OK = 0,
  QSA_ERR_INVALID = 1,
  QSA_ERR_UNSUPPORTED = 2,
  QSA_ERR_WORKSPACE = 3,
  QSA_ERR_HIP = 4
} qsa_status;

typedef struct {
  int32_t batch;       /* sequences in the call */
  int32_t n_q_heads;   /* Hq */
  int32_t n_kv_heads;  /* Hkv; Hq % Hkv == 0 */
  int32_t head_dim;    /* d */
  int32_t block_size;  /* Bs: tokens per compressed block */
  int32_t top_k;       /* k: kept blocks per (token, KV head), always-kept block included */
  int32_t dtype;       /* QSA_F32 or QSA_BF16: type of Q, K, V and out */
  float scale;         /* softmax/score scale; 0 selects 1/sqrt(head_dim) */
  int32_t keep_tail;   /* selection frame: 0 = own block always kept, 1 = only the partial tail */
} qsa_shape;

/* Version of this ABI (QSA_ABI_VERSION). */
int qsa_abi_version(void);

/* Static, human-readable name of a status code. */
const char* qsa_status_str(qsa_status status);

/* Bytes of device workspace the given op needs for these sizes (0 if none;
 * (size_t)-1 if the arguments are invalid or the op does not serve the
 * shape: selection (default or indexer), and decode steps that select
 * separately, with k > 64 over more than 65536 candidates per row). op is one of QSA_OP_*.
 * QSA_OP_SELECT, QSA_OP_PREFILL, QSA_OP_INDEXER_SELECT and QSA_OP_PREFILL_Q8
 * (0: the call runs one row per workgroup) take q_len and
 * kv_len = q_pos0 + q_len;
 * QSA_OP_DECODE takes kv_len (q_len ignored).
 * QSA_OP_DECODE_STEP_RAGGED and QSA_OP_SELECT_RAGGED take the longest
 * sequence's length as kv_len (q_len ignored) and return (size_t)-1 for
 * shapes those calls do not serve.
 * Zero-fill a workspace once before its first use. Decode workspaces, and
 * selection workspaces whose rows are split over several workgroups, start
 * with one arrival counter per row ((sequence, KV head), resp. (sequence,
 * token, KV head): 4 bytes each, the area rounded up to 256 bytes); the last
 * workgroup of a row to finish does the row's final step and resets its
 * counter, so every call leaves that area at zero and the workspace can be
 * reused by any later call of the same op it is large enough for. Decode-step
 * workspaces (QSA_OP_DECODE_STEP, QSA_OP_DECODE_STEP_RAGGED) start with two
 * such areas at fixed offsets, which every path of the step leaves at zero,
 * so one workspace serves steps that take different paths. The rest is
 * scratch of one call. */
size_t qsa_workspace_bytes(const qsa_shape* shape, int op, int64_t q_len, int64_t kv_len);

/* Block compression ("Qwen4 architecture: QSA, GatedResidual, PLE", section 1:
 * keys are compressed into small blocks; the mean is this library's reading).
 * Writes k_comp rows for the complete blocks block_begin .. kv_len/Bs - 1 of
 * every (b, KV head); other rows are left untouched. block_begin = 0
 * compresses everything; a decode loop passes the first block not yet
 * compressed. k: device [b][Hkv][kv_cap][d]; k_comp: device float32
 * [b][Hkv][kv_cap/Bs][d]. Needs no workspace. When the range holds no
 * complete block the call does nothing and k, k_comp may be NULL. */
qsa_status qsa_compress_keys(const qsa_shape* shape, const void* k, int64_t kv_len, int64_t kv_cap,
                             int64_t block_begin, float* k_comp, void* stream);

/* Indexer scoring and top-k block selection ("Qwen4 in llama.cpp: Dissecting
 * PR #27742", section "QSA Is an Address-Selection Problem...": compressed
 * blocks are scored, the top-k kept and turned into cache addresses).
 * Query row t of q ([b][q_len][Hq][d]) sits at absolute position q_pos0 + t;
 * requires kv_len == q_pos0 + q_len (decode: q_len = 1, q_pos0 = kv_len-1).
 * k_comp must hold every candidate block of the rows' frames (the complete
 * blocks before the own block, or with keep_tail all complete blocks among
 * the first kv_len positions); it may be NULL when no row has a candidate.
 * Writes sel [b][q_len][Hkv][k] (block ids ascending, the always-kept block
 * last, padded with -1) and, if sel_scores is not NULL, the float32 score
 * of each kept block at the same index (+inf for the always-kept block, -inf
 * for padding). k <= 64 keeps the running top set in registers; k > 64 (up
 * to the released budget of 512 blocks plus the tail slot) writes every
 * candidate score to the workspace and radix-selects the cutoff per row.
 * ws: device scratch of qsa_workspace_bytes(shape, QSA_OP_SELECT, q_len, kv_len). */
qsa_status qsa_score_select(const qsa_shape* shape, const void* q, int64_t q_len, int64_t q_pos0,
                            const float* k_comp, int64_t kv_len, int64_t kv_cap, int32_t* sel,
                            float* sel_scores, void* ws, size_t ws_bytes, void* stream);

/* Sparse attention for one new token per sequence at position kv_len-1
 * ("Qwen4 in llama.cpp: Dissecting PR #27742", section "QSA Is an
 * Address-Selection Problem...": ordinary attention restricted to the
 * selected cells). q: [b][Hq][d]; k, v: [b][Hkv][kv_cap][d];
 * sel: [b][Hkv][k] from qsa_score_select; out: [b][Hq][d]. Blocks shorter
 * than 32 keys are gathered several to one 32-key MFMA step. When a row is
 * split over several workgroups, the last one to finish merges the slices
 * (see the workspace note of qsa_workspace_bytes: zero-filled before first use).
 * ws: device scratch of qsa_workspace_bytes(shape, QSA_OP_DECODE, 1, kv_len). */
qsa_status qsa_sparse_attn_decode(const qsa_shape* shape, const void* q, const void* k, const void* v,
                                  int64_t kv_len, int64_t kv_cap, const int32_t* sel, void* out,
                                  void* ws, size_t ws_bytes, void* stream);

/* Causal sparse attention for q_len query rows at positions q_pos0 .. q_pos0+q_len-1
 * (same passage as decode, every row with its own selection; causal inside
 * the own block). q, out: [b][q_len][Hq][d]; k, v: [b][Hkv][kv_cap][d]
 * holding at least q_pos0 + q_len positions; sel: [b][q_len][Hkv][k].
 * bf16: blocks of 32 keys or more with top_k <= 64 run as tiles of query
 * rows sharing staged K/V (the workspace holds a copy of V in the MFMA
 * operand order); shorter blocks and larger top_k (the released budget of
 * 512 blocks of 4 keys plus the tail) run one query row per workgroup, with
 * no workspace. float32 runs one query row per wave, no workspace.
 * ws: device scratch of qsa_workspace_bytes(shape, QSA_OP_PREFILL, q_len, q_pos0 + q_len). */
qsa_status qsa_sparse_attn_prefill(const qsa_shape* shape, const void* q, const void* k, const void* v,
                                   int64_t q_len, int64_t q_pos0, int64_t kv_cap, const int32_t* sel,
                                   void* out, void* ws, size_t ws_bytes, void* stream);

/* One whole decode step: the same results as qsa_compress_keys(shape, k,
 * kv_len, kv_cap, block_begin = (kv_len-1)/Bs, k_comp), then
 * qsa_score_select for the token at kv_len-1, then qsa_sparse_attn_decode
 * (the passages cited there). k_comp must already hold the blocks completed
 * before the new token; the block it completes (if any) is written to it.
 * sel [b][Hkv][k] and sel_scores (optional) are written as by
 * qsa_score_select, out [b][Hq][d] as by qsa_sparse_attn_decode.
 * For bf16, k <= 64 and Bs >= 32, rows that are short (compressed keys of a
 * row up to 512 KiB) or numerous (64 rows or more) run in one kernel: one
 * workgroup per (sequence, KV head) compresses, selects and attends with no
 * hand-off of the selection through memory (with few rows, several
 * workgroups per row each attend over a slice of the same selection and the
 * last one merges them, as the decode call does); the attention states merge
 * in another order than the decode call's, so outputs agree within
 * rounding. Other shapes run the three calls in order, the selection on the
 * first part of the workspace and the attention on the rest. ws: device
 * scratch of qsa_workspace_bytes(shape, QSA_OP_DECODE_STEP, 1, kv_len),
 * zero-filled before its first use as for the decode call. */
qsa_status qsa_decode_step(const qsa_shape* shape, const void* q, const void* k, const void* v, float* k_comp,
                           int64_t kv_len, int64_t kv_cap, int32_t* sel, float* sel_scores, void* out,
                           void* ws, size_t ws_bytes, void* stream);

/* 1 when qsa_decode_step runs these sizes as the single fused kernel, 0 when
 * it runs the separate calls, -1 for invalid arguments. */
int qsa_decode_step_fused(const qsa_shape* shape, int64_t kv_len);

/* One decode step for a batch of sequences of different lengths (a ragged
 * batch): for every sequence b, the same results as qsa_decode_step with
 * kv_len = kv_lens[b] on that sequence alone ("Qwen4 in llama.cpp:
 * Dissecting PR #27742", section "QSA Is an Address-Selection Problem, Not a
 * New Attention Equation": selection and attention are per token; here each
 * sequence's token sits at its own position kv_lens[b]-1).
 *   kv_lens     device int32 [batch], 4-byte aligned; values are clamped
 *               into [1, max_kv_len] (so accesses stay in bounds).
 *   max_kv_len  host bound, >= every kv_lens[b] and <= kv_cap; it sizes the
 *               launch and the workspace.
 * Other arguments as for qsa_decode_step; sequence b reads K/V positions
 * [0, kv_lens[b]) and k_comp blocks [0, kv_lens[b]/Bs) of its own rows.
 * bf16 with k <= 64 and Bs >= 32 runs as the fused kernel. Every other
 * shape (at most 65536 candidates per row, else QSA_ERR_UNSUPPORTED) runs
 * the large selection's score pass, which also compresses each sequence's
 * closed block, then for bf16 the pick-and-attend kernel, for float32 the
 * per-row pick and the float32 attention; every kernel reads the
 * per-sequence lengths. ws: qsa_workspace_bytes(shape,
 * QSA_OP_DECODE_STEP_RAGGED, 1, max_kv_len) bytes, zero-filled before first
 * use. Outputs equal the per-sequence qsa_decode_step's up to the rounding
 * of the attention merge order (selections are identical). */
qsa_status qsa_decode_step_ragged(const qsa_shape* shape, const void* q, const void* k, const void* v,
                                  float* k_comp, const int32_t* kv_lens, int64_t max_kv_len, int64_t kv_cap,
                                  int32_t* sel, float* sel_scores, void* out, void* ws, size_t ws_bytes,
                                  void* stream);

/* The selection of a ragged decode batch as a call of its own: for every
 * sequence b, the selection of qsa_score_select for the single token at
 * position kv_lens[b] - 1 (q_len = 1, q_pos0 = kv_lens[b] - 1) on that
 * sequence alone. kv_lens and max_kv_len as for qsa_decode_step_ragged; q
 * [b][Hq][d]; k_comp as for qsa_score_select, holding every block complete
 * before each sequence's token (sequence b reads blocks [0, n_cand of its
 * row)); sel [b][Hkv][k] and sel_scores (optional) as for qsa_score_select.
 * Any top_k: the large selection's per-row score pass and pick read the
 * per-sequence lengths (at most 65536 candidates per row, else
 * QSA_ERR_UNSUPPORTED). Selections equal the oracle's for each sequence (a
 * tie within rounding may resolve either way, as for qsa_score_select; for
 * k > 64 they equal qsa_score_select's bit for bit). ws: device scratch of
 * qsa_workspace_bytes(shape, QSA_OP_SELECT_RAGGED, 1, max_kv_len) bytes
 * (scores and chunk lists; 0 when no row has a candidate). */
qsa_status qsa_score_select_ragged(const qsa_shape* shape, const void* q, const float* k_comp,
                                   const int32_t* kv_lens, int64_t max_kv_len, int64_t kv_cap, int32_t* sel,
                                   float* sel_scores, void* ws, size_t ws_bytes, void* stream);

/* The attention of a ragged decode batch as a call of its own: for every
 * sequence b, qsa_sparse_attn_decode with kv_len = kv_lens[b] on that
 * sequence alone (the causal bound of its token at kv_lens[b] - 1).
 * kv_lens and max_kv_len as for qsa_decode_step_ragged; q, k, v, sel, out as
 * for qsa_sparse_attn_decode (sequence b reads K/V positions [0,
 * kv_lens[b]) of its rows). Same kernels and plan as the decode call at
 * kv_len = max_kv_len, so outputs equal a per-sequence decode call's up to
 * the rounding of the slice merge order. ws: device scratch of
 * qsa_workspace_bytes(shape, QSA_OP_DECODE, 1, max_kv_len), zero-filled
 * before its first use as for the decode call. */
qsa_status qsa_sparse_attn_decode_ragged(const qsa_shape* shape, const void* q, const void* k, const void* v,
                                         const int32_t* kv_lens, int64_t max_kv_len, int64_t kv_cap,
                                         const int32_t* sel, void* out, void* ws, size_t ws_bytes,
                                         void* stream);

/* ------------------------------------------------------------------------
 * Learned-indexer variant of the selection ("Qwen4 in llama.cpp: Dissecting
 * PR #27742", section "QSA Is an Address-Selection Problem, Not a New
 * Attention Equation": indexer projections feed the compressed-block
 * representation that is scored to pick the kept blocks). The pages give
 * neither the projections nor how a group's heads combine; this library's
 * reading: keys and query heads are projected into an indexer space of
 * `dim` dimensions by W_k and W_q (float32 [head_dim][dim], shared by all
 * heads), a block's indexer key is the mean of its projected keys, each
 * query head scores a candidate with scale * <q W_q, indexer key>, and the
 * heads of a KV head's group combine by `agg`:
 *   QSA_AGG_SUM      the sum of the head scores;
 *   QSA_AGG_MAX      the largest head score;
 *   QSA_AGG_SOFTMAX  each head's scores turned into a softmax over the row's
 *                    candidates, summed over the heads.
 * Frame, forced block, top_k, tie rule and output format are those of
 * qsa_score_select. */
enum { QSA_AGG_SUM = 0, QSA_AGG_MAX = 1, QSA_AGG_SOFTMAX = 2 };

typedef struct {
  int32_t dim;  /* indexer dimension: 64 or 128 */
  int32_t agg;  /* QSA_AGG_* */
  float scale;  /* score scale; 0 means 1/sqrt(dim) */
} qsa_indexer;

/* Indexer keys k_idx [b][Hkv][kv_cap/Bs][dim] (float32) of the complete
 * blocks block_begin .. kv_len/Bs - 1: W_k^T times the block's compressed key
 * (k_comp as written by qsa_compress_keys), which equals the mean of the
 * block's projected keys. w_k: device float32 [head_dim][dim]. No workspace.
 * Errors as qsa_compress_keys; QSA_ERR_INVALID also for a bad indexer
 * struct (dim not 64 or 128, agg out of range, scale negative or not
 * finite). */
qsa_status qsa_indexer_keys(const qsa_shape* shape, const qsa_indexer* idx, const float* w_k,
                            const float* k_comp, int64_t kv_len, int64_t kv_cap, int64_t block_begin,
                            float* k_idx, void* stream);

/* Selection scored in indexer space for query rows at positions q_pos0 ..
 * q_pos0+q_len-1 (layouts and frame as qsa_score_select; kv_len must be
 * q_pos0 + q_len). w_q: device float32 [head_dim][dim]; k_idx as written by
 * qsa_indexer_keys for every block below the rows' own blocks (and, with
 * keep_tail, the complete own block). sel_scores (optional) receives the
 * aggregated score of every kept candidate (+inf for the forced block, -inf
 * for padding). One workgroup per (sequence, row, KV head) scores the row's
 * candidates. top_k <= 64: the row's top list is kept in registers and ws is
 * not used. top_k > 64: every candidate's aggregated score goes to ws and
 * the large selection's per-row pick (radix cutoff) runs on them, as in
 * qsa_score_select; ws: qsa_workspace_bytes(shape, QSA_OP_INDEXER_SELECT,
 * q_len, kv_len) bytes (no zero-fill needed), else QSA_ERR_WORKSPACE;
 * QSA_ERR_UNSUPPORTED with more than 65536 candidates per row. */
qsa_status qsa_indexer_select(const qsa_shape* shape, const qsa_indexer* idx, const float* w_q, const void* q,
                              int64_t q_len, int64_t q_pos0, const float* k_idx, int64_t kv_len, int64_t kv_cap,
                              int32_t* sel, float* sel_scores, void* ws, size_t ws_bytes, void* stream);

/* One decode step with the learned indexer, in one kernel: the same results
 * as qsa_compress_keys and qsa_indexer_keys over the block the new token
 * closes (if any; block_begin = (kv_len-1)/Bs), then qsa_indexer_select
 * (q_len = 1, q_pos0 = kv_len-1) and qsa_sparse_attn_decode on its
 * selection ("Qwen4 in llama.cpp: Dissecting PR #27742", section "QSA Is an
 * Address-Selection Problem, Not a New Attention Equation": the indexer
 * scores compressed blocks, and attention runs over the kept ones).
 *   q           [b][Hq][d] bf16, the new token's query heads;
 *   k, v        [b][Hkv][kv_cap][d] bf16, holding positions 0 .. kv_len-1;
 *   k_comp      [b][Hkv][kv_cap/Bs][d] float32, blocks below (kv_len-1)/Bs
 *               written; the closed block is added;
 *   k_idx       [b][Hkv][kv_cap/Bs][dim] float32, the same blocks; the
 *               closed block's indexer key is added;
 *   w_q, w_k    device float32 [d][dim];
 *   sel, sel_scores, out: as qsa_decode_step.
 * One workgroup per (sequence, KV head); no workspace. Serves bf16 with
 * top_k <= 64 (QSA_ERR_UNSUPPORTED otherwise: use the separate calls).
 * Selections and the two caches equal the separate calls' bit for bit;
 * outputs agree up to the rounding of the attention's merge order.
 * QSA_ERR_INVALID for null or misaligned pointers (all 16-byte aligned),
 * kv_len outside [1, kv_cap] or a bad indexer struct. */
qsa_status qsa_indexer_decode_step(const qsa_shape* shape, const qsa_indexer* idx, const float* w_q,
                                   const float* w_k, const void* q, const void* k, const void* v, float* k_comp,
                                   float* k_idx, int64_t kv_len, int64_t kv_cap, int32_t* sel, float* sel_scores,
                                   void* out, void* stream);

/* ------------------------------------------------------------------------
 * Rotated 8-bit K/V cache ("Qwen4 in llama.cpp: Dissecting PR #27742",
 * section "Quantized KV Exposed a Backend Storage Invariant": K and V are
 * stored Hadamard-rotated and quantized, attention runs in the rotated basis
 * and its output is rotated back; the indexer's compressed keys stay
 * unrotated, so qsa_compress_keys and qsa_score_select keep reading the
 * bf16 keys). This library's reading of the storage:
 *   rotation  the unnormalised Walsh-Hadamard transform of each head_dim
 *             row (Sylvester order), butterfly stages h = 1, 2, ...,
 *             head_dim/2 in that order, pair (i, i+h) -> (x_i + x_{i+h},
 *             x_i - x_{i+h}), in float32;
 *   codes     per 32 values of a rotated row: scale = (largest magnitude /
 *             127) rounded to float16, code = round-half-even(value /
 *             scale) clamped to [-127, 127] (0 if the scale is 0);
 *             value = code * scale.
 * Layouts: k_q, v_q int8 [b][Hkv][kv_cap][head_dim]; k_scales, v_scales
 * float16 bit patterns [b][Hkv][kv_cap][head_dim/32]; all 16-byte aligned. */

/* Rotate and quantize positions pos_begin .. kv_len-1 of K and V (bf16,
 * [b][Hkv][kv_cap][head_dim]) into the 8-bit cache. No workspace.
 * QSA_ERR_UNSUPPORTED for float32 shapes; QSA_OK without work when
 * pos_begin >= kv_len. */
qsa_status qsa_kv_quantize(const qsa_shape* shape, const void* k, const void* v, int64_t kv_len, int64_t kv_cap,
                           int64_t pos_begin, int8_t* k_q, int8_t* v_q, uint16_t* k_scales, uint16_t* v_scales,
                           void* stream);

/* qsa_sparse_attn_decode over the 8-bit cache: the query heads are rotated,
 * scores use (H q).(H k)/head_dim, and every slice's output is rotated back
 * before the slices merge. Same selection, plan and workspace as
 * qsa_sparse_attn_decode (ws: qsa_workspace_bytes(shape, QSA_OP_DECODE, 1,
 * kv_len) bytes, zero-filled before first use). Blocks shorter than 32 keys
 * gather each 32-key unit's rows from several entries, as the bf16 kernel
 * does. bf16 only, else QSA_ERR_UNSUPPORTED. */
qsa_status qsa_sparse_attn_decode_q8(const qsa_shape* shape, const void* q, const int8_t* k_q, const int8_t* v_q,
                                     const uint16_t* k_scales, const uint16_t* v_scales, int64_t kv_len,
                                     int64_t kv_cap, const int32_t* sel, void* out, void* ws, size_t ws_bytes,
                                     void* stream);

/* qsa_sparse_attn_prefill over the 8-bit cache: query rows at positions
 * q_pos0 .. q_pos0+q_len-1 (q, sel and out laid out as for
 * qsa_sparse_attn_prefill), k_q, v_q, k_scales, v_scales holding positions
 * 0 .. q_pos0+q_len-1. Each row's query heads are rotated, its scores are
 * (H q).(H k)/head_dim over the codes, causal at the row's own position, and
 * its output is rotated back. Two ways, the same results up to rounding:
 *   tiled   where the tiled bf16 prefill serves the shape (Bs >= 32,
 *           top_k <= 64) and the rows' selected keys (q_len * top_k * Bs)
 *           are at least the cache's q_pos0 + q_len positions, and ws holds
 *           qsa_workspace_bytes(shape, QSA_OP_PREFILL_Q8, q_len,
 *           q_pos0 + q_len) bytes (16-byte aligned, no zero-fill needed):
 *           those positions are dequantized and rotated back into bf16 rows
 *           in ws (H H = head_dim I, so attention over them with the plain
 *           query equals attention over the rotated codes with the rotated
 *           query, rotated back), then the tiled kernel runs on them;
 *   rows    otherwise (ws may be null): one workgroup per (sequence, row, KV
 *           head) over the codes, any top_k and block size.
 * bf16 only, else QSA_ERR_UNSUPPORTED (also when the rows way is taken and
 * batch * q_len * Hkv exceeds 2^31 - 1). */
qsa_status qsa_sparse_attn_prefill_q8(const qsa_shape* shape, const void* q, const int8_t* k_q, const int8_t* v_q,
                                      const uint16_t* k_scales, const uint16_t* v_scales, int64_t q_len,
                                      int64_t q_pos0, int64_t kv_cap, const int32_t* sel, void* out, void* ws,
                                      size_t ws_bytes, void* stream);

/* One decode step over the 8-bit cache: qsa_kv_quantize of the new position
 * kv_len - 1, then, in one kernel, what qsa_decode_step does (compress the
 * block the new token closes from the bf16 keys k, select from k_comp) with
 * the attention of qsa_sparse_attn_decode_q8 over the codes. k and v are the
 * bf16 cache the new position is quantized from ([b][Hkv][kv_cap][head_dim],
 * read only at kv_len - 1 and, for the compression, in the closed block);
 * k_q, v_q, k_scales, v_scales as for qsa_kv_quantize, holding positions
 * 0 .. kv_len - 2 already. sel, sel_scores (optional), out as for
 * qsa_decode_step. bf16 only (else QSA_ERR_UNSUPPORTED). On the shapes
 * qsa_decode_step runs as its fused kernel (qsa_decode_step_fused(shape,
 * kv_len) == 1) the quantization of the new position, the compression,
 * selection and attention are one kernel (the codes equal qsa_kv_quantize's
 * bit for bit); on the others (top_k > 64, blocks shorter than 32 keys) the selection of
 * qsa_decode_step (compressing the closed block from the bf16 keys) writes
 * sel, then the attention of qsa_sparse_attn_decode_q8 reads it; top_k > 64
 * keeps the selection's limit of 65536 candidate blocks per row
 * (QSA_ERR_UNSUPPORTED beyond). ws: device scratch of
 * qsa_workspace_bytes(shape, QSA_OP_DECODE_STEP, 1, kv_len), zero-filled
 * before its first use (the layout of qsa_decode_step: one workspace serves
 * a loop whose kv_len, and with it the path, changes from step to step). */
qsa_status qsa_decode_step_q8(const qsa_shape* shape, const void* q, const void* k, const void* v, float* k_comp,
                              int8_t* k_q, int8_t* v_q, uint16_t* k_scales, uint16_t* v_scales, int64_t kv_len,
                              int64_t kv_cap, int32_t* sel, float* sel_scores, void* out, void* ws, size_t ws_bytes,
                              void* stream);

/* ------------------------------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * qsa_decode_step with its workspace in library-owned device memory instead
 * of a caller buffer. Same arguments, results and errors as qsa_decode_step
 * without ws / ws_bytes; the same kernels run.
 *   scratch   a device array of QSA_NOALLOC_SCRATCH_BYTES inside the library,
 *             one per GPU the library runs on, held until the process ends;
 *             its address is looked up on the first call on each device.
 *   errors    QSA_ERR_WORKSPACE when the step's workspace
 *             (qsa_workspace_bytes(shape, QSA_OP_DECODE_STEP, 1, kv_len))
 *             exceeds QSA_NOALLOC_SCRATCH_BYTES; QSA_ERR_HIP when the lookup
 *             fails; the rest as qsa_decode_step (every check runs before
 *             anything is enqueued).
 *   work      a small kernel zeroes the step's arrival counters in the
 *             scratch, then the step runs; both on `stream`. Nothing is
 *             allocated or freed.
 *   races     every call on one GPU shares that GPU's scratch: calls that
 *             may overlap on one GPU (other streams, other host threads)
 *             race and must be ordered by the caller. */
#define QSA_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

qsa_status qsa_decode_step_noalloc(const qsa_shape* shape, const void* q, const void* k, const void* v,
                                   float* k_comp, int64_t kv_len, int64_t kv_cap, int32_t* sel, float* sel_scores,
                                   void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
