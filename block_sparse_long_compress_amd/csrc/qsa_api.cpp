// C ABI of the QSA library: argument validation, workspace sizing and
// dispatch to the kernels. Every check runs on the host before any HIP call;
// on failure nothing is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/qsa.h"
#include "qsa_internal.h"

namespace {

using qsa::Dims;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool pow2_in(int x, int lo, int hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }

// Decode-step workspace: two arrival-counter areas at fixed offsets (the
// fused step's or the attention's counters, then the split selection's),
// then scratch whose size follows kv_len (the selection's chunk lists or
// scores, then the attention's slice states). Whatever path a step takes,
// its counters live in those two areas, which every call leaves at zero, so
// one workspace zero-filled once serves a decode loop whose kv_len, and
// with it the path, changes from step to step.
struct StepWs {
  size_t sel_off;   // the selection's workspace (a split selection's counters land on the second area)
  size_t part_off;  // the attention's slice states
  size_t total;     // 0 when the step needs no workspace
};

StepWs step_ws(const Dims& s, int64_t kv_len, bool q8 = false) {
  StepWs w{};
  const size_t cnt = qsa::counter_bytes((int64_t)s.batch * s.hkv);
  const qsa::StepPlan sp = qsa::plan_decode_step(s, kv_len, false, q8);
  size_t att = 0, sel_ws = 0, sel_scratch = 0;
  w.sel_off = cnt;
  if (sp.fused) {
    att = sp.ws_bytes;
  } else {
    const qsa::SelectPlan sel_plan = qsa::plan_select(s, 1, kv_len - 1);
    sel_ws = sel_plan.ws_bytes;
    if (sel_plan.large) {  // scores and lists, no counters
      w.sel_off = 2 * cnt;
      sel_scratch = sel_ws;
    } else {
      sel_scratch = sel_ws > cnt ? sel_ws - cnt : 0;
    }
    if (s.dtype == QSA_BF16)  // q8: the full selection, then the 8-bit cache's decode attention
      att = q8                ? qsa::plan_decode(s, kv_len, false).ws_bytes
            : sel_plan.large  ? qsa::plan_pick_attend(s, sel_plan.n_chunks).ws_bytes
                              : qsa::plan_decode(s, kv_len).ws_bytes;
  }
  w.part_off = 2 * cnt + qsa::align_up(sel_scratch, 256);
  w.total = (att == 0 && sel_ws == 0) ? 0 : w.part_off + (att > cnt ? att - cnt : 0);
  return w;
}

// The ragged decode step on the shapes it serves without the fused kernel
// (bf16 with top_k > 64 or blocks shorter than 32 keys, float32): the large
// selection's score pass (at least one chunk, so that sequences closing a
// block compress it even when no sequence has a candidate yet), then for
// bf16 the pick-and-attend kernel's slice states, in the decode step's
// layout (float32 picks into sel and attends without a workspace).
StepWs ragged_large_ws(const Dims& s, int64_t max_kv_len, int64_t* n_chunks) {
  StepWs w{};
  const int64_t rows = (int64_t)s.batch * s.hkv;
  const size_t cnt = qsa::counter_bytes(rows);
  int64_t nc = qsa::plan_select_large(s, 1, max_kv_len - 1).n_chunks;
  if (nc < 1) nc = 1;
  const size_t sel_ws = (size_t)rows * nc * (256 * sizeof(uint32_t) + 16 * sizeof(uint64_t));
  // bf16: the pick-and-attend kernel's slice states; float32 attends with
  // one wave per row and needs none
  const size_t att = s.dtype == QSA_BF16 ? qsa::plan_pick_attend(s, nc).ws_bytes : 0;
  w.sel_off = 2 * cnt;
  w.part_off = 2 * cnt + qsa::align_up(sel_ws, 256);
  w.total = w.part_off + (att > cnt ? att - cnt : 0);
  if (n_chunks) *n_chunks = nc;
  return w;
}

// Prefill over the 8-bit cache by the tiled bf16 kernel: the cache's
// positions [0, q_pos0 + q_len) dequantized and rotated back into bf16 rows
// (K at k_off, V at v_off, each [b][Hkv][n_pad][d], n_pad a whole number of
// blocks), then the tiled kernel's own workspace at att_off. Taken where the
// tiled kernel serves the shape and the rows' selected keys (q_len * top_k *
// Bs) at least match the positions to convert; otherwise tiled is false and
// the call runs one query row per workgroup over the codes.
struct Q8PrefillWs {
  bool tiled;
  int64_t n_pad;
  size_t k_off, v_off, att_off, total;
};
Q8PrefillWs q8_prefill_ws(const Dims& s, int64_t q_len, int64_t q_pos0) {
  Q8PrefillWs w{};
  if (s.dtype != QSA_BF16) return w;
  const qsa::PrefillPlan plan = qsa::plan_prefill(s, q_len, q_pos0);
  const int64_t n_pos = q_pos0 + q_len;
  if (plan.rows || q_len * s.top_k * s.bs < n_pos) return w;
  w.tiled = true;
  w.n_pad = (n_pos + s.bs - 1) / s.bs * s.bs;
  const size_t cache = qsa::align_up((size_t)s.batch * s.hkv * w.n_pad * s.d * sizeof(uint16_t), 256);
  w.k_off = 0;
  w.v_off = cache;
  w.att_off = 2 * cache;
  w.total = w.att_off + plan.ws_bytes;
  return w;
}

// Shape checks shared by every entry point.
qsa_status check_shape(const qsa_shape* sh, Dims* out) {
  if (!sh) return QSA_ERR_INVALID;
  if (sh->batch <= 0 || sh->n_q_heads <= 0 || sh->n_kv_heads <= 0 || sh->head_dim <= 0 || sh->block_size <= 0 ||
      sh->top_k <= 0)
    return QSA_ERR_INVALID;
  if (sh->n_q_heads % sh->n_kv_heads != 0) return QSA_ERR_INVALID;
  if (sh->dtype != QSA_F32 && sh->dtype != QSA_BF16) return QSA_ERR_INVALID;
  if (!std::isfinite(sh->scale) || sh->scale < 0.f) return QSA_ERR_INVALID;
  if (sh->keep_tail != 0 && sh->keep_tail != 1) return QSA_ERR_INVALID;
  if (sh->keep_tail && sh->top_k < 2) return QSA_ERR_INVALID;  // a complete-block row would see nothing
  const int G = sh->n_q_heads / sh->n_kv_heads;
  if (sh->head_dim != 64 && sh->head_dim != 128) return QSA_ERR_UNSUPPORTED;
  if (!pow2_in(sh->block_size, 4, 128)) return QSA_ERR_UNSUPPORTED;
  if (sh->top_k > qsa::kMaxTopKLarge) return QSA_ERR_UNSUPPORTED;
  if (!pow2_in(G, 1, 16)) return QSA_ERR_UNSUPPORTED;
  if (sh->batch > 65535 || sh->n_kv_heads > 65535) return QSA_ERR_UNSUPPORTED;
  out->batch = sh->batch;
  out->hq = sh->n_q_heads;
  out->hkv = sh->n_kv_heads;
  out->group = G;
  out->d = sh->head_dim;
  out->bs = sh->block_size;
  out->top_k = sh->top_k;
  out->dtype = sh->dtype;
  out->scale = sh->scale == 0.f ? (float)(1.0 / std::sqrt((double)sh->head_dim)) : sh->scale;
  out->keep_tail = sh->keep_tail;
  return QSA_OK;
}

// Positions are bounded so that block ids fit in int32 and grids stay small.
constexpr int64_t kMaxPositions = int64_t(1) << 31;

qsa_status check_prefill_limits(const Dims& s, int64_t q_len, int64_t q_pos0) {
  if (q_len > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
  // one workgroup per query row on the per-row path
  if (s.dtype == QSA_BF16 && qsa::plan_prefill(s, q_len, q_pos0).rows &&
      (int64_t)s.batch * q_len * s.hkv > 0x7FFFFFFF)
    return QSA_ERR_UNSUPPORTED;
  return QSA_OK;
}

qsa_status hip_status(hipError_t e) { return e == hipSuccess ? QSA_OK : QSA_ERR_HIP; }

}  // namespace

extern "C" {

int qsa_abi_version(void) { return QSA_ABI_VERSION; }

const char* qsa_status_str(qsa_status status) {
  switch (status) {
    case QSA_OK:
      return "QSA_OK";
    case QSA_ERR_INVALID:
      return "QSA_ERR_INVALID: invalid argument";
    case QSA_ERR_UNSUPPORTED:
      return "QSA_ERR_UNSUPPORTED: valid but unsupported shape";
    case QSA_ERR_WORKSPACE:
      return "QSA_ERR_WORKSPACE: workspace missing or too small";
    case QSA_ERR_HIP:
      return "QSA_ERR_HIP: kernel launch failed";
  }
  return "QSA_ERR_UNKNOWN";
}

size_t qsa_workspace_bytes(const qsa_shape* shape, int op, int64_t q_len, int64_t kv_len) {
  Dims s;
  if (check_shape(shape, &s) != QSA_OK) return (size_t)-1;
  switch (op) {
    case QSA_OP_COMPRESS:
      return 0;
    case QSA_OP_SELECT:
      if (q_len <= 0 || kv_len < q_len || kv_len > kMaxPositions) return (size_t)-1;
      // k > 64 serves at most kMaxCandLarge candidates per row
      if (s.top_k > 64 && qsa::max_candidates(s, kv_len) > qsa::kMaxCandLarge) return (size_t)-1;
      return qsa::plan_select(s, q_len, kv_len - q_len).ws_bytes;
    case QSA_OP_DECODE:
      if (kv_len <= 0 || kv_len > kMaxPositions) return (size_t)-1;
      // the narrow plan's (the 8-bit decode's), which covers the bf16 decode's too
      return s.dtype == QSA_BF16 ? qsa::plan_decode(s, kv_len, false).ws_bytes : 0;
    case QSA_OP_PREFILL:
      if (q_len <= 0 || kv_len < q_len || kv_len > kMaxPositions) return (size_t)-1;
      return qsa::plan_prefill(s, q_len, kv_len - q_len).ws_bytes;
    case QSA_OP_DECODE_STEP: {
      if (kv_len <= 0 || kv_len > kMaxPositions) return (size_t)-1;
      if (!qsa::plan_decode_step(s, kv_len).fused && s.top_k > 64 && qsa::max_candidates(s, kv_len) > qsa::kMaxCandLarge)
        return (size_t)-1;  // the selection's large-k limit
    {
      // the plain step's and the 8-bit step's (same layout; the latter may split rows more)
      const size_t a = step_ws(s, kv_len).total, b8 = step_ws(s, kv_len, true).total;
      return a > b8 ? a : b8;
    }
    }
    case QSA_OP_PREFILL_Q8:
      if (q_len <= 0 || kv_len < q_len || kv_len > kMaxPositions) return (size_t)-1;
      return q8_prefill_ws(s, q_len, kv_len - q_len).total;
    case QSA_OP_SELECT_RAGGED:
      if (kv_len <= 0 || kv_len > kMaxPositions) return (size_t)-1;
      if (qsa::max_candidates(s, kv_len) > qsa::kMaxCandLarge) return (size_t)-1;
      return qsa::plan_select_large(s, 1, kv_len - 1).ws_bytes;
    case QSA_OP_INDEXER_SELECT:
      if (q_len <= 0 || kv_len < q_len || kv_len > kMaxPositions) return (size_t)-1;
      if (s.top_k <= 64) return 0;
      // the large selection's scores and chunk lists (at most kMaxCandLarge candidates per row)
      if (qsa::max_candidates(s, kv_len) > qsa::kMaxCandLarge) return (size_t)-1;
      return qsa::plan_select(s, q_len, kv_len - q_len).ws_bytes;
    case QSA_OP_DECODE_STEP_RAGGED: {
      if (kv_len <= 0 || kv_len > kMaxPositions) return (size_t)-1;
      // the decode step's layout: two arrival-counter areas, then the rest
      const qsa::StepPlan sp = qsa::plan_decode_step(s, kv_len, true);
      if (!sp.fused) {
        if (qsa::max_candidates(s, kv_len) > qsa::kMaxCandLarge) return (size_t)-1;
        return ragged_large_ws(s, kv_len, nullptr).total;
      }
      return sp.ws_bytes > 0 ? sp.ws_bytes + qsa::counter_bytes((int64_t)s.batch * s.hkv) : 0;
    }
  }
  return (size_t)-1;
}

qsa_status qsa_compress_keys(const qsa_shape* shape, const void* k, int64_t kv_len, int64_t kv_cap,
                             int64_t block_begin, float* k_comp, void* stream) {
  Dims s;
  qsa_status st = check_shape(shape, &s);
  if (st != QSA_OK) return st;
  if (kv_len < 0 || kv_cap <= 0 || kv_len > kv_cap || block_begin < 0) return QSA_ERR_INVALID;
  if (kv_cap > kMaxPositions) return QSA_ERR_UNSUPPORTED;
  const int64_t blk_end = kv_len / s.bs;
  if (block_begin >= blk_end) return QSA_OK;  // no complete block in range: nothing is read or written
  if (!k || !k_comp || !aligned16(k) || !aligned16(k_comp)) return QSA_ERR_INVALID;
  return hip_status(qsa::launch_compress(s, k, kv_cap, block_begin, blk_end, k_comp,
                                         static_cast<hipStream_t>(stream)));
}

qsa_status qsa_score_select(const qsa_shape* shape, const void* q, int64_t q_len, int64_t q_pos0,
                            const float* k_comp, int64_t kv_len, int64_t kv_cap, int32_t* sel, float* sel_scores,
                            void* ws, size_t ws_bytes, void* stream) {
  Dims s;
  qsa_status st = check_shape(shape, &s);
  if (st != QSA_OK) return st;
  if (!q || !sel || !aligned16(q) || !aligned16(sel)) return QSA_ERR_INVALID;
  if (sel_scores && !aligned16(sel_scores)) return QSA_ERR_INVALID;
  if (q_len <= 0 || q_pos0 < 0 || kv_len != q_pos0 + q_len || kv_cap <= 0 || kv_len > kv_cap) return QSA_ERR_INVALID;
  // k_comp is read only for candidate blocks, which exist once a row sits past the first block
  if (qsa::max_candidates(s, kv_len) > 0 && (!k_comp || !aligned16(k_comp))) return QSA_ERR_INVALID;
  if (kv_cap > kMaxPositions) return QSA_ERR_UNSUPPORTED;
  if (s.top_k > 64 && qsa::max_candidates(s, kv_len) > qsa::kMaxCandLarge) return QSA_ERR_UNSUPPORTED;
  const qsa::SelectPlan plan = qsa::plan_select(s, q_len, q_pos0);
  if (plan.grid > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
  if (plan.ws_bytes > 0 && (!ws || ws_bytes < plan.ws_bytes || !aligned16(ws))) return QSA_ERR_WORKSPACE;
  return hip_status(qsa::launch_select(s, plan, q, q_len, q_pos0, k_comp, kv_cap, sel, sel_scores, ws,
                                       static_cast<hipStream_t>(stream)));
}

qsa_status qsa_sparse_attn_decode(const qsa_shape* shape, const void* q, const void* k, const void* v,
                                  int64_t kv_len, int64_t kv_cap, const int32_t* sel, void* out, void* ws,
                                  size_t ws_bytes, void* stream) {
  Dims s;
  qsa_status st = check_shape(shape, &s);
  if (st != QSA_OK) return st;
  if (!q || !k || !v || !sel || !out) return QSA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(sel) || !aligned16(out)) return QSA_ERR_INVALID;
  if (kv_len <= 0 || kv_cap <= 0 || kv_len > kv_cap) return QSA_ERR_INVALID;
  if (kv_cap > kMaxPositions) return QSA_ERR_UNSUPPORTED;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (s.dtype == QSA_F32)
    return hip_status(qsa::launch_attn_f32(s, static_cast<const float*>(q), static_cast<const float*>(k),
                                           static_cast<const float*>(v), 1, kv_len - 1, kv_cap, sel,
                                           static_cast<float*>(out), hs));
  const qsa::DecodePlan plan = qsa::plan_decode(s, kv_len);
  if ((int64_t)s.batch * s.hkv * plan.n_split > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
  if (plan.ws_bytes > 0 && (!ws || ws_bytes < plan.ws_bytes || !aligned16(ws))) return QSA_ERR_WORKSPACE;
  // arrival counters at the start of the workspace, the slice states after them
  char* part = ws ? static_cast<char*>(ws) + qsa::counter_bytes((int64_t)s.batch * s.hkv) : nullptr;
  return hip_status(qsa::launch_decode(s, plan, q, k, v, kv_len, kv_cap, sel, out, ws, part, hs));
}

qsa_status qsa_sparse_attn_prefill(const qsa_shape* shape, const void* q, const void* k, const void* v,
                                   int64_t q_len, int64_t q_pos0, int64_t kv_cap, const int32_t* sel, void* out,
                                   void* ws, size_t ws_bytes, void* stream) {
  Dims s;
  qsa_status st = check_shape(shape, &s);
  if (st != QSA_OK) return st;
  if (!q || !k || !v || !sel || !out) return QSA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(sel) || !aligned16(out)) return QSA_ERR_INVALID;
  if (q_len <= 0 || q_pos0 < 0 || kv_cap <= 0 || q_pos0 + q_len > kv_cap) return QSA_ERR_INVALID;
  if (kv_cap > kMaxPositions) return QSA_ERR_UNSUPPORTED;
  st = check_prefill_limits(s, q_len, q_pos0);
  if (st != QSA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (s.dtype == QSA_F32)
    return hip_status(qsa::launch_attn_f32(s, static_cast<const float*>(q), static_cast<const float*>(k),
                                           static_cast<const float*>(v), q_len, q_pos0, kv_cap, sel,
                                           static_cast<float*>(out), hs));
  const qsa::PrefillPlan plan = qsa::plan_prefill(s, q_len, q_pos0);
  if (plan.ws_bytes > 0 && (!ws || ws_bytes < plan.ws_bytes || !aligned16(ws))) return QSA_ERR_WORKSPACE;
  return hip_status(qsa::launch_prefill(s, plan, q, k, v, q_len, q_pos0, kv_cap, sel, out, ws, hs));
}

int qsa_decode_step_fused(const qsa_shape* shape, int64_t kv_len) {
  Dims s;
  if (check_shape(shape, &s) != QSA_OK || kv_len <= 0 || kv_len > kMaxPositions) return -1;
  return qsa::plan_decode_step(s, kv_len).fused ? 1 : 0;
}

}  // extern "C"

namespace qsa {
// Every check of qsa_decode_step except the workspace's, in the order the
// call makes them, including the limits of the plan the step will take: a
// step that passes enqueues all its launches (barring a runtime failure).
qsa_status decode_step_validate(const qsa_shape* shape, const void* q, const void* k, const void* v,
                                const float* k_comp, int64_t kv_len, int64_t kv_cap, const int32_t* sel,
                                const float* sel_scores, const void* out) {
  Dims s;
  qsa_status st = check_shape(shape, &s);
  if (st != QSA_OK) return st;
  if (!q || !k || !v || !k_comp || !sel || !out) return QSA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_comp) || !aligned16(sel) || !aligned16(out))
    return QSA_ERR_INVALID;
  if (sel_scores && !aligned16(sel_scores)) return QSA_ERR_INVALID;
  if (kv_len <= 0 || kv_cap <= 0 || kv_len > kv_cap) return QSA_ERR_INVALID;
  if (kv_cap > kMaxPositions) return QSA_ERR_UNSUPPORTED;
  const qsa::StepPlan sp = qsa::plan_decode_step(s, kv_len);
  if (sp.fused)
    return (int64_t)(s.batch * (int64_t)s.hkv + 7) * sp.n_split * 8 > 0x7FFFFFFF ? QSA_ERR_UNSUPPORTED : QSA_OK;
  if (s.top_k > 64 && qsa::max_candidates(s, kv_len) > qsa::kMaxCandLarge) return QSA_ERR_UNSUPPORTED;
  const qsa::SelectPlan sel_plan = qsa::plan_select(s, 1, kv_len - 1);
  if ((int64_t)s.batch * s.hkv * (sel_plan.n_chunks > 0 ? sel_plan.n_chunks : 1) > 0x7FFFFFFF)
    return QSA_ERR_UNSUPPORTED;
  if (s.dtype == QSA_BF16 && sel_plan.large) {
    if ((int64_t)s.batch * s.hkv * qsa::plan_pick_attend(s, sel_plan.n_chunks).n_split > 0x7FFFFFFF)
      return QSA_ERR_UNSUPPORTED;
  } else if (s.dtype == QSA_BF16) {
    if ((int64_t)s.batch * s.hkv * qsa::plan_decode(s, kv_len).n_split > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
  }
  return QSA_OK;
}
}  // namespace qsa

extern "C" {

qsa_status qsa_decode_step(const qsa_shape* shape, const void* q, const void* k, const void* v, float* k_comp,
                           int64_t kv_len, int64_t kv_cap, int32_t* sel, float* sel_scores, void* out, void* ws,
                           size_t ws_bytes, void* stream) {
  qsa_status st = qsa::decode_step_validate(shape, q, k, v, k_comp, kv_len, kv_cap, sel, sel_scores, out);
  if (st != QSA_OK) return st;
  Dims s;
  check_shape(shape, &s);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const qsa::StepPlan sp = qsa::plan_decode_step(s, kv_len);
  const StepWs lay = step_ws(s, kv_len);
  if (lay.total > 0 && (!ws || ws_bytes < lay.total || !aligned16(ws))) return QSA_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  char* sel_ws = base ? base + lay.sel_off : nullptr;
  char* part = base ? base + lay.part_off : nullptr;
  if (sp.fused)
    return hip_status(
        qsa::launch_decode_step(s, sp, q, k, v, k_comp, kv_len, kv_cap, sel, sel_scores, out, base, part, hs));
  // separate launches: the selection (which also compresses the block the new
  // token closes, if any, before scoring it), then the attention
  const qsa::SelectPlan sel_plan = qsa::plan_select(s, 1, kv_len - 1);
  const int64_t close_block = kv_len % s.bs == 0 ? kv_len / s.bs - 1 : -1;
  if (s.dtype == QSA_BF16 && sel_plan.large) {
    // the score pass, then one kernel that picks each row's blocks and
    // attends over them
    const qsa::PickAttendPlan pa = qsa::plan_pick_attend(s, sel_plan.n_chunks);
    st = hip_status(qsa::launch_select(s, sel_plan, q, 1, kv_len - 1, k_comp, kv_cap, sel, sel_scores, sel_ws, hs, k,
                                       close_block, false));
    if (st != QSA_OK) return st;
    return hip_status(
        qsa::launch_pick_attend(s, pa, q, k, v, sel, sel_scores, sel_ws, out, base, part, kv_len, kv_cap, hs));
  }
  st = hip_status(
      qsa::launch_select(s, sel_plan, q, 1, kv_len - 1, k_comp, kv_cap, sel, sel_scores, sel_ws, hs, k, close_block));
  if (st != QSA_OK) return st;
  if (s.dtype == QSA_F32) return qsa_sparse_attn_decode(shape, q, k, v, kv_len, kv_cap, sel, out, nullptr, 0, stream);
  const qsa::DecodePlan plan = qsa::plan_decode(s, kv_len);
  return hip_status(qsa::launch_decode(s, plan, q, k, v, kv_len, kv_cap, sel, out, base, part, hs));
}

qsa_status qsa_score_select_ragged(const qsa_shape* shape, const void* q, const float* k_comp,
                                   const int32_t* kv_lens, int64_t max_kv_len, int64_t kv_cap, int32_t* sel,
                                   float* sel_scores, void* ws, size_t ws_bytes, void* stream) {
  Dims s;
  qsa_status st = check_shape(shape, &s);
  if (st != QSA_OK) return st;
  if (!q || !kv_lens || !sel || !aligned16(q) || !aligned16(sel) || (reinterpret_cast<uintptr_t>(kv_lens) & 3u) != 0)
    return QSA_ERR_INVALID;
  if (sel_scores && !aligned16(sel_scores)) return QSA_ERR_INVALID;
  if (max_kv_len <= 0 || kv_cap <= 0 || max_kv_len > kv_cap) return QSA_ERR_INVALID;
  // k_comp is read only for candidate blocks, which exist once a row sits past the first block
  if (qsa::max_candidates(s, max_kv_len) > 0 && (!k_comp || !aligned16(k_comp))) return QSA_ERR_INVALID;
  if (kv_cap > kMaxPositions) return QSA_ERR_UNSUPPORTED;
  if (qsa::max_candidates(s, max_kv_len) > qsa::kMaxCandLarge) return QSA_ERR_UNSUPPORTED;
  // every top_k through the large selection's per-row score pass and pick,
  // which read the per-sequence lengths (no key cache: nothing is compressed)
  const qsa::SelectPlan plan = qsa::plan_select_large(s, 1, max_kv_len - 1);
  if (plan.grid > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
  if (plan.ws_bytes > 0 && (!ws || ws_bytes < plan.ws_bytes || !aligned16(ws))) return QSA_ERR_WORKSPACE;
  return hip_status(qsa::launch_select(s, plan, q, 1, max_kv_len - 1, k_comp, kv_cap, sel, sel_scores, ws,
                                       static_cast<hipStream_t>(stream), nullptr, -1, true, kv_lens));
}

qsa_status qsa_sparse_attn_decode_ragged(const qsa_shape* shape, const void* q, const void* k, const void* v,
                                         const int32_t* kv_lens, int64_t max_kv_len, int64_t kv_cap,
                                         const int32_t* sel, void* out, void* ws, size_t ws_bytes,
                                         void* stream) {
  Dims s;
  qsa_status st = check_shape(shape, &s);
  if (st != QSA_OK) return st;
  if (!q || !k || !v || !kv_lens || !sel || !out) return QSA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(sel) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(kv_lens) & 3u) != 0)
    return QSA_ERR_INVALID;
  if (max_kv_len <= 0 || kv_cap <= 0 || max_kv_len > kv_cap) return QSA_ERR_INVALID;
  if (kv_cap > kMaxPositions) return QSA_ERR_UNSUPPORTED;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (s.dtype == QSA_F32)
    return hip_status(qsa::launch_attn_f32(s, static_cast<const float*>(q), static_cast<const float*>(k),
                                           static_cast<const float*>(v), 1, max_kv_len - 1, kv_cap, sel,
                                           static_cast<float*>(out), hs, kv_lens));
  const qsa::DecodePlan plan = qsa::plan_decode(s, max_kv_len);
  if ((int64_t)s.batch * s.hkv * plan.n_split > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
  if (plan.ws_bytes > 0 && (!ws || ws_bytes < plan.ws_bytes || !aligned16(ws))) return QSA_ERR_WORKSPACE;
  // arrival counters at the start of the workspace, the slice states after them
  char* part = ws ? static_cast<char*>(ws) + qsa::counter_bytes((int64_t)s.batch * s.hkv) : nullptr;
  return hip_status(qsa::launch_decode(s, plan, q, k, v, max_kv_len, kv_cap, sel, out, ws, part, hs, kv_lens));
}

qsa_status qsa_decode_step_ragged(const qsa_shape* shape, const void* q, const void* k, const void* v,
                                  float* k_comp, const int32_t* kv_lens, int64_t max_kv_len, int64_t kv_cap,
                                  int32_t* sel, float* sel_scores, void* out, void* ws, size_t ws_bytes,
                                  void* stream) {
  Dims s;
  qsa_status st = check_shape(shape, &s);
  if (st != QSA_OK) return st;
  if (!q || !k || !v || !k_comp || !kv_lens || !sel || !out) return QSA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_comp) || !aligned16(sel) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(kv_lens) & 3u) != 0)
    return QSA_ERR_INVALID;
  if (sel_scores && !aligned16(sel_scores)) return QSA_ERR_INVALID;
  if (max_kv_len <= 0 || kv_cap <= 0 || max_kv_len > kv_cap) return QSA_ERR_INVALID;
  if (kv_cap > kMaxPositions) return QSA_ERR_UNSUPPORTED;
  const qsa::StepPlan sp = qsa::plan_decode_step(s, max_kv_len, true);
  if (!sp.fused) {
    // every shape without the fused kernel (bf16 with k > 64 or blocks
    // shorter than 32 keys, float32): the large selection's score pass,
    // which compresses each sequence's closed block, then for bf16 the
    // pick-and-attend kernel, for float32 the per-row pick and the float32
    // attention; every kernel reads the per-sequence lengths
    if (qsa::max_candidates(s, max_kv_len) > qsa::kMaxCandLarge) return QSA_ERR_UNSUPPORTED;
    int64_t n_chunks = 0;
    const StepWs lay = ragged_large_ws(s, max_kv_len, &n_chunks);
    const int64_t rows = (int64_t)s.batch * s.hkv;
    const qsa::PickAttendPlan pa = qsa::plan_pick_attend(s, n_chunks);
    if (rows * n_chunks > 0x7FFFFFFF || rows * pa.n_split > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < lay.total || !aligned16(ws)) return QSA_ERR_WORKSPACE;
    qsa::SelectPlan sel_plan = qsa::plan_select_large(s, 1, max_kv_len - 1);
    sel_plan.n_chunks = n_chunks;
    char* base = static_cast<char*>(ws);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const bool f32 = s.dtype == QSA_F32;
    st = hip_status(qsa::launch_select(s, sel_plan, q, 1, max_kv_len - 1, k_comp, kv_cap, sel, sel_scores,
                                       base + lay.sel_off, hs, k, -1, f32, kv_lens));
    if (st != QSA_OK) return st;
    if (f32)
      return hip_status(qsa::launch_attn_f32(s, static_cast<const float*>(q), static_cast<const float*>(k),
                                             static_cast<const float*>(v), 1, max_kv_len - 1, kv_cap, sel,
                                             static_cast<float*>(out), hs, kv_lens));
    return hip_status(qsa::launch_pick_attend(s, pa, q, k, v, sel, sel_scores, base + lay.sel_off, out, base,
                                              base + lay.part_off, max_kv_len, kv_cap, hs, kv_lens));
  }
  if ((int64_t)(s.batch * (int64_t)s.hkv + 7) * sp.n_split * 8 > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
  const size_t cnt = qsa::counter_bytes((int64_t)s.batch * s.hkv);
  const size_t need = sp.ws_bytes > 0 ? sp.ws_bytes + cnt : 0;  // two counter areas, then the rest
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return QSA_ERR_WORKSPACE;
  char* part = ws ? static_cast<char*>(ws) + 2 * cnt : nullptr;
  return hip_status(qsa::launch_decode_step(s, sp, q, k, v, k_comp, max_kv_len, kv_cap, sel, sel_scores, out, ws,
                                            part, static_cast<hipStream_t>(stream), kv_lens));
}

namespace {
qsa_status check_indexer(const qsa_indexer* idx, const Dims& s, qsa::IndexerDims* out) {
  if (!idx) return QSA_ERR_INVALID;
  if (idx->dim != 64 && idx->dim != 128) return QSA_ERR_INVALID;
  if (idx->agg < QSA_AGG_SUM || idx->agg > QSA_AGG_SOFTMAX) return QSA_ERR_INVALID;
  if (!std::isfinite(idx->scale) || idx->scale < 0.f) return QSA_ERR_INVALID;
  (void)s;
  out->dim = idx->dim;
  out->agg = idx->agg;
  out->scale = idx->scale == 0.f ? (float)(1.0 / std::sqrt((double)idx->dim)) : idx->scale;
  return QSA_OK;
}
}  // namespace

qsa_status qsa_indexer_keys(const qsa_shape* shape, const qsa_indexer* idx, const float* w_k,
                            const float* k_comp, int64_t kv_len, int64_t kv_cap, int64_t block_begin,
                            float* k_idx, void* stream) {
  Dims s;
  qsa_status st = check_shape(shape, &s);
  if (st != QSA_OK) return st;
  qsa::IndexerDims ix;
  st = check_indexer(idx, s, &ix);
  if (st != QSA_OK) return st;
  if (kv_len < 0 || kv_cap <= 0 || kv_len > kv_cap || block_begin < 0) return QSA_ERR_INVALID;
  if (kv_cap > kMaxPositions) return QSA_ERR_UNSUPPORTED;
  const int64_t blk_end = kv_len / s.bs;
  if (block_begin >= blk_end) return QSA_OK;  // no complete block in range
  if (!w_k || !k_comp || !k_idx || !aligned16(w_k) || !aligned16(k_comp) || !aligned16(k_idx))
    return QSA_ERR_INVALID;
  return hip_status(qsa::launch_indexer_keys(s, ix, w_k, k_comp, kv_cap, block_begin, blk_end, k_idx,
                                             static_cast<hipStream_t>(stream)));
}

qsa_status qsa_indexer_select(const qsa_shape* shape, const qsa_indexer* idx, const float* w_q, const void* q,
                              int64_t q_len, int64_t q_pos0, const float* k_idx, int64_t kv_len, int64_t kv_cap,
                              int32_t* sel, float* sel_scores, void* ws, size_t ws_bytes, void* stream) {
  Dims s;
  qsa_status st = check_shape(shape, &s);
  if (st != QSA_OK) return st;
  qsa::IndexerDims ix;
  st = check_indexer(idx, s, &ix);
  if (st != QSA_OK) return st;
  if (q_len <= 0 || q_pos0 < 0 || kv_len != q_pos0 + q_len || kv_cap <= 0 || kv_len > kv_cap) return QSA_ERR_INVALID;
  if (!w_q || !q || !sel || !aligned16(w_q) || !aligned16(q) || !aligned16(sel)) return QSA_ERR_INVALID;
  if (sel_scores && !aligned16(sel_scores)) return QSA_ERR_INVALID;
  if (kv_cap > kMaxPositions) return QSA_ERR_UNSUPPORTED;
  if (s.top_k > 64 && qsa::max_candidates(s, kv_len) > qsa::kMaxCandLarge) return QSA_ERR_UNSUPPORTED;
  if ((int64_t)s.batch * q_len * s.hkv > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
  if (qsa::max_candidates(s, kv_len) > 0 && (!k_idx || !aligned16(k_idx))) return QSA_ERR_INVALID;
  if (s.top_k > 64) {
    // the large selection's score and list workspace, and its list launch (rows x chunks)
    const qsa::SelectPlan plan = qsa::plan_select(s, q_len, q_pos0);
    if ((int64_t)s.batch * q_len * s.hkv * plan.n_chunks > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
    if (plan.ws_bytes > 0 && (!ws || ws_bytes < plan.ws_bytes || !aligned16(ws))) return QSA_ERR_WORKSPACE;
  }
  return hip_status(qsa::launch_indexer_select(s, ix, w_q, q, q_len, q_pos0, k_idx, kv_cap, sel, sel_scores, ws,
                                               static_cast<hipStream_t>(stream)));
}

qsa_status qsa_indexer_decode_step(const qsa_shape* shape, const qsa_indexer* idx, const float* w_q,
                                   const float* w_k, const void* q, const void* k, const void* v, float* k_comp,
                                   float* k_idx, int64_t kv_len, int64_t kv_cap, int32_t* sel, float* sel_scores,
                                   void* out, void* stream) {
  Dims s;
  qsa_status st = check_shape(shape, &s);
  if (st != QSA_OK) return st;
  qsa::IndexerDims ix;
  st = check_indexer(idx, s, &ix);
  if (st != QSA_OK) return st;
  if (kv_len <= 0 || kv_cap <= 0 || kv_len > kv_cap) return QSA_ERR_INVALID;
  if (!w_q || !w_k || !q || !k || !v || !k_comp || !k_idx || !sel || !out) return QSA_ERR_INVALID;
  if (!aligned16(w_q) || !aligned16(w_k) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_comp) ||
      !aligned16(k_idx) || !aligned16(sel) || !aligned16(out))
    return QSA_ERR_INVALID;
  if (sel_scores && !aligned16(sel_scores)) return QSA_ERR_INVALID;
  if (kv_cap > kMaxPositions) return QSA_ERR_UNSUPPORTED;
  if (s.dtype != QSA_BF16 || s.top_k > 64) return QSA_ERR_UNSUPPORTED;
  return hip_status(qsa::launch_indexer_step(s, ix, w_q, w_k, q, k, v, k_comp, k_idx, kv_len, kv_cap, sel,
                                             sel_scores, out, static_cast<hipStream_t>(stream)));
}

qsa_status qsa_kv_quantize(const qsa_shape* shape, const void* k, const void* v, int64_t kv_len, int64_t kv_cap,
                           int64_t pos_begin, int8_t* k_q, int8_t* v_q, uint16_t* k_scales, uint16_t* v_scales,
                           void* stream) {
  Dims s;
  qsa_status st = check_shape(shape, &s);
  if (st != QSA_OK) return st;
  if (kv_len < 0 || kv_cap <= 0 || kv_len > kv_cap || pos_begin < 0) return QSA_ERR_INVALID;
  if (s.dtype != QSA_BF16) return QSA_ERR_UNSUPPORTED;
  if (kv_cap > kMaxPositions) return QSA_ERR_UNSUPPORTED;
  if (pos_begin >= kv_len) return QSA_OK;  // nothing in range
  if (!k || !v || !k_q || !v_q || !k_scales || !v_scales) return QSA_ERR_INVALID;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_q) || !aligned16(v_q) || !aligned16(k_scales) ||
      !aligned16(v_scales))
    return QSA_ERR_INVALID;
  if ((int64_t)s.batch * s.hkv * (kv_len - pos_begin) * 2 / 4 + 1 > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
  return hip_status(qsa::launch_kv_quantize(s, k, v, kv_cap, pos_begin, kv_len, k_q, v_q, k_scales, v_scales,
                                            static_cast<hipStream_t>(stream)));
}

qsa_status qsa_sparse_attn_decode_q8(const qsa_shape* shape, const void* q, const int8_t* k_q, const int8_t* v_q,
                                     const uint16_t* k_scales, const uint16_t* v_scales, int64_t kv_len,
                                     int64_t kv_cap, const int32_t* sel, void* out, void* ws, size_t ws_bytes,
                                     void* stream) {
  Dims s;
  qsa_status st = check_shape(shape, &s);
  if (st != QSA_OK) return st;
  if (!q || !k_q || !v_q || !k_scales || !v_scales || !sel || !out) return QSA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k_q) || !aligned16(v_q) || !aligned16(k_scales) || !aligned16(v_scales) ||
      !aligned16(sel) || !aligned16(out))
    return QSA_ERR_INVALID;
  if (kv_len <= 0 || kv_cap <= 0 || kv_len > kv_cap) return QSA_ERR_INVALID;
  if (s.dtype != QSA_BF16) return QSA_ERR_UNSUPPORTED;
  if (kv_cap > kMaxPositions) return QSA_ERR_UNSUPPORTED;
  const qsa::DecodePlan plan = qsa::plan_decode(s, kv_len, false);  // 4-wave slices at every row count
  if ((int64_t)s.batch * s.hkv * plan.n_split > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
  if (plan.ws_bytes > 0 && (!ws || ws_bytes < plan.ws_bytes || !aligned16(ws))) return QSA_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  return hip_status(qsa::launch_decode_q8(s, plan, q, k_q, v_q, k_scales, v_scales, kv_len, kv_cap, sel, out, base,
                                          base ? base + qsa::counter_bytes((int64_t)s.batch * s.hkv) : nullptr,
                                          static_cast<hipStream_t>(stream)));
}

qsa_status qsa_sparse_attn_prefill_q8(const qsa_shape* shape, const void* q, const int8_t* k_q, const int8_t* v_q,
                                      const uint16_t* k_scales, const uint16_t* v_scales, int64_t q_len,
                                      int64_t q_pos0, int64_t kv_cap, const int32_t* sel, void* out, void* ws,
                                      size_t ws_bytes, void* stream) {
  Dims s;
  qsa_status st = check_shape(shape, &s);
  if (st != QSA_OK) return st;
  if (!q || !k_q || !v_q || !k_scales || !v_scales || !sel || !out) return QSA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k_q) || !aligned16(v_q) || !aligned16(k_scales) || !aligned16(v_scales) ||
      !aligned16(sel) || !aligned16(out))
    return QSA_ERR_INVALID;
  if (q_len <= 0 || q_pos0 < 0 || kv_cap <= 0 || q_pos0 + q_len > kv_cap) return QSA_ERR_INVALID;
  if (s.dtype != QSA_BF16) return QSA_ERR_UNSUPPORTED;
  if (kv_cap > kMaxPositions) return QSA_ERR_UNSUPPORTED;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const Q8PrefillWs lay = q8_prefill_ws(s, q_len, q_pos0);
  if (lay.tiled && ws && ws_bytes >= lay.total && aligned16(ws)) {
    // the codes rotated back into bf16 rows, then the tiled bf16 kernel
    char* base = static_cast<char*>(ws);
    uint16_t* kb = reinterpret_cast<uint16_t*>(base + lay.k_off);
    uint16_t* vb = reinterpret_cast<uint16_t*>(base + lay.v_off);
    st = hip_status(qsa::launch_dequant_unrotate(s, k_q, v_q, k_scales, v_scales, kv_cap, q_pos0 + q_len, lay.n_pad,
                                                 kb, vb, hs));
    if (st != QSA_OK) return st;
    return hip_status(qsa::launch_prefill(s, qsa::plan_prefill(s, q_len, q_pos0), q, kb, vb, q_len, q_pos0,
                                          lay.n_pad, sel, out, base + lay.att_off, hs));
  }
  if ((int64_t)s.batch * q_len * s.hkv > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;  // one workgroup per row
  return hip_status(qsa::launch_prefill_q8(s, q, k_q, v_q, k_scales, v_scales, q_len, q_pos0, kv_cap, sel, out, hs));
}

qsa_status qsa_decode_step_q8(const qsa_shape* shape, const void* q, const void* k, const void* v, float* k_comp,
                              int8_t* k_q, int8_t* v_q, uint16_t* k_scales, uint16_t* v_scales, int64_t kv_len,
                              int64_t kv_cap, int32_t* sel, float* sel_scores, void* out, void* ws, size_t ws_bytes,
                              void* stream) {
  Dims s;
  qsa_status st = check_shape(shape, &s);
  if (st != QSA_OK) return st;
  if (!q || !k || !v || !k_comp || !k_q || !v_q || !k_scales || !v_scales || !sel || !out) return QSA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_comp) || !aligned16(k_q) || !aligned16(v_q) ||
      !aligned16(k_scales) || !aligned16(v_scales) || !aligned16(sel) || !aligned16(out))
    return QSA_ERR_INVALID;
  if (sel_scores && !aligned16(sel_scores)) return QSA_ERR_INVALID;
  if (kv_len <= 0 || kv_cap <= 0 || kv_len > kv_cap) return QSA_ERR_INVALID;
  if (kv_cap > kMaxPositions) return QSA_ERR_UNSUPPORTED;
  if (s.dtype != QSA_BF16) return QSA_ERR_UNSUPPORTED;  // the 8-bit cache holds bf16 rows
  const int64_t rows = (int64_t)s.batch * s.hkv;
  const qsa::StepPlan sp = qsa::plan_decode_step(s, kv_len, false, true);
  qsa::SelectPlan sel_plan{};
  qsa::DecodePlan att_plan{};
  if (sp.fused) {
    if ((rows + 7) * sp.n_split * 8 > 0x7FFFFFFF) return QSA_ERR_UNSUPPORTED;
  } else {
    if (s.top_k > 64 && qsa::max_candidates(s, kv_len) > qsa::kMaxCandLarge) return QSA_ERR_UNSUPPORTED;
    sel_plan = qsa::plan_select(s, 1, kv_len - 1);
    att_plan = qsa::plan_decode(s, kv_len, false);
    if (rows * (sel_plan.n_chunks > 0 ? sel_plan.n_chunks : 1) > 0x7FFFFFFF || rows * att_plan.n_split > 0x7FFFFFFF)
      return QSA_ERR_UNSUPPORTED;
  }
  const StepWs lay = step_ws(s, kv_len, true);
  if (lay.total > 0 && (!ws || ws_bytes < lay.total || !aligned16(ws))) return QSA_ERR_WORKSPACE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  char* part = base ? base + lay.part_off : nullptr;
  // the fused kernel writes the new position into the 8-bit cache itself;
  // the separate calls quantize it first
  if (!sp.fused) {
    st = hip_status(qsa::launch_kv_quantize(s, k, v, kv_cap, kv_len - 1, kv_len, k_q, v_q, k_scales, v_scales, hs));
    if (st != QSA_OK) return st;
  }
  if (sp.fused) {
    const qsa::Q8Cache cache{k_q, v_q, k_scales, v_scales};
    return hip_status(qsa::launch_decode_step(s, sp, q, k, v, k_comp, kv_len, kv_cap, sel, sel_scores, out, base,
                                              part, hs, nullptr, &cache));
  }
  // the other shapes (top_k > 64, blocks shorter than 32 keys): the
  // selection, which compresses the block the new token closes from the bf16
  // keys before scoring it and picks every row's blocks, then the 8-bit
  // cache's decode attention; the selection's counters (if any) sit in the
  // second counter area, the attention's in the first
  const int64_t close_block = kv_len % s.bs == 0 ? kv_len / s.bs - 1 : -1;
  st = hip_status(qsa::launch_select(s, sel_plan, q, 1, kv_len - 1, k_comp, kv_cap, sel, sel_scores,
                                     base ? base + lay.sel_off : nullptr, hs, k, close_block));
  if (st != QSA_OK) return st;
  return hip_status(qsa::launch_decode_q8(s, att_plan, q, k_q, v_q, k_scales, v_scales, kv_len, kv_cap, sel, out, base,
                                          part, hs));
}

}  // extern "C"
