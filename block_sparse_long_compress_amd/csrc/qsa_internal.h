// Host-side launch entry points shared between the C ABI layer and the
// kernel translation units. Arguments are already validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

namespace qsa {

struct Dims {
  int batch, hq, hkv, group, d, bs, top_k, dtype;
  float scale;     // resolved (never 0)
  int keep_tail;   // selection frame: 0 = own block kept, 1 = only the partial tail kept
};

// Learned-indexer variant of the selection: indexer dimension (64 or 128),
// aggregation of the group's head scores, resolved scale (never 0).
constexpr int kAggSum = 0, kAggMax = 1, kAggSoftmax = 2;
struct IndexerDims {
  int dim, agg;
  float scale;
};
// Indexer keys of blocks [blk_begin, blk_end): W_k^T k_comp per block.
hipError_t launch_indexer_keys(const Dims& s, const IndexerDims& ix, const float* w_k, const float* k_comp,
                               int64_t kv_cap, int64_t blk_begin, int64_t blk_end, float* k_idx, hipStream_t st);
// Selection of every (sequence, query row, KV head) scored in indexer space.
// top_k > 64: the scores go to ws (the large selection's layout, n_chunks =
// plan_select(s, q_len, q_pos0).n_chunks) and the large pick runs on them.
hipError_t launch_indexer_select(const Dims& s, const IndexerDims& ix, const float* w_q, const void* q,
                                 int64_t q_len, int64_t q_pos0, const float* k_idx, int64_t kv_cap, int32_t* sel,
                                 float* sel_scores, void* ws, hipStream_t st);
// One decode step with the learned indexer (bf16, top_k <= 64), one
// workgroup per (sequence, KV head): compress the block the new token at
// kv_len - 1 closes (if any) into k_comp and its indexer key into k_idx,
// select in indexer space, attend over the selection into out.
hipError_t launch_indexer_step(const Dims& s, const IndexerDims& ix, const float* w_q, const float* w_k,
                               const void* q, const void* k, const void* v, float* k_comp, float* k_idx,
                               int64_t kv_len, int64_t kv_cap, int32_t* sel, float* sel_scores, void* out,
                               hipStream_t st);

// Rotated 8-bit K/V cache: positions [pos_begin, pos_end) of every (b, g)
// rotated (Walsh-Hadamard) and quantized (codes + float16 scale per 32).
hipError_t launch_kv_quantize(const Dims& s, const void* k, const void* v, int64_t kv_cap, int64_t pos_begin,
                              int64_t pos_end, int8_t* kq, int8_t* vq, uint16_t* ks, uint16_t* vs, hipStream_t st);

// Block compression, blocks [blk_begin, blk_end) of every (b, g).
hipError_t launch_compress(const Dims& s, const void* k, int64_t kv_cap, int64_t blk_begin, int64_t blk_end,
                           float* k_comp, hipStream_t st);

// Bytes at the start of a workspace holding one arrival counter per row (of
// the decode attention, or of the split selection); they must be zero before
// the first call and every call leaves them zero.
inline size_t counter_bytes(int64_t rows) { return ((size_t)rows * 4 + 255) / 256 * 256; }

// Selection ------------------------------------------------------------------
struct SelectPlan {
  bool tiled;          // prefill-style tile path (rows share candidates); with large, the tiled score pass
  bool large;          // top_k > 64: score pass + per-row radix select
  int chunk;           // split path: candidates per chunk (multiple of 64)
  int64_t n_chunks;    // split / large path: chunks per row (the longest row's)
  int64_t grid;        // workgroups of the plan's largest launch
  size_t ws_bytes;
};
// Largest top_k of the large-k selection path (its candidate pool fits LDS).
constexpr int kMaxTopKLarge = 513;
// Largest candidate count per row of the large-k selection path.
constexpr int64_t kMaxCandLarge = 65536;
// Candidate blocks of the row at position kv_len - 1 (the most of any row).
int64_t max_candidates(const Dims& s, int64_t kv_len);
SelectPlan plan_select(const Dims& s, int64_t q_len, int64_t q_pos0);
// The large-k path's plan (score pass over 256-candidate chunks, then the
// per-row pick) for any top_k: the ragged decode step takes it for every
// shape the fused kernel does not serve.
SelectPlan plan_select_large(const Dims& s, int64_t q_len, int64_t q_pos0);
// close_block >= 0 (decode, q_len = 1): the selection also compresses that
// block of k_cache into k_comp first (the block the new token closes).
// pick = false (large path only): the score pass alone, for launch_pick_attend.
// kv_lens (device, [batch], large path with pick = false and q_len = 1 only):
// a ragged decode batch; each row's position comes from its sequence's
// length (clamped into [1, q_pos0 + 1]) and each row compresses the block
// its own new token closes (close_block is then ignored).
hipError_t launch_select(const Dims& s, const SelectPlan& plan, const void* q, int64_t q_len, int64_t q_pos0,
                         const float* k_comp, int64_t kv_cap, int32_t* sel, float* sel_scores, void* ws,
                         hipStream_t st, const void* k_cache = nullptr, int64_t close_block = -1,
                         bool pick = true, const int32_t* kv_lens = nullptr);

// The large selection's pick over scores already in ws (scores of rows x
// n_chunks x 256 candidates, then the chunk lists): lists = true first
// rebuilds the chunk lists from the scores where a row's candidates exceed
// the pick pool (a score pass that wrote scores only).
hipError_t launch_large_pick(const Dims& s, int64_t q_len, int64_t q_pos0, int64_t n_chunks, void* ws, bool lists,
                             int32_t* sel, float* sel_scores, hipStream_t st);

// Decode attention --------------------------------------------------------------
struct DecodePlan {
  int waves;  // per workgroup: 4, or 8 with one slice per row when the rows fill the GPU
  int blocks_per_wg;
  int n_split;
  size_t ws_bytes;
};
// wide = false keeps 4-wave slices for every row count (the 8-bit cache
// decode, whose waves keep one unit in flight and so want more workgroups).
// The decode workspace is sized by the narrow plan, which covers both.
DecodePlan plan_decode(const Dims& s, int64_t kv_len, bool wide = true);

// counters: the plan's arrival counters (counter_bytes(rows), zero between
// calls); part: its slice states (ws_bytes past the counters). The decode
// call keeps both in one workspace, the decode step at separate places.
// kv_lens (device, [batch], nullable): per-sequence lengths, each clamped
// into [1, kv_len] (the causal bound of sequence b's token); null means every
// sequence has kv_len.
hipError_t launch_decode(const Dims& s, const DecodePlan& plan, const void* q, const void* k, const void* v,
                         int64_t kv_len, int64_t kv_cap, const int32_t* sel, void* out, void* counters, void* part,
                         hipStream_t st, const int32_t* kv_lens = nullptr);
// Prefill attention over the rotated 8-bit cache, one workgroup per query
// row (any top_k and block size); no workspace.
// The 8-bit cache's positions [0, n_pos) of every (sequence, KV head),
// dequantized and rotated back into bf16 rows k_out, v_out ([b][Hkv][n_pad][d],
// rows [n_pos, n_pad) zero), for the tiled prefill kernel.
hipError_t launch_dequant_unrotate(const Dims& s, const int8_t* kq, const int8_t* vq, const uint16_t* ks,
                                  const uint16_t* vs, int64_t kv_cap, int64_t n_pos, int64_t n_pad, uint16_t* k_out,
                                  uint16_t* v_out, hipStream_t st);
hipError_t launch_prefill_q8(const Dims& s, const void* q, const int8_t* kq, const int8_t* vq, const uint16_t* ks,
                             const uint16_t* vs, int64_t q_len, int64_t q_pos0, int64_t kv_cap, const int32_t* sel,
                             void* out, hipStream_t st);
// Decode attention over the rotated 8-bit cache (the narrow plan; counters
// and slice states as for launch_decode).
hipError_t launch_decode_q8(const Dims& s, const DecodePlan& plan, const void* q, const int8_t* kq, const int8_t* vq,
                            const uint16_t* ks, const uint16_t* vs, int64_t kv_len, int64_t kv_cap,
                            const int32_t* sel, void* out, void* counters, void* part, hipStream_t st);

// Prefill attention -------------------------------------------------------------
struct PrefillPlan {
  bool rows;        // bf16 shapes the tiled kernel does not serve: one workgroup per query row
  int rows_per_wg;
  size_t ws_bytes;
};
PrefillPlan plan_prefill(const Dims& s, int64_t q_len, int64_t q_pos0);
// bf16 prefill one query row per workgroup (decode unit loop, causal at the
// row's position, any block size, any top_k); no workspace.
hipError_t launch_prefill_rows(const Dims& s, const void* q, const void* k, const void* v, int64_t q_len,
                               int64_t q_pos0, int64_t kv_cap, const int32_t* sel, void* out, hipStream_t st);
hipError_t launch_prefill(const Dims& s, const PrefillPlan& plan, const void* q, const void* k, const void* v,
                          int64_t q_len, int64_t q_pos0, int64_t kv_cap, const int32_t* sel, void* out, void* ws,
                          hipStream_t st);

// Fused decode step (compress the closed block, select, attend) --------------
// Whether the fused kernel serves this shape (otherwise the step runs as the
// separate compress, selection and decode launches), and with how many
// workgroups (slices of the selection) per row.
struct StepPlan {
  bool fused;
  int blocks_per_wg;
  int n_split;  // workgroups attending over slices of a row's selection
  int n_scan;   // workgroups scanning shares of a row's candidates (n_split == 1)
  int n_attend; // of those, the ones attending over a slice of the selection each
  size_t ws_bytes;
};
// ragged: a batch of sequences of their own lengths (kv_len is then the
// longest), which always runs fused when the kernel serves the shape.
StepPlan plan_decode_step(const Dims& s, int64_t kv_len, bool ragged = false, bool q8 = false);
// kv_lens (device, [batch], nullable): per-sequence lengths, each clamped
// into [1, kv_len]; null means every sequence has kv_len.
// counters / part: as for launch_decode (used when plan.n_split > 1). q8:
// attend over the rotated 8-bit cache instead of k and v (compression and
// selection still read k); Bs >= 32.
// A quantized K/V cache (8-bit codes, one float16 scale per 32 values of a
// row: value = code * scale), read by attend_units<..., true> in place of
// the bf16 cache; the values are widened to bf16 operands on load.
struct Q8Cache {
  const int8_t* k;     // codes [positions][D] of the row's keys
  const int8_t* v;     // codes of its values
  const uint16_t* ks;  // float16 scales [positions][D/32]
  const uint16_t* vs;
};

hipError_t launch_decode_step(const Dims& s, const StepPlan& plan, const void* q, const void* k, const void* v,
                              float* k_comp, int64_t kv_len, int64_t kv_cap, int32_t* sel, float* sel_scores,
                              void* out, void* counters, void* part, hipStream_t st,
                              const int32_t* kv_lens = nullptr, const Q8Cache* q8 = nullptr);

// Decode step with k > 64 (bf16): the selection's score pass, then one kernel
// that picks each row's ids and attends over them (S workgroups per row).
struct PickAttendPlan {
  int blocks_per_wg;
  int n_split;
  int64_t n_chunks;  // of the score pass
  size_t ws_bytes;   // arrival counters (counter_bytes(rows)), then slice states
};
PickAttendPlan plan_pick_attend(const Dims& s, int64_t n_chunks);
// counters / part: as for launch_decode. kv_lens (device, [batch], nullable):
// a ragged batch, each sequence at its own length (clamped into [1, kv_len]).
hipError_t launch_pick_attend(const Dims& s, const PickAttendPlan& pa, const void* q, const void* k, const void* v,
                              int32_t* sel, float* sel_scores, const void* ws_select, void* out, void* counters,
                              void* part, int64_t kv_len, int64_t kv_cap, hipStream_t st,
                              const int32_t* kv_lens = nullptr);

// Generic float32 attention (one wave per query row); used for dtype QSA_F32.
// kv_lens (q_len = 1): per-sequence lengths of a ragged decode batch.
hipError_t launch_attn_f32(const Dims& s, const float* q, const float* k, const float* v, int64_t q_len,
                           int64_t q_pos0, int64_t kv_cap, const int32_t* sel, float* out, hipStream_t st,
                           const int32_t* kv_lens = nullptr);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Raises kernel Fn's dynamic LDS limit to `bytes`, once per device: the
// attribute is set for the device current at the call, so a process that
// drives several GPUs sets it on each of them before the kernel's first
// launch there. Returns the result of that device's call.
template <auto Fn>
hipError_t allow_dynamic_lds(int bytes) {
  constexpr int kDevices = 64;
  static std::once_flag once[kDevices];
  static hipError_t err[kDevices];
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev, bytes] {
    err[dev] = hipFuncSetAttribute(reinterpret_cast<const void*>(Fn), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  });
  return err[dev];
}

}  // namespace qsa
