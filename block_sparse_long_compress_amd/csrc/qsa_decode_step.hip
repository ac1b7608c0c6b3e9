// One whole decode step per (sequence, KV head) in one workgroup: compress the
// block the new token completed, score the compressed blocks and keep the
// top-k ("Qwen4 in llama.cpp: Dissecting PR #27742", section "QSA Is an
// Address-Selection Problem, Not a New Attention Equation": compressed-block
// scoring, top-k, cache addresses), then attend over the kept blocks (same
// section: ordinary attention over the selected cells).
//
// The separate calls hand the selection from kernel to kernel through HBM
// and pay a launch and a cold read at each hand-off; for rows of a few
// thousand candidates those latencies dominate the step. Here the 8 waves of
// a workgroup stream the row's compressed keys (64 per wave-step, the
// selection kernels' coalesced dot products) into per-wave top lists, merge
// them in LDS, write the row's selection, and attend over it from LDS with the
// decode kernels' unit loop; the waves' softmax states merge in LDS. When
// the rows alone leave most of the GPU idle, each row gets S workgroups:
// every one of them computes the (cheap) selection itself, attends over its
// own slice of it, and the last to finish merges the S partial states
// through the workspace exactly as the decode kernel merges its slices.
// Selections equal the separate calls' (same arithmetic); outputs agree
// within rounding (another merge order of the attention states).
#include <cstdlib>

#include "qsa_decode_unit.h"
#include "qsa_device.h"
#include "qsa_internal.h"
#include "qsa_select_large.h"
#include "qsa_select_wave.h"

namespace qsa {
namespace {

constexpr int kStepWaves = 8;
// Polls of a scan part waiting for the other parts' lists (each poll an
// atomic load and a short sleep, well under a microsecond) before it scores
// their candidates itself: far beyond the few microseconds parts that run
// together take, and a bound on the wait when a partner is not yet running.
// The environment variable QSA_SCAN_WAIT_POLLS overrides it (tests set 0 to
// drive every part through the fallback).
constexpr int kScanWaitPolls = 4096;
int scan_wait_polls() {
  const char* e = getenv("QSA_SCAN_WAIT_POLLS");
  if (!e || !*e) return kScanWaitPolls;
  const long v = strtol(e, nullptr, 10);
  return v < 0 ? 0 : (v > (1 << 20) ? (1 << 20) : (int)v);
}

template <int D, bool ROT = false>
struct StepSmem {
  static constexpr int RS = kStageRowBytes<D>;
  static constexpr int kStage = kStepWaves * kUnit * RS;  // V staging, one 32-row slice per wave
  // the waves' softmax states (and, rotated cache, the workgroup's combined one)
  static constexpr int kComb = (kStepWaves + (ROT ? 1 : 0)) * (32 + 16 * kCombStride<D>) * 4;
  static constexpr int kBytes = kStage > kComb ? kStage : kComb;
};

// Q8: the attention reads the rotated 8-bit cache (q8: codes and scales of
// every row, [b][Hkv][kv_cap] like k and v); the query heads are rotated
// first and the output rotated back. Compression and selection still read
// the bf16 keys.
template <int D, int BS, bool Q8 = false>
__global__ __launch_bounds__(kStepWaves * kWave) void decode_step_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    float* __restrict__ k_comp, int32_t* __restrict__ sel, float* __restrict__ sel_scores, uint16_t* __restrict__ out,
    float* __restrict__ part_ws, uint32_t* __restrict__ counters, uint32_t* __restrict__ scan_tickets,
    const int32_t* __restrict__ kv_lens,
    int64_t kv_len_max, int64_t kv_cap, int hq, int hkv, int G, int top_k, float scale, int keep_tail, int bpw,
    int n_split, int n_scan, int n_attend, int wait_polls, int64_t n_rows, Q8Cache q8) {
  using SM = StepSmem<D, Q8>;
  constexpr int LPR = D / 4;  // lanes covering one compressed key row (float32)
  constexpr int DT = D / 16;
  __shared__ __align__(16) unsigned char big[SM::kBytes];
  __shared__ uint64_t lists[kStepWaves][kWave];
  __shared__ __align__(16) float knew[D];
  __shared__ int ids[kWave];
  __shared__ int last_wg;
  __shared__ __align__(16) uint16_t qrot[Q8 ? 16 * D : 8];  // rotated query heads (bf16)

  // Several slices per row: all slices of a row on one XCD (workgroups go
  // to the 8 XCDs round-robin), so that they share its L2 copy of the row's
  // compressed keys; grid slots past the last row exit at once.
  // Several scan parts per row (n_scan > 1: rows that fill a fraction of
  // the GPU, or long rows): part j scores the j-th share of the row's
  // candidates, the parts exchange their top lists (2b), and the first
  // n_attend parts each attend over a slice of the selection.
  int64_t row;
  int split = 0, part = 0;
  if (n_split > 1) {
    const int64_t slot = blockIdx.x / 8;
    row = (int64_t)(blockIdx.x % 8) + 8 * (slot / n_split);
    split = (int)(slot % n_split);
    if (row >= n_rows) return;
  } else if (n_scan > 1) {
    row = blockIdx.x / n_scan;
    part = (int)(blockIdx.x % n_scan);
  } else {
    row = blockIdx.x;
  }
  const int64_t b = row / hkv;
  const int g = (int)(row % hkv);
  const int lane = lane_id(), w = wave_id();
  // this sequence's length: one for the batch, or its own (ragged batch,
  // clamped into [1, kv_len_max] so that every access stays in bounds)
  int64_t kv_len = kv_len_max;
  if (kv_lens) {
    const int64_t n = kv_lens[b];
    kv_len = n < 1 ? 1 : (n > kv_len_max ? kv_len_max : n);
  }
  const int64_t p = kv_len - 1;
  const Frame fr = row_frame(p, BS, keep_tail);
  const int slots = frame_slots(fr, top_k);
  const int64_t nb_cap = kv_cap / BS;
  const int64_t kv_off = ((int64_t)b * hkv + g) * kv_cap;
  const uint16_t* q_heads = q + (b * hq + (int64_t)g * G) * D;
  float* kc_row = k_comp + ((int64_t)b * hkv + g) * nb_cap * D;

  // 1. the block completed by the new token (if any): its mean goes to
  // k_comp for later steps and, with keep_tail (where it is a candidate of
  // this step), to LDS first. A wave computes it as the compression kernel
  // does. In the default frame it is the token's own block, never a
  // candidate: with several slices per row, slice 0 stores it during the
  // attention phase instead, off the scan's critical path (see 3.).
  const bool closes = kv_len % BS == 0;
  const int c_new = (int)(kv_len / BS) - 1;
  const bool new_is_cand = closes && c_new < fr.n_cand;
  auto compress_new = [&](bool to_lds) {
    constexpr int VEC = 8;             // bf16 per 16-byte load
    constexpr int LPK = D / VEC;       // lanes covering one key row
    constexpr int RPL = kWave / LPK;   // rows per wave-wide load
    constexpr int NLOAD = BS / RPL;
    const int r0 = lane / LPK, c0 = (lane % LPK) * VEC;
    const uint16_t* src = k + (kv_off + (int64_t)c_new * BS + r0) * D + c0;
    u32x4_t raw[NLOAD];
#pragma unroll
    for (int j = 0; j < NLOAD; ++j) raw[j] = *reinterpret_cast<const u32x4_t*>(src + (int64_t)j * RPL * D);
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
    for (int j = 0; j < NLOAD; ++j)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        acc[2 * h] += bf16_lo(raw[j][h]);
        acc[2 * h + 1] += bf16_hi(raw[j][h]);
      }
#pragma unroll
    for (int m = LPK; m < kWave; m <<= 1)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += shfl_xor_f32(acc[e], m);
    if (r0 == 0) {
      constexpr float inv = 1.0f / BS;
      float* dst = kc_row + (int64_t)c_new * D + c0;
#pragma unroll
      for (int e = 0; e < VEC; e += 4) {
        const f32x4_t val = {acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
        if (split == 0 && part == n_scan - 1) *reinterpret_cast<f32x4_t*>(dst + e) = val;
        if (to_lds) *reinterpret_cast<f32x4_t*>(&knew[c0 + e]) = val;
      }
    }
  };
  // deferred when the row has slices: slice 0's last wave then holds few or
  // no attention units (with one slice per row every wave has units, and the
  // compression measured cheaper here, during the scan)
  const bool defer_new = closes && !new_is_cand && n_split > 1;
  // slice 0 (the last scan part) stores it
  if (closes && !defer_new && w == kStepWaves - 1 && part == n_scan - 1) compress_new(new_is_cand);

  // 2. scores and the top list of each wave (candidates read from k_comp; the
  // new block, when it competes, from LDS below)
  const f32x4_t qv = group_sum4(q_heads + 4 * (lane % LPR), G, D);
  const int64_t n_glob = fr.n_cand - (new_is_cand ? 1 : 0);
  int64_t c_lo = 0, c_hi = n_glob;  // this part's candidates
  const int64_t per_part = ((n_glob + n_scan - 1) / n_scan + kWave - 1) / kWave * kWave;
  if (n_scan > 1) {
    c_lo = part * per_part < n_glob ? part * per_part : n_glob;
    c_hi = c_lo + per_part < n_glob ? c_lo + per_part : n_glob;
  }
  uint64_t cur = 0ull;
  auto scan = [&](int64_t lo, int64_t hi) {
    for (int64_t base = lo + (int64_t)kWave * w; base < hi; base += kWave * kStepWaves) {
      const float s = dot64_rows<D>(kc_row + base * D, hi - base, qv);
      const int64_t cand = base + dot64_row<D>(lane);
      cur = topk_fold(cur, cand < hi ? make_key(s * scale, (int)cand) : 0ull, slots);
    }
  };
  if (slots > 0) scan(c_lo, c_hi);
  __syncthreads();  // knew written
  if (new_is_cand && slots > 0 && w == 0 && part == n_scan - 1) {
    float part = qv[0] * knew[4 * (lane % LPR)] + qv[1] * knew[4 * (lane % LPR) + 1] +
                 qv[2] * knew[4 * (lane % LPR) + 2] + qv[3] * knew[4 * (lane % LPR) + 3];
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) part += xor_lane_f32(part, m);
    cur = topk_fold(cur, lane == 0 ? make_key(part * scale, c_new) : 0ull, slots);
  }
  cur = merge_wave_lists<kStepWaves>(lists, cur, slots > 0 ? slots : 1);

  // 2b. several scan parts: every part posts its top list (descending keys)
  // to the workspace and counts itself in the row's ticket word (low 16
  // bits: parts posted), then waits, bounded, until every part has posted,
  // and merges every list: all parts hold the same selection. A part that
  // times out (a partner not yet running) scores the other parts'
  // candidates itself instead, with the same result. Each part then counts
  // itself done (high 16 bits); the part completing that count resets the
  // word for the next call (by then every part has stopped polling it).
  // Hand-off: the lists are written with device-coherent (sc1) stores, which
  // go through the XCD's L2 to the device-coherent level, and the posting
  // wave waits for them to complete (s_waitcnt) before it issues the
  // ticket's atomic, which is itself performed at the device-coherent level.
  // A part that observes another part's count has therefore observed an
  // atomic issued after that part's stores were complete, and it reads the
  // lists with sc1 loads, served from the device-coherent level and not from
  // a stale L2 line of its own XCD. No release/acquire fence is needed (an
  // agent-scope release would write back the whole L2).
  if (n_scan > 1) {
    uint32_t* scan_word = scan_tickets + row;
    const auto lrs = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<uint32_t*>(part_ws) + row * n_scan * 2 * kWave,
                                                       0, n_scan * 2 * kWave * 4, kBufferFlags);
    const bool attends = part < n_attend;
    if (w == 0) {
      if (slots > 0 && lane < slots)
        store2_coherent(lrs, 2 * (part * kWave + lane), (uint32_t)cur, (uint32_t)(cur >> 32));
      __builtin_amdgcn_s_waitcnt(0);  // this wave's list stores have completed
      if (lane == 0 && !attends) {
        // a part that does not attend is done once its list is posted
        const uint32_t prev = __hip_atomic_fetch_add(scan_word, 1u | (1u << 16), __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if ((int)(prev >> 16) + 1 == n_scan) __hip_atomic_store(scan_word, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (lane == 0 && attends) {
        uint32_t seen = __hip_atomic_fetch_add(scan_word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
        for (int poll = 0; (int)(seen & 0xFFFFu) < n_scan && poll < wait_polls; ++poll) {
          __builtin_amdgcn_s_sleep(2);
          seen = __hip_atomic_load(scan_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        last_wg = (int)(seen & 0xFFFFu) >= n_scan ? 1 : 0;  // 1: every list posted
      }
    }
    if (!attends) return;
    __syncthreads();
    // wave 0 keeps this part's merged list; the other waves (whose lists are
    // in it already) start afresh and fold the other parts' lists, or score
    // their candidates, and the waves' lists merge below
    if (w != 0) cur = 0ull;
    if (last_wg) {
      if (slots > 0) {
        // the other parts' lists, several loads in flight per wave, then folded
        constexpr int kLoads = 4;
        for (int j0 = w; j0 < n_scan; j0 += kStepWaves * kLoads) {
          u32x2_t x[kLoads];
#pragma unroll
          for (int i = 0; i < kLoads; ++i) {
            const int j = j0 + i * kStepWaves;
            x[i] = (j < n_scan && j != part && lane < slots) ? load2_coherent(lrs, 2 * (j * kWave + lane))
                                                           : u32x2_t{0u, 0u};
          }
#pragma unroll
          for (int i = 0; i < kLoads; ++i) cur = topk_fold_sorted(cur, ((uint64_t)x[i][1] << 32) | x[i][0], slots);
        }
      }
    } else {
      // the other parts' candidates, scored here (and the closed block when
      // it competes: the last part scores it from LDS, so recompute it here)
      if (slots > 0) {
        for (int j = 0; j < n_scan; ++j) {
          if (j == part) continue;
          const int64_t lo = j * per_part < n_glob ? j * per_part : n_glob;
          scan(lo, lo + per_part < n_glob ? lo + per_part : n_glob);
        }
        if (new_is_cand && part != n_scan - 1 && w == kStepWaves - 1) compress_new(true);
      }
      __syncthreads();
      if (new_is_cand && slots > 0 && w == 0 && part != n_scan - 1) {
        float dp = qv[0] * knew[4 * (lane % LPR)] + qv[1] * knew[4 * (lane % LPR) + 1] +
                   qv[2] * knew[4 * (lane % LPR) + 2] + qv[3] * knew[4 * (lane % LPR) + 3];
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1) dp += xor_lane_f32(dp, m);
        cur = topk_fold(cur, lane == 0 ? make_key(dp * scale, c_new) : 0ull, slots);
      }
    }
    cur = merge_wave_lists<kStepWaves>(lists, cur, slots > 0 ? slots : 1);
    if (w == 0 && lane == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(scan_word, 1u << 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((int)(prev >> 16) + 1 == n_scan) __hip_atomic_store(scan_word, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (w == 0) {
    // every slice holds the same selection; slice 0 writes it out
    const int64_t off = row * top_k;
    if (split == 0 && part == 0)
      finalize_row(cur, slots, fr.forced, top_k, sel + off, sel_scores ? sel_scores + off : nullptr, ids);
    else finalize_row(cur, slots, fr.forced, top_k, nullptr, nullptr, ids);
  }
  __syncthreads();

  // 3. attention over the selection, units round-robin over the waves
  u32x4_t qf[D / 32];
  if constexpr (Q8) {
    // The new token's K and V rows into the 8-bit cache (the caller's cache
    // is writable; only this step kernel writes through these pointers). The
    // slice that attends the token's block writes them, so its own waves read
    // them back after the barrier below: stores and loads of one CU, with the
    // stores complete in L2 before the barrier and no line of these rows in
    // the CU's L1 before them (the kernel reads the cache only in the
    // attention). When no slice attends that block (a complete block that
    // lost the selection in the keep-tail frame) slice 0 writes them, for
    // later steps.
    {
      const int own_blk = (int)(p / BS);
      const int sl = n_scan > 1 ? part : split;
      const int e0w = sl * bpw;
      const int n_w = top_k - e0w < bpw ? top_k - e0w : bpw;  // top_k <= 64 in this kernel
      const unsigned long long hit = __ballot(lane < top_k && ids[lane] == own_blk);
      const int at = hit != 0ull ? __builtin_ctzll(hit) : -1;
      const bool writer = at >= 0 ? (at >= e0w && at < e0w + n_w) : sl == 0;
      if (writer && w < 2) {
        const int64_t ro = (kv_off + p) * D;
        quantize_row_wave<D>((w == 0 ? k : v) + ro, const_cast<int8_t*>(w == 0 ? q8.k : q8.v) + ro,
                             const_cast<uint16_t*>(w == 0 ? q8.ks : q8.vs) + (kv_off + p) * (D / 32));
        __builtin_amdgcn_s_waitcnt(0);
      }
    }
    // (H q).(H k) = D q.k: the 1/D goes into the scale below
    constexpr int EPL = D / kWave;
    for (int h = w; h < G; h += kStepWaves) {
      float x[EPL];
#pragma unroll
      for (int i = 0; i < EPL; ++i) x[i] = bf16_to_f32(q_heads[(int64_t)h * D + lane + kWave * i]);
      fwht_wave<D>(x);
#pragma unroll
      for (int i = 0; i < EPL; ++i) qrot[h * D + lane + kWave * i] = f32_to_bf16(x[i]);
    }
    __syncthreads();
    load_q8_query_operands<D>(qrot, G, qf);
  } else {
    load_q_operands<D>(q_heads, G, qf);
  }
  // the attention slice: a scan part attends over its share of the selection
  const int slice = n_scan > 1 ? part : split, n_slices = n_scan > 1 ? n_attend : n_split;
  const int e0 = slice * bpw;
  const int n_e = top_k - e0 < bpw ? top_k - e0 : bpw;  // this slice's entries of the selection
  const int sel_mine = lane < n_e ? ids[e0 + lane] : -1;
  float m_run = -__builtin_inff(), l_run = 0.f;
  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the closed block of the default frame (not a candidate) when deferred:
  // stored by slice 0's last wave, which holds the fewest units of the slice
  if (defer_new && split == 0 && w == kStepWaves - 1) compress_new(false);
  const float scale_log2 = scale * 1.4426950408889634f / (Q8 ? (float)D : 1.0f);
  const Q8Cache rq = Q8 ? Q8Cache{q8.k + kv_off * D, q8.v + kv_off * D, q8.ks + kv_off * (D / 32),
                                  q8.vs + kv_off * (D / 32)}
                        : q8;
  attend_units<D, false, Q8>(qf, k + kv_off * D, v + kv_off * D, sel_mine, n_e, BS, p, scale_log2,
                             big + w * kUnit * SM::RS, w, kStepWaves, m_run, l_run, o, rq);
  l_run = sum_col4(l_run);
  float* states = n_scan > 1 ? part_ws + n_rows * n_scan * 2 * kWave : part_ws;  // [row][n_attend] states
  finish_row_slice<D, kStepWaves, Q8>(m_run, l_run, o, big, &last_wg, out, states, counters, row, b, g, hq, G, slice,
                                      n_slices);
}

// Decode step with k > 64 (the released budget): after the large-k score
// pass, each of a row's S workgroups takes the row's cutoff and ids itself
// (pick_row over the stored scores and chunk lists; slice 0 also writes
// them out), attends over its slice of the selection, and the last slice
// merges. The selection reaches the attention through LDS, not through HBM
// and another launch.
static_assert(kPickThreads == kStepWaves * kWave, "the pick runs on the step's workgroup");

template <int D, bool GATHER>
__global__ __launch_bounds__(kStepWaves * kWave) void pick_attend_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int32_t* __restrict__ sel, float* __restrict__ sel_scores, const uint32_t* __restrict__ ws_scores,
    const uint64_t* __restrict__ ws_lists, uint16_t* __restrict__ out, float* part, uint32_t* counters,
    const int32_t* __restrict__ kv_lens, int64_t kv_len, int64_t kv_cap, int hq, int hkv, int G, int bs, int top_k,
    float scale_log2, int keep_tail, int64_t n_chunks, int bpw, int n_split) {
  using SM = StepSmem<D>;
  constexpr int DT = D / 16;
  __shared__ __align__(16) unsigned char big[SM::kBytes];
  __shared__ PickSmem sm;
  __shared__ int ids[kMaxTopKLarge];
  __shared__ int last_wg;

  const int64_t row = blockIdx.x / n_split;
  const int split = (int)(blockIdx.x % n_split);
  const int64_t b = row / hkv;
  const int g = (int)(row % hkv);
  const int lane = lane_id(), w = wave_id();
  // this sequence's length: the batch's, or its own (ragged batch, clamped
  // into [1, kv_len] as the score pass clamps it)
  int64_t n = kv_len;
  if (kv_lens) {
    n = kv_lens[b];
    n = n < 1 ? 1 : (n > kv_len ? kv_len : n);
  }
  const int64_t p = n - 1;
  const Frame fr = row_frame(p, bs, keep_tail);
  const int64_t off = row * top_k;
  pick_row(sm, ws_scores + row * n_chunks * kLargeChunk, ws_lists + row * n_chunks * kLargeList, fr.n_cand,
           frame_slots(fr, top_k), fr.forced, top_k, split == 0 ? sel + off : nullptr,
           (split == 0 && sel_scores) ? sel_scores + off : nullptr, ids);
  __syncthreads();

  const int64_t kv_off = ((int64_t)b * hkv + g) * kv_cap;
  u32x4_t qf[D / 32];
  load_q_operands<D>(q + (b * hq + (int64_t)g * G) * D, G, qf);
  const int e0 = split * bpw;
  const int n_e = top_k - e0 < bpw ? top_k - e0 : bpw;
  const int sel_mine = lane < n_e ? ids[e0 + lane] : -1;
  float m_run = -__builtin_inff(), l_run = 0.f;
  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  attend_units<D, GATHER>(qf, k + kv_off * D, v + kv_off * D, sel_mine, n_e, bs, p, scale_log2,
                          big + w * kUnit * SM::RS, w, kStepWaves, m_run, l_run, o);
  l_run = sum_col4(l_run);
  finish_row_slice<D, kStepWaves>(m_run, l_run, o, big, &last_wg, out, part, counters, row, b, g, hq, G, split,
                                  n_split);
}

template <int D>
hipError_t launch_pick_attend_d(const Dims& s, const PickAttendPlan& pa, const void* q, const void* k, const void* v,
                                int32_t* sel, float* sel_scores, const uint32_t* ws_scores, const uint64_t* ws_lists,
                                void* out, uint32_t* counters, float* part, int64_t kv_len, int64_t kv_cap,
                                const int32_t* kv_lens, hipStream_t st) {
  const int64_t rows = (int64_t)s.batch * s.hkv;
  if (pa.n_split == 1) part = nullptr;
  auto kern = s.bs < kUnit ? pick_attend_kernel<D, true> : pick_attend_kernel<D, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)(rows * pa.n_split)), dim3(kStepWaves * kWave), 0, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), sel, sel_scores, ws_scores, ws_lists,
                     static_cast<uint16_t*>(out), part, counters, kv_lens, kv_len, kv_cap, s.hq, s.hkv, s.group, s.bs,
                     s.top_k, s.scale * 1.4426950408889634f, s.keep_tail, pa.n_chunks, pa.blocks_per_wg, pa.n_split);
  return hipGetLastError();
}

template <int D, bool Q8>
hipError_t launch_step_d(const Dims& s, const StepPlan& plan, const void* q, const void* k, const void* v,
                         float* k_comp, int64_t kv_len, int64_t kv_cap, int32_t* sel, float* sel_scores, void* out,
                         uint32_t* counters, float* part, const int32_t* kv_lens, const Q8Cache& q8,
                         hipStream_t st) {
  const int64_t rows = (int64_t)s.batch * s.hkv;
  const int64_t n_wg = plan.n_split > 1 ? 8 * ((rows + 7) / 8) * plan.n_split : rows * plan.n_scan;
  const dim3 grid((unsigned)n_wg), block(kStepWaves * kWave);
  if (plan.n_split == 1 && plan.n_scan == 1) part = nullptr;
  const auto* qp = static_cast<const uint16_t*>(q);
  const auto* kp = static_cast<const uint16_t*>(k);
  const auto* vp = static_cast<const uint16_t*>(v);
  auto* op = static_cast<uint16_t*>(out);
  auto kern = s.bs == 32 ? decode_step_kernel<D, 32, Q8>
                         : (s.bs == 64 ? decode_step_kernel<D, 64, Q8> : decode_step_kernel<D, 128, Q8>);
  if (s.bs != 32 && s.bs != 64 && s.bs != 128) return hipErrorInvalidValue;
  // the scan tickets: the second arrival-counter area of the step's workspace
  uint32_t* scan_tickets = counters ? counters + counter_bytes(rows) / 4 : nullptr;
  hipLaunchKernelGGL(kern, grid, block, 0, st, qp, kp, vp, k_comp, sel, sel_scores, op, part, counters, scan_tickets,
                     kv_lens,
                     kv_len, kv_cap, s.hq, s.hkv, s.group, s.top_k, s.scale, s.keep_tail, plan.blocks_per_wg,
                     plan.n_split, plan.n_scan, plan.n_attend, plan.n_scan > 1 ? scan_wait_polls() : 0, rows, q8);
  return hipGetLastError();
}

}  // namespace

StepPlan plan_decode_step(const Dims& s, int64_t kv_len, bool ragged, bool q8) {
  (void)ragged;
  StepPlan p{};
  p.fused = false;
  if (s.dtype != 1 || s.top_k > 64 || s.bs < 32) return p;
  p.fused = true;
  const int64_t rows = (int64_t)s.batch * s.hkv;
  const int64_t cand = max_candidates(s, kv_len);
  const bool long_rows = cand * s.d * 4 > (512 << 10);  // compressed keys of a row beyond 512 KiB
  p.blocks_per_wg = s.top_k;
  p.n_split = 1;
  p.n_scan = 1;
  p.n_attend = 1;
  // Few short rows: slices of the selection down to one block per
  // workgroup, as long as the grid stays within 256 workgroups. Every slice
  // repeats the (L2-resident) scan; more, shorter slices still measured
  // faster at 32K positions (1, 2, 4, 8, 16 slices per row: 24.1, 22.3,
  // 18.4, 17.3, 17.1 us per step), since the attention's latency chain
  // shortens.
  if (rows <= 32 && !long_rows) {
    const int cap = (int)(256 / rows);
    const int n = s.top_k < cap ? s.top_k : cap;
    if (n > 1) {
      p.blocks_per_wg = (s.top_k + n - 1) / n;
      p.n_split = (s.top_k + p.blocks_per_wg - 1) / p.blocks_per_wg;
    }
  }
  if (q8 && rows > 32 && !long_rows) {
    // over the 8-bit cache the attention phase is latency-bound (each unit
    // waits for its codes, then widens them): two slices per row, each
    // rescanning the row's compressed keys, measured 48.6 us against 54.2 us
    // per 64 x 128K step (four slices: 74 us)
    p.blocks_per_wg = (s.top_k + 1) / 2;
    p.n_split = (s.top_k + p.blocks_per_wg - 1) / p.blocks_per_wg;
  }
  if (p.n_split == 1 && rows < 256 && (!q8 || long_rows)) {
    // Rows that leave CUs idle with one workgroup each, or that are long:
    // split every row's candidate scan over several workgroups (at least
    // 256 candidates each, at most 64 per row and one round of the GPU's 256
    // CUs), which exchange their top lists. The first n_attend of them
    // attend over a share of the selection each: as many as give every
    // wave of a workgroup one 32-key unit (8 units), so that the slices to
    // merge stay few; the others are done once their list is posted.
    int64_t n = 256 / rows;
    const int64_t by_cand = (cand + 255) / 256;
    if (by_cand < n) n = by_cand;
    if (n > 64) n = 64;
    if (n > 1) {
      p.n_scan = (int)n;
      const int per_slice = (8 * kUnit + s.bs - 1) / s.bs;  // blocks giving every wave one unit
      int n_att = (s.top_k + per_slice - 1) / per_slice;
      if (n_att > p.n_scan) n_att = p.n_scan;
      p.n_attend = n_att;
      p.blocks_per_wg = (s.top_k + n_att - 1) / n_att;
    }
  }
  p.ws_bytes = p.n_split > 1 ? counter_bytes(rows) +
                                   (size_t)rows * p.n_split * (2 * s.group + s.group * s.d) * sizeof(float)
                             : 0;
  if (p.n_scan > 1)  // the lists, then the slice states
    p.ws_bytes = counter_bytes(rows) + (size_t)rows * p.n_scan * kWave * sizeof(uint64_t) +
                 (size_t)rows * p.n_attend * (2 * s.group + s.group * s.d) * sizeof(float);
  return p;
}

hipError_t launch_decode_step(const Dims& s, const StepPlan& plan, const void* q, const void* k, const void* v,
                              float* k_comp, int64_t kv_len, int64_t kv_cap, int32_t* sel, float* sel_scores,
                              void* out, void* counters, void* part, hipStream_t st, const int32_t* kv_lens,
                              const Q8Cache* q8) {
  uint32_t* c = static_cast<uint32_t*>(counters);
  float* pt = static_cast<float*>(part);
  if (q8)
    return s.d == 64 ? launch_step_d<64, true>(s, plan, q, k, v, k_comp, kv_len, kv_cap, sel, sel_scores, out, c, pt,
                                               kv_lens, *q8, st)
                     : launch_step_d<128, true>(s, plan, q, k, v, k_comp, kv_len, kv_cap, sel, sel_scores, out, c,
                                                pt, kv_lens, *q8, st);
  const Q8Cache none{nullptr, nullptr, nullptr, nullptr};
  return s.d == 64 ? launch_step_d<64, false>(s, plan, q, k, v, k_comp, kv_len, kv_cap, sel, sel_scores, out, c, pt,
                                              kv_lens, none, st)
                   : launch_step_d<128, false>(s, plan, q, k, v, k_comp, kv_len, kv_cap, sel, sel_scores, out, c, pt,
                                               kv_lens, none, st);
}

PickAttendPlan plan_pick_attend(const Dims& s, int64_t n_chunks) {
  PickAttendPlan p{};
  const int64_t rows = (int64_t)s.batch * s.hkv;
  // one 32-key unit per wave and slice (a slice holds at most 64 entries)
  int bpw = s.bs < kUnit ? kStepWaves * (kUnit / s.bs) : (kStepWaves * kUnit + s.bs - 1) / s.bs;
  if (bpw > kWave) bpw = kWave;
  p.blocks_per_wg = bpw;
  p.n_split = (s.top_k + bpw - 1) / bpw;
  p.n_chunks = n_chunks;
  p.ws_bytes = counter_bytes(rows) + (size_t)rows * p.n_split * (2 * s.group + s.group * s.d) * sizeof(float);
  return p;
}

hipError_t launch_pick_attend(const Dims& s, const PickAttendPlan& pa, const void* q, const void* k, const void* v,
                              int32_t* sel, float* sel_scores, const void* ws_select, void* out, void* counters,
                              void* part, int64_t kv_len, int64_t kv_cap, hipStream_t st, const int32_t* kv_lens) {
  const int64_t rows = (int64_t)s.batch * s.hkv;
  // the score pass's workspace: scores [rows][n_chunks * 256], then the lists
  const uint32_t* wss = reinterpret_cast<const uint32_t*>(ws_select);
  const uint64_t* wsl = reinterpret_cast<const uint64_t*>(wss + rows * pa.n_chunks * kLargeChunk);
  uint32_t* c = static_cast<uint32_t*>(counters);
  float* pt = static_cast<float*>(part);
  return s.d == 64 ? launch_pick_attend_d<64>(s, pa, q, k, v, sel, sel_scores, wss, wsl, out, c, pt, kv_len, kv_cap,
                                              kv_lens, st)
                   : launch_pick_attend_d<128>(s, pa, q, k, v, sel, sel_scores, wss, wsl, out, c, pt, kv_len, kv_cap,
                                               kv_lens, st);
}

}  // namespace qsa
