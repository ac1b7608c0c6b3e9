// Learned-indexer selection: block selection scored in a separate, lower-
// dimensional indexer space ("Qwen4 in llama.cpp: Dissecting PR #27742",
// section "QSA Is an Address-Selection Problem, Not a New Attention
// Equation": indexer projections feed the compressed-block representation,
// which is scored to pick the kept blocks).
//
// Indexer keys: the compressed attention keys projected by W_k ([d][dim],
// shared by all heads); projecting a block's mean equals averaging its
// projected keys. Indexer scores: every query head of a KV head's group is
// projected by W_q and scored against each candidate's indexer key, and the
// heads' scores are aggregated (sum, max, or each head's softmax over the
// candidates summed over the heads). Selection frame, forced block and
// output format are those of the default selection.
//
// Both kernels stream small, L2-resident data; they favour plain fixed-order
// float32 arithmetic (deterministic) over peak rate.
#include "qsa_decode_unit.h"
#include "qsa_device.h"
#include "qsa_internal.h"
#include "qsa_select_wave.h"

namespace qsa {
namespace {

// One wave per (sequence, KV head, block): k_idx = W_k^T k_comp, the sum
// over the d inputs in ascending order. W_k is staged in LDS once per
// workgroup (16-byte loads, all in flight together); lane l holds the
// compressed key's elements l, l + 64 (d = 128), each broadcast from its
// lane in turn.
template <int D, int DI>
__global__ __launch_bounds__(256) void indexer_keys_kernel(const float* __restrict__ k_comp,
                                                           const float* __restrict__ w_k, float* __restrict__ k_idx,
                                                           int64_t nb_cap, int64_t blk_begin, int64_t n_blk,
                                                           int64_t n_items) {
  constexpr int EPL = DI / kWave;  // outputs per lane
  constexpr int IPL = D / kWave;   // inputs per lane
  __shared__ __align__(16) float wk_s[D * DI];
  {
    constexpr int NW4 = D * DI / 4 / 256;
    f32x4_t wv[NW4];
#pragma unroll
    for (int i = 0; i < NW4; ++i) wv[i] = *reinterpret_cast<const f32x4_t*>(w_k + 4 * (threadIdx.x + 256 * i));
#pragma unroll
    for (int i = 0; i < NW4; ++i) *reinterpret_cast<f32x4_t*>(&wk_s[4 * (threadIdx.x + 256 * i)]) = wv[i];
  }
  __syncthreads();
  const int64_t item = (int64_t)blockIdx.x * 4 + wave_id();
  if (item >= n_items) return;
  const int64_t bg = item / n_blk;
  const int64_t c = blk_begin + item % n_blk;
  const int lane = lane_id();
  const float* src = k_comp + (bg * nb_cap + c) * D;
  float x[IPL];
#pragma unroll
  for (int i = 0; i < IPL; ++i) x[i] = src[lane + kWave * i];
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
#pragma unroll
  for (int i = 0; i < IPL; ++i) {
#pragma unroll 8
    for (int j = 0; j < kWave; ++j) {
      const float kj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x[i]), j));
      const float* wr = wk_s + (kWave * i + j) * DI + lane;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = __builtin_fmaf(kj, wr[kWave * e], acc[e]);
    }
  }
  float* dst = k_idx + (bg * nb_cap + c) * DI + lane;
#pragma unroll
  for (int e = 0; e < EPL; ++e) dst[kWave * e] = acc[e];
}


// One workgroup per (sequence, query row, KV head), 4 or 8 waves.
// 1. the G query heads are projected into LDS (already scaled);
// 2. each wave scores 64 candidates per pass with fp32 MFMA, the G head
//    scores of each candidate aggregated across the product's head columns;
//    with the softmax aggregation a first pass finds every head's maximum
//    and normaliser over the row's candidates and a second pass scores;
// 3. per-wave top lists, merged, and the row's selection written as the
//    default selection writes it; or (LARGE, top_k > 64) every candidate's
//    aggregated score written to ws_scores in the large selection's layout
//    ([row][n_chunks * 256] score order bits), for its per-row pick.
// STEP (a decode step, bf16, q_len = 1, top_k <= 64): before 2., the last
// wave compresses the block the new token closes (if any) into k_comp_w,
// then projects it into k_idx_w while the other waves project the query
// heads (its indexer key is read from LDS where it is a candidate, with
// keep_tail); after 3. the workgroup attends over its selection as the
// fused decode step does, one slice, and writes out.
template <int D, int NW>
constexpr int idx_stage_bytes() {
  const int stage = NW * kUnit * kStageRowBytes<D>;
  const int comb = NW * (32 + 16 * kCombStride<D>) * 4;
  return stage > comb ? stage : comb;
}

template <typename T, int D, int DI, int AGG, int kIdxThreads, bool LARGE, bool STEP = false>
__global__ __launch_bounds__(kIdxThreads) void indexer_select_kernel(
    const T* __restrict__ q, const float* __restrict__ w_q, const float* __restrict__ k_idx,
    int32_t* __restrict__ sel, float* __restrict__ sel_scores, uint32_t* __restrict__ ws_scores, int64_t n_chunks,
    int64_t q_len, int64_t q_pos0, int64_t nb_cap, int hq, int hkv, int G, int bs, int top_k, float scale,
    int keep_tail, const T* __restrict__ k_cache = nullptr, const T* __restrict__ v_cache = nullptr,
    const float* __restrict__ w_k = nullptr, float* __restrict__ k_comp_w = nullptr, float* __restrict__ k_idx_w = nullptr,
    T* __restrict__ out = nullptr, int64_t kv_cap = 0, float attn_scale_log2 = 0.f) {
  constexpr int kIdxWaves = kIdxThreads / kWave;
  static_assert(!(STEP && LARGE), "the fused step keeps the selection in the workgroup");
  __shared__ __align__(16) float qi[16 * DI];
  __shared__ __align__(16) float qs[16 * D];    // the group's query heads, as float
  __shared__ uint64_t lists[kIdxWaves][kWave];
  __shared__ float red_m[kIdxWaves][16], red_z[kIdxWaves][16];
  __shared__ float head_m[16], head_z[16];
  // STEP only: the attention's staging and combine area, the closed block's
  // mean key and indexer key, and the selection
  __shared__ __align__(16) unsigned char big[STEP ? idx_stage_bytes<D, kIdxWaves>() : 16];
  __shared__ __align__(16) float knew[STEP ? D : 4];
  __shared__ __align__(16) float kinew[STEP ? DI : 4];
  __shared__ int ids[STEP ? kWave : 1];
  __shared__ int last_wg;

  const int64_t row = blockIdx.x;
  const int g = (int)(row % hkv);
  const int64_t bt = row / hkv;
  const int64_t t = bt % q_len;
  const int64_t b = bt / q_len;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int64_t p = q_pos0 + t;
  const Frame fr = row_frame(p, bs, keep_tail);
  const int slots = frame_slots(fr, top_k);
  // STEP: the block the token at p closes, if any, and the candidate whose
  // indexer key comes from LDS (that block, where it competes)
  const bool closes = STEP && (p + 1) % bs == 0;
  const int64_t c_new = (p + 1) / bs - 1;
  const int64_t c_lds = closes && keep_tail ? c_new : -1;
  const int64_t bg_off = ((int64_t)b * hkv + g) * nb_cap;  // this (sequence, KV head)'s first block
  if constexpr (STEP) {
    static_assert(sizeof(T) == 2, "the fused step attends over a bf16 cache");
    if (closes && w == kIdxWaves - 1)
      compress_block_wave<T, D>(k_cache + (((int64_t)b * hkv + g) * kv_cap + c_new * bs) * D, bs,
                                k_comp_w + (bg_off + c_new) * D, knew);
  }

  // 1. projected, scaled query heads by fp32 MFMA: the heads (as float, in
  // LDS) as operand A, W_q read straight from memory as operand B; wave w
  // computes the 16 outputs 16n .. 16n+15 (n = w, w + waves, ...) of every
  // head, the d terms in steps of 4 (the MFMA's own sum within a step)
  const T* qh = q + ((b * q_len + t) * hq + (int64_t)g * G) * D;
  for (int i = tid; i < G * D / 4; i += kIdxThreads)
    *reinterpret_cast<f32x4_t*>(&qs[4 * i]) = load4_f32(qh + 4 * i);
  __syncthreads();
  {
    const int pk = lane >> 4, pm = lane & 15;
    for (int n = w; n < DI / 16; n += kIdxWaves) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int u = 0; u < D / 16; ++u) {
        const int d0 = 16 * u + 4 * pk;
        f32x4_t a = {0.f, 0.f, 0.f, 0.f};
        if (pm < G) a = *reinterpret_cast<const f32x4_t*>(&qs[pm * D + d0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mfma_f32(a[e], w_q[(int64_t)(d0 + e) * DI + 16 * n + pm], acc);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (4 * pk + v < G) qi[(4 * pk + v) * DI + 16 * n + pm] = acc[v] * scale;
    }
  }
  if constexpr (STEP) {
    // the closed block's indexer key, in the indexer keys kernel's order (a
    // fused multiply-add chain over the d inputs in ascending order)
    if (closes && w == kIdxWaves - 1) {
      constexpr int EPL = DI / kWave;
      float acc[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
#pragma unroll 16
      for (int i = 0; i < D; ++i) {
        const float kj = knew[i];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = __builtin_fmaf(kj, w_k[(int64_t)i * DI + lane + kWave * e], acc[e]);
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        k_idx_w[(bg_off + c_new) * DI + lane + kWave * e] = acc[e];
        kinew[lane + kWave * e] = acc[e];
      }
    }
  }
  __syncthreads();

  const float* krow = k_idx + ((b * hkv + g) * nb_cap) * DI;
  // Head scores by fp32 MFMA (16x16x4): the indexer keys of 16 candidates as
  // operand A, the projected query heads as operand B (head m in column m,
  // columns >= G zero), so lane (kg, m) ends a tile with the scores of
  // candidates 4kg .. 4kg+3 for head m. Its head's query dims 16u + 4kg + e
  // stay in registers (qb[4u + e]).
  const int kg = lane >> 4, m = lane & 15;
  float qb[DI / 4];
#pragma unroll
  for (int u = 0; u < DI / 16; ++u) {
    f32x4_t a = {0.f, 0.f, 0.f, 0.f};
    if (m < G) a = *reinterpret_cast<const f32x4_t*>(&qi[m * DI + 16 * u + 4 * kg]);
#pragma unroll
    for (int e = 0; e < 4; ++e) qb[4 * u + e] = a[e];
  }
  // scores of candidates c0 + 16 t + 4 kg + v (t < 4) for head m, into acc[t][v]
  auto pass_scores = [&](int c0, f32x4_t (&acc)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int c = c0 + 16 * t + m;  // this lane's operand row
      const bool ok = c < fr.n_cand;
#pragma unroll
      for (int u = 0; u < DI / 16; ++u) {
        f32x4_t kv = ok ? *reinterpret_cast<const f32x4_t*>(krow + (int64_t)c * DI + 16 * u + 4 * kg)
                        : f32x4_t{0.f, 0.f, 0.f, 0.f};
        if constexpr (STEP)
          if (c == c_lds) kv = *reinterpret_cast<const f32x4_t*>(&kinew[16 * u + 4 * kg]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t] = mfma_f32(kv[e], qb[4 * u + e], acc[t]);
      }
    }
  };

  if constexpr (AGG == kAggSoftmax) {
    // pass 1: every head's maximum and normaliser over the candidates (lane
    // (kg, m) folds its 16 candidates per pass for head m, then the lanes of
    // a head and the waves are combined)
    float mh = -__builtin_inff(), zh = 0.f;
    for (int base = kWave * w; base < fr.n_cand; base += kIdxThreads) {
      f32x4_t acc[4];
      pass_scores(base, acc);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (base + 16 * t + 4 * kg + v < fr.n_cand) {
            const float x = acc[t][v];
            const float mn = fmaxf(mh, x);
            zh = zh * __expf(mh - mn) + __expf(x - mn);
            mh = mn;
          }
        }
    }
#pragma unroll
    for (int d = 16; d < kWave; d <<= 1) {
      const float mo = __shfl_xor(mh, d, kWave), zo = __shfl_xor(zh, d, kWave);
      const float mn = fmaxf(mh, mo);
      zh = (mn == -__builtin_inff()) ? 0.f : zh * __expf(mh - mn) + zo * __expf(mo - mn);
      mh = mn;
    }
    if (lane < 16) {
      red_m[w][lane] = mh;
      red_z[w][lane] = zh;
    }
    __syncthreads();
    if (tid < G) {
      float hm = -__builtin_inff(), hz = 0.f;
      for (int ww = 0; ww < kIdxWaves; ++ww) {
        const float mo = red_m[ww][tid], zo = red_z[ww][tid];
        const float mn = fmaxf(hm, mo);
        hz = (mn == -__builtin_inff()) ? 0.f : hz * __expf(hm - mn) + zo * __expf(mo - mn);
        hm = mn;
      }
      head_m[tid] = hm;
      head_z[tid] = hz;
    }
    __syncthreads();
  }

  // 2. aggregated scores: per candidate over the 16 head lanes, then lane
  // (kg, m) takes candidate 16 (m / 4) + 4 kg + m % 4 of the pass into the
  // wave's top list (64 candidates per pass, one per lane)
  uint64_t cur = 0ull;
  if (slots > 0) {
    float hm = 0.f, hz = 1.f;
    if constexpr (AGG == kAggSoftmax) {
      if (m < G) {
        hm = head_m[m];
        hz = head_z[m];
      }
    }
    for (int base = kWave * w; base < fr.n_cand; base += kIdxThreads) {
      f32x4_t acc[4];
      pass_scores(base, acc);
      float red[4][4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float x = acc[t][v];
          if constexpr (AGG == kAggMax) x = m < G ? x : -__builtin_inff();
          if constexpr (AGG == kAggSoftmax) x = m < G ? __expf(x - hm) / hz : 0.f;
#pragma unroll
          for (int d = 1; d < 16; d <<= 1) {
            const float o = xor_lane_f32(x, d);
            x = AGG == kAggMax ? fmaxf(x, o) : x + o;
          }
          red[t][v] = x;
        }
      const int t_me = m >> 2, v_me = m & 3;
      float a = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (t == t_me && v == v_me) a = red[t][v];
      const int c = base + 16 * t_me + 4 * kg + v_me;
      if constexpr (LARGE) {
        if (c < fr.n_cand) ws_scores[row * n_chunks * 256 + c] = score_order_bits(a);
      } else {
        cur = topk_fold(cur, c < fr.n_cand ? make_key(a, c) : 0ull, slots);
      }
    }
  }
  if constexpr (LARGE) return;
  cur = merge_wave_lists<kIdxWaves>(lists, cur, slots > 0 ? slots : 1);
  if (w == 0) {
    const int64_t off = row * top_k;
    finalize_row(cur, slots, fr.forced, top_k, sel + off, sel_scores ? sel_scores + off : nullptr,
                 STEP ? ids : nullptr);
  }
  if constexpr (STEP) {
    // 4. attention over the selection (ids: ascending, forced block last,
    // -1 padding), the whole selection as one slice
    __syncthreads();
    const int64_t kv_off = ((int64_t)b * hkv + g) * kv_cap;
    const uint16_t* kc = reinterpret_cast<const uint16_t*>(k_cache) + kv_off * D;
    const uint16_t* vc = reinterpret_cast<const uint16_t*>(v_cache) + kv_off * D;
    u32x4_t qf[D / 32];
    load_q_operands<D>(reinterpret_cast<const uint16_t*>(qh), G, qf);
    const int sel_mine = lane < top_k ? ids[lane] : -1;
    float m_run = -__builtin_inff(), l_run = 0.f;
    f32x4_t o[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    unsigned char* vs = big + w * kUnit * kStageRowBytes<D>;
    if (bs < kUnit)
      attend_units<D, true>(qf, kc, vc, sel_mine, top_k, bs, p, attn_scale_log2, vs, w, kIdxWaves, m_run, l_run, o);
    else
      attend_units<D, false>(qf, kc, vc, sel_mine, top_k, bs, p, attn_scale_log2, vs, w, kIdxWaves, m_run, l_run, o);
    l_run = sum_col4(l_run);
    finish_row_slice<D, kIdxWaves>(m_run, l_run, o, big, &last_wg, reinterpret_cast<uint16_t*>(out), nullptr, nullptr,
                                   row, b, g, hq, G, 0, 1);
  }
}

template <int D, int DI>
hipError_t launch_keys(const float* w_k, const float* k_comp, int64_t nb_cap, int64_t blk_begin, int64_t n_blk,
                       int64_t n_items, float* k_idx, hipStream_t st) {
  hipLaunchKernelGGL((indexer_keys_kernel<D, DI>), dim3((unsigned)((n_items + 3) / 4)), dim3(256), 0, st, k_comp, w_k,
                     k_idx, nb_cap, blk_begin, n_blk, n_items);
  return hipGetLastError();
}

template <typename T, int D, int DI, int NT, bool LARGE>
hipError_t launch_select_nl(const Dims& s, const IndexerDims& ix, const float* w_q, const void* q, int64_t q_len,
                            int64_t q_pos0, const float* k_idx, int64_t kv_cap, int32_t* sel, float* sel_scores,
                            uint32_t* ws_scores, int64_t n_chunks, hipStream_t st) {
  const int64_t rows = (int64_t)s.batch * q_len * s.hkv;
  const int64_t nb_cap = kv_cap / s.bs;
  const T* qp = static_cast<const T*>(q);
  const dim3 grid((unsigned)rows), block(NT);
  auto kern = ix.agg == kAggSum   ? indexer_select_kernel<T, D, DI, kAggSum, NT, LARGE>
              : ix.agg == kAggMax ? indexer_select_kernel<T, D, DI, kAggMax, NT, LARGE>
                                  : indexer_select_kernel<T, D, DI, kAggSoftmax, NT, LARGE>;
  hipLaunchKernelGGL(kern, grid, block, 0, st, qp, w_q, k_idx, sel, sel_scores, ws_scores, n_chunks, q_len, q_pos0,
                     nb_cap, s.hq, s.hkv, s.group, s.bs, s.top_k, ix.scale, s.keep_tail, static_cast<const T*>(nullptr),
                     static_cast<const T*>(nullptr), static_cast<const float*>(nullptr), static_cast<float*>(nullptr),
                     static_cast<float*>(nullptr), static_cast<T*>(nullptr), (int64_t)0, 0.f);
  return hipGetLastError();
}

template <typename T, int D, int DI, int NT>
hipError_t launch_select_nt(const Dims& s, const IndexerDims& ix, const float* w_q, const void* q, int64_t q_len,
                            int64_t q_pos0, const float* k_idx, int64_t kv_cap, int32_t* sel, float* sel_scores,
                            uint32_t* ws_scores, int64_t n_chunks, hipStream_t st) {
  if (ws_scores)
    return launch_select_nl<T, D, DI, NT, true>(s, ix, w_q, q, q_len, q_pos0, k_idx, kv_cap, sel, sel_scores,
                                                ws_scores, n_chunks, st);
  return launch_select_nl<T, D, DI, NT, false>(s, ix, w_q, q, q_len, q_pos0, k_idx, kv_cap, sel, sel_scores, nullptr,
                                               0, st);
}

// Rows fewer than the CUs (decode): 8 waves per row, so that the projection
// and the candidates of the few rows spread over more of each CU (32K decode,
// 2 rows: the call 18.2 -> 15.9 us event-timed; 16 waves would cap the
// registers at 128 and spill a candidate's indexer key); otherwise 4 waves.
template <typename T, int D, int DI>
hipError_t launch_select_t(const Dims& s, const IndexerDims& ix, const float* w_q, const void* q, int64_t q_len,
                           int64_t q_pos0, const float* k_idx, int64_t kv_cap, int32_t* sel, float* sel_scores,
                           uint32_t* ws_scores, int64_t n_chunks, hipStream_t st) {
  const int64_t rows = (int64_t)s.batch * q_len * s.hkv;
  if (rows < 256)
    return launch_select_nt<T, D, DI, 512>(s, ix, w_q, q, q_len, q_pos0, k_idx, kv_cap, sel, sel_scores, ws_scores, n_chunks, st);
  return launch_select_nt<T, D, DI, 256>(s, ix, w_q, q, q_len, q_pos0, k_idx, kv_cap, sel, sel_scores, ws_scores, n_chunks, st);
}

template <typename T>
hipError_t launch_select_d(const Dims& s, const IndexerDims& ix, const float* w_q, const void* q, int64_t q_len,
                           int64_t q_pos0, const float* k_idx, int64_t kv_cap, int32_t* sel, float* sel_scores,
                           uint32_t* ws_scores, int64_t n_chunks, hipStream_t st) {
  if (s.d == 64)
    return ix.dim == 64 ? launch_select_t<T, 64, 64>(s, ix, w_q, q, q_len, q_pos0, k_idx, kv_cap, sel, sel_scores, ws_scores, n_chunks, st)
                        : launch_select_t<T, 64, 128>(s, ix, w_q, q, q_len, q_pos0, k_idx, kv_cap, sel, sel_scores, ws_scores, n_chunks, st);
  return ix.dim == 64 ? launch_select_t<T, 128, 64>(s, ix, w_q, q, q_len, q_pos0, k_idx, kv_cap, sel, sel_scores, ws_scores, n_chunks, st)
                      : launch_select_t<T, 128, 128>(s, ix, w_q, q, q_len, q_pos0, k_idx, kv_cap, sel, sel_scores, ws_scores, n_chunks, st);
}

template <int D, int DI, int NT>
hipError_t launch_step_nt(const Dims& s, const IndexerDims& ix, const float* w_q, const float* w_k, const void* q,
                          const void* k, const void* v, float* k_comp, float* k_idx, int64_t kv_len, int64_t kv_cap,
                          int32_t* sel, float* sel_scores, void* out, hipStream_t st) {
  const int64_t rows = (int64_t)s.batch * s.hkv;
  const auto* qp = static_cast<const uint16_t*>(q);
  auto kern = ix.agg == kAggSum   ? indexer_select_kernel<uint16_t, D, DI, kAggSum, NT, false, true>
              : ix.agg == kAggMax ? indexer_select_kernel<uint16_t, D, DI, kAggMax, NT, false, true>
                                  : indexer_select_kernel<uint16_t, D, DI, kAggSoftmax, NT, false, true>;
  hipLaunchKernelGGL(kern, dim3((unsigned)rows), dim3(NT), 0, st, qp, w_q, k_idx, sel, sel_scores, nullptr,
                     (int64_t)0, (int64_t)1, kv_len - 1, kv_cap / s.bs, s.hq, s.hkv, s.group, s.bs, s.top_k, ix.scale,
                     s.keep_tail, static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), w_k, k_comp,
                     k_idx, static_cast<uint16_t*>(out), kv_cap, s.scale * 1.4426950408889634f);
  return hipGetLastError();
}

template <int D, int DI>
hipError_t launch_step_t(const Dims& s, const IndexerDims& ix, const float* w_q, const float* w_k, const void* q,
                         const void* k, const void* v, float* k_comp, float* k_idx, int64_t kv_len, int64_t kv_cap,
                         int32_t* sel, float* sel_scores, void* out, hipStream_t st) {
  // as the selection: 8 waves per row when the rows are fewer than the CUs
  if ((int64_t)s.batch * s.hkv < 256)
    return launch_step_nt<D, DI, 512>(s, ix, w_q, w_k, q, k, v, k_comp, k_idx, kv_len, kv_cap, sel, sel_scores, out, st);
  return launch_step_nt<D, DI, 256>(s, ix, w_q, w_k, q, k, v, k_comp, k_idx, kv_len, kv_cap, sel, sel_scores, out, st);
}

}  // namespace

hipError_t launch_indexer_step(const Dims& s, const IndexerDims& ix, const float* w_q, const float* w_k,
                               const void* q, const void* k, const void* v, float* k_comp, float* k_idx,
                               int64_t kv_len, int64_t kv_cap, int32_t* sel, float* sel_scores, void* out,
                               hipStream_t st) {
  if (s.d == 64)
    return ix.dim == 64
               ? launch_step_t<64, 64>(s, ix, w_q, w_k, q, k, v, k_comp, k_idx, kv_len, kv_cap, sel, sel_scores, out, st)
               : launch_step_t<64, 128>(s, ix, w_q, w_k, q, k, v, k_comp, k_idx, kv_len, kv_cap, sel, sel_scores, out, st);
  return ix.dim == 64
             ? launch_step_t<128, 64>(s, ix, w_q, w_k, q, k, v, k_comp, k_idx, kv_len, kv_cap, sel, sel_scores, out, st)
             : launch_step_t<128, 128>(s, ix, w_q, w_k, q, k, v, k_comp, k_idx, kv_len, kv_cap, sel, sel_scores, out, st);
}

hipError_t launch_indexer_keys(const Dims& s, const IndexerDims& ix, const float* w_k, const float* k_comp,
                               int64_t kv_cap, int64_t blk_begin, int64_t blk_end, float* k_idx, hipStream_t st) {
  const int64_t n_blk = blk_end - blk_begin;
  if (n_blk <= 0) return hipSuccess;
  const int64_t nb_cap = kv_cap / s.bs;
  const int64_t n_items = (int64_t)s.batch * s.hkv * n_blk;
  if (s.d == 64)
    return ix.dim == 64 ? launch_keys<64, 64>(w_k, k_comp, nb_cap, blk_begin, n_blk, n_items, k_idx, st)
                        : launch_keys<64, 128>(w_k, k_comp, nb_cap, blk_begin, n_blk, n_items, k_idx, st);
  return ix.dim == 64 ? launch_keys<128, 64>(w_k, k_comp, nb_cap, blk_begin, n_blk, n_items, k_idx, st)
                      : launch_keys<128, 128>(w_k, k_comp, nb_cap, blk_begin, n_blk, n_items, k_idx, st);
}

hipError_t launch_indexer_select(const Dims& s, const IndexerDims& ix, const float* w_q, const void* q,
                                 int64_t q_len, int64_t q_pos0, const float* k_idx, int64_t kv_cap, int32_t* sel,
                                 float* sel_scores, void* ws, hipStream_t st) {
  if (s.top_k <= 64)
    return s.dtype == 1
               ? launch_select_d<uint16_t>(s, ix, w_q, q, q_len, q_pos0, k_idx, kv_cap, sel, sel_scores, nullptr, 0, st)
               : launch_select_d<float>(s, ix, w_q, q, q_len, q_pos0, k_idx, kv_cap, sel, sel_scores, nullptr, 0, st);
  // top_k > 64: every candidate's aggregated score in ws (the large
  // selection's layout), then its per-row pick, which also writes the rows
  // without candidates (the forced block and padding)
  const int64_t n_chunks = plan_select(s, q_len, q_pos0).n_chunks;
  if (n_chunks > 0) {
    uint32_t* ws_scores = static_cast<uint32_t*>(ws);
    const hipError_t e =
        s.dtype == 1 ? launch_select_d<uint16_t>(s, ix, w_q, q, q_len, q_pos0, k_idx, kv_cap, sel, sel_scores,
                                                 ws_scores, n_chunks, st)
                     : launch_select_d<float>(s, ix, w_q, q, q_len, q_pos0, k_idx, kv_cap, sel, sel_scores, ws_scores,
                                              n_chunks, st);
    if (e != hipSuccess) return e;
  }
  return launch_large_pick(s, q_len, q_pos0, n_chunks, ws, true, sel, sel_scores, st);
}

}  // namespace qsa
