// Sparse attention for one query token per sequence over its selected blocks
// ("Qwen4 in llama.cpp: Dissecting PR #27742", section "QSA Is an
// Address-Selection Problem, Not a New Attention Equation": ordinary softmax
// attention restricted to the cells the selector returned).
//
// The per-wave unit loop (bf16 MFMA, float32 online softmax, gathered units
// for blocks shorter than 32 keys) is in qsa_decode_unit.h.
//
// Grid: one workgroup per (sequence, KV head, slice of the selection list):
// 4 waves on slices of a few blocks when the rows are few, 8 waves on the
// whole selection when the rows alone fill the GPU (as the fused decode
// step). Waves take units round-robin; the workgroup merges its waves'
// partial softmax states in LDS and writes the output directly when a row
// has one slice. Otherwise it writes its partial state to the workspace at
// the device-coherent level and takes a ticket from the row's arrival
// counter; the last workgroup of the row merges all slices in slice order
// and resets the counter to zero. The merge order is fixed, so results are
// bitwise reproducible whichever workgroup arrives last.
#include "qsa_decode_unit.h"
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

template <int D, int NW>
struct DecodeSmem {
  static constexpr int RS = kStageRowBytes<D>;
  static constexpr int kStage = NW * kUnit * RS;          // V staging, one 32-row slice per wave
  static constexpr int kComb = NW * (32 + 16 * kCombStride<D>) * 4;  // the waves' softmax states
  static constexpr int kBytes = kStage > kComb ? kStage : kComb;
};

template <int D, bool GATHER, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ sel, uint16_t* __restrict__ out, float* __restrict__ part,
    uint32_t* __restrict__ counters, int64_t kv_len, int64_t kv_cap, int hq, int hkv, int G, int bs, int top_k,
    float scale_log2, int bpw, int n_split, const int32_t* __restrict__ kv_lens) {
  using SM = DecodeSmem<D, NW>;
  constexpr int DT = D / 16;  // 16-wide dim tiles of the PV product
  __shared__ __align__(16) unsigned char smem[SM::kBytes];
  __shared__ int last_wg;

  const int64_t row = blockIdx.x / n_split;
  const int split = blockIdx.x % n_split;
  const int64_t b = row / hkv;
  const int g = (int)(row % hkv);
  const int lane = lane_id(), w = wave_id();
  // the token's position: kv_len - 1, or with kv_lens (a ragged batch)
  // sequence b's own length, clamped into [1, kv_len], less one
  int64_t n = kv_len;
  if (kv_lens) {
    n = kv_lens[b];
    n = n < 1 ? 1 : (n > kv_len ? kv_len : n);
  }
  const int64_t p = n - 1;
  const int e0 = split * bpw;
  const int e1 = e0 + bpw < top_k ? e0 + bpw : top_k;
  const int n_e = e1 - e0;
  const int32_t* sel_row = sel + row * top_k;
  const int64_t kv_off = ((int64_t)b * hkv + g) * kv_cap;

  // The slice's block ids, one per lane (bpw <= 64), loaded with Q.
  const int sel_mine = lane < n_e ? sel_row[e0 + lane] : -1;
  u32x4_t qf[D / 32];
  load_q_operands<D>(q + (b * hq + (int64_t)g * G) * D, G, qf);

  float m_run = -__builtin_inff(), l_run = 0.f;
  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  attend_units<D, GATHER>(qf, k + kv_off * D, v + kv_off * D, sel_mine, n_e, bs, p, scale_log2,
                          smem + w * kUnit * SM::RS, w, NW, m_run, l_run, o);
  l_run = sum_col4(l_run);
  finish_row_slice<D, NW>(m_run, l_run, o, smem, &last_wg, out, part, counters, row, b, g, hq, G, split, n_split);
}

// Prefill rows one at a time: one 8-wave workgroup per (sequence, query
// row, KV head), attending over the row's whole selection in chunks of 64
// entries (one per lane) with the decode unit loop, causal at the row's own
// position; the waves' states merge in LDS and the row is written directly.
// This serves the shapes the tiled prefill kernel does not: blocks shorter
// than 32 keys (gathered 32-key units) and selections of more than 64
// blocks, such as the released budget of 512 blocks of 4 keys plus the tail
// ("Qwen4 in llama.cpp: Dissecting PR #27742", section "QSA Is an
// Address-Selection Problem, Not a New Attention Equation"). Every row reads
// its own keys: rows share none of their K/V traffic, as in decode.
template <int D, bool GATHER>
__global__ __launch_bounds__(8 * kWave) void prefill_rows_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ sel, uint16_t* __restrict__ out, int64_t q_len, int64_t q_pos0, int64_t kv_cap,
    int hq, int hkv, int G, int bs, int top_k, float scale_log2) {
  constexpr int NW = 8;
  using SM = DecodeSmem<D, NW>;
  constexpr int DT = D / 16;
  __shared__ __align__(16) unsigned char smem[SM::kBytes];
  __shared__ int last_wg;

  const int64_t row = blockIdx.x;           // ((b * q_len) + t) * hkv + g
  const int64_t bt = row / hkv;             // b * q_len + t
  const int g = (int)(row % hkv);
  const int64_t b = bt / q_len;
  const int64_t p = q_pos0 + bt % q_len;    // the row's absolute position
  const int lane = lane_id(), w = wave_id();
  const int32_t* sel_row = sel + row * top_k;
  const int64_t kv_off = ((int64_t)b * hkv + g) * kv_cap;

  u32x4_t qf[D / 32];
  load_q_operands<D>(q + (bt * hq + (int64_t)g * G) * D, G, qf);
  float m_run = -__builtin_inff(), l_run = 0.f;
  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int e0 = 0; e0 < top_k; e0 += kWave) {
    const int n_e = top_k - e0 < kWave ? top_k - e0 : kWave;
    const int sel_mine = lane < n_e ? sel_row[e0 + lane] : -1;
    attend_units<D, GATHER>(qf, k + kv_off * D, v + kv_off * D, sel_mine, n_e, bs, p, scale_log2,
                            smem + w * kUnit * SM::RS, w, NW, m_run, l_run, o);
  }
  l_run = sum_col4(l_run);
  finish_row_slice<D, NW>(m_run, l_run, o, smem, &last_wg, out, nullptr, nullptr, row, bt, g, hq, G, 0, 1);
}

template <int D>
hipError_t launch_prefill_rows_d(const Dims& s, const void* q, const void* k, const void* v, int64_t q_len,
                                 int64_t q_pos0, int64_t kv_cap, const int32_t* sel, void* out, hipStream_t st) {
  const int64_t rows = (int64_t)s.batch * q_len * s.hkv;
  auto kern = s.bs < kUnit ? prefill_rows_kernel<D, true> : prefill_rows_kernel<D, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)rows), dim3(8 * kWave), 0, st, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), sel,
                     static_cast<uint16_t*>(out), q_len, q_pos0, kv_cap, s.hq, s.hkv, s.group, s.bs, s.top_k,
                     s.scale * 1.4426950408889634f);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Dims& s, const DecodePlan& plan, const void* q, const void* k, const void* v,
                    int64_t kv_len, int64_t kv_cap, const int32_t* sel, void* out, uint32_t* counters, float* part,
                    hipStream_t st, const int32_t* kv_lens) {
  const int64_t rows = (int64_t)s.batch * s.hkv;
  const float scale_log2 = s.scale * 1.4426950408889634f;
  auto kern = plan.waves == 8 ? (s.bs < kUnit ? decode_attn_kernel<D, true, 8> : decode_attn_kernel<D, false, 8>)
                              : (s.bs < kUnit ? decode_attn_kernel<D, true, 4> : decode_attn_kernel<D, false, 4>);
  if (plan.n_split == 1) part = nullptr;
  hipLaunchKernelGGL(kern, dim3((unsigned)(rows * plan.n_split)), dim3(plan.waves * kWave), 0, st,
                     static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), sel,
                     static_cast<uint16_t*>(out), part, counters, kv_len, kv_cap, s.hq, s.hkv, s.group, s.bs, s.top_k,
                     scale_log2, plan.blocks_per_wg, plan.n_split, kv_lens);
  return hipGetLastError();
}

}  // namespace

DecodePlan plan_decode(const Dims& s, int64_t kv_len, bool wide) {
  (void)kv_len;
  DecodePlan p{};
  const int64_t rows = (int64_t)s.batch * s.hkv;
  p.waves = 4;
  if (wide && rows >= 128 && s.top_k <= kWave) {
    // the rows alone fill the GPU: one 8-wave workgroup per row over the
    // whole selection (the fused decode step's shape; 64 x 128K attention
    // 19.2 -> 16.6 us against 4-block slices), no slice states to merge
    p.waves = 8;
    p.blocks_per_wg = s.top_k;
    p.n_split = 1;
    p.ws_bytes = 0;
    return p;
  }
  // Smallest slices that still give every wave a unit, grown while the grid
  // stays above ~512 workgroups (fewer partial states to merge). A slice
  // holds at most 64 entries (one per lane).
  int bpw = (4 * kUnit + s.bs - 1) / s.bs;  // blocks giving one unit per wave
  if (bpw < 1) bpw = 1;
  while (2 * bpw <= kWave && bpw < s.top_k && rows * ((s.top_k + 2 * bpw - 1) / (2 * bpw)) >= 512) bpw *= 2;
  if (bpw > s.top_k) bpw = s.top_k;
  p.blocks_per_wg = bpw;
  p.n_split = (s.top_k + bpw - 1) / bpw;
  // arrival counters (kept at zero between calls), then the partial states
  p.ws_bytes = p.n_split > 1 ? counter_bytes(rows) +
                                   (size_t)rows * p.n_split * (2 * s.group + s.group * s.d) * sizeof(float)
                             : 0;
  return p;
}

hipError_t launch_prefill_rows(const Dims& s, const void* q, const void* k, const void* v, int64_t q_len,
                               int64_t q_pos0, int64_t kv_cap, const int32_t* sel, void* out, hipStream_t st) {
  return s.d == 64 ? launch_prefill_rows_d<64>(s, q, k, v, q_len, q_pos0, kv_cap, sel, out, st)
                   : launch_prefill_rows_d<128>(s, q, k, v, q_len, q_pos0, kv_cap, sel, out, st);
}

hipError_t launch_decode(const Dims& s, const DecodePlan& plan, const void* q, const void* k, const void* v,
                         int64_t kv_len, int64_t kv_cap, const int32_t* sel, void* out, void* counters, void* part,
                         hipStream_t st, const int32_t* kv_lens) {
  uint32_t* c = static_cast<uint32_t*>(counters);
  float* pt = static_cast<float*>(part);
  return s.d == 64 ? launch_d<64>(s, plan, q, k, v, kv_len, kv_cap, sel, out, c, pt, st, kv_lens)
                   : launch_d<128>(s, plan, q, k, v, kv_len, kv_cap, sel, out, c, pt, st, kv_lens);
}

}  // namespace qsa
