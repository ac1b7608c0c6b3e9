// Rotated, 8-bit quantized K/V cache and the decode and prefill attention
// that read it
// ("Qwen4 in llama.cpp: Dissecting PR #27742", section "Quantized KV Exposed
// a Backend Storage Invariant": K and V are stored in a Hadamard-rotated
// basis and quantized; attention runs in the rotated basis and its output is
// rotated back, which is exact because the scaled Hadamard matrix is its own
// inverse; the indexer keeps reading the unrotated compressed keys).
//
// Rotation: the unnormalised Walsh-Hadamard transform of a head vector
// (entries +-1, Sylvester order), butterfly stages h = 1, 2, ..., d/2 in that
// order, pair (i, i + h) becoming (x_i + x_{i+h}, x_i - x_{i+h}) in float32.
// Since H^T H = d I, scores use (H q).(H k) / d and outputs H (sum p H v) / d.
//
// Quantization (per 32 values of a rotated row, float32): scale = the
// largest magnitude / 127, rounded to float16 and stored; code =
// round-half-even(value / scale) clamped to [-127, 127] (0 when the scale
// is 0); dequantized value = code * scale.
#include "qsa_decode_unit.h"
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

// One wave per (sequence, KV head, position, K or V): rotate the row, then
// quantize each 32-value group.
template <int D>
__global__ __launch_bounds__(256) void kv_quantize_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                          int8_t* __restrict__ kq, int8_t* __restrict__ vq,
                                                          uint16_t* __restrict__ ks, uint16_t* __restrict__ vs,
                                                          int64_t kv_cap, int64_t pos_begin, int64_t n_pos,
                                                          int64_t n_items) {
  const int64_t item = (int64_t)blockIdx.x * 4 + wave_id();
  if (item >= 2 * n_items) return;
  const bool is_v = item >= n_items;
  const int64_t it = is_v ? item - n_items : item;
  const int64_t bg = it / n_pos;
  const int64_t pos = pos_begin + it % n_pos;
  const int64_t rowoff = (bg * kv_cap + pos) * D;
  quantize_row_wave<D>((is_v ? v : k) + rowoff, (is_v ? vq : kq) + rowoff,
                       (is_v ? vs : ks) + (bg * kv_cap + pos) * (D / 32));
}

template <int D, int NW>
struct Q8Smem {
  static constexpr int RS = kStageRowBytes<D>;
  static constexpr int kStage = NW * kUnit * RS;
  static constexpr int kComb = NW * (32 + 16 * kCombStride<D>) * 4;
  static constexpr int kBytes = kStage > kComb ? kStage : kComb;
};

// Decode attention over the rotated quantized cache: one workgroup per
// (sequence, KV head, slice of the selection), 4 or 8 waves as the bf16
// decode kernel plans them. The G query heads are
// rotated into LDS (bf16 operands), the units are those of the bf16 decode
// kernel with the codes widened on load, and the combined state of the
// slice is rotated back (H O / d) before it is written, which commutes with
// the softmax merge of the slices (a linear combination of the states).
template <int D, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_attn_q8_kernel(
    const uint16_t* __restrict__ q, const int8_t* __restrict__ kq, const int8_t* __restrict__ vq,
    const uint16_t* __restrict__ ks, const uint16_t* __restrict__ vs_, const int32_t* __restrict__ sel,
    uint16_t* __restrict__ out, float* __restrict__ part, uint32_t* __restrict__ counters, int64_t kv_len,
    int64_t kv_cap, int hq, int hkv, int G, int bs, int top_k, float scale_log2, int bpw, int n_split) {
  using SM = Q8Smem<D, NW>;
  constexpr int NT = NW * kWave;
  constexpr int DT = D / 16;
  constexpr int EPL = D / kWave;
  __shared__ __align__(16) unsigned char smem[SM::kBytes];
  __shared__ __align__(16) uint16_t qrot[16 * D];
  __shared__ __align__(16) float comb_o[16 * D];  // the slice's combined output, rotated back
  __shared__ float comb_m[16], comb_l[16];
  __shared__ int last_wg;

  const int64_t row = blockIdx.x / n_split;
  const int split = blockIdx.x % n_split;
  const int64_t b = row / hkv;
  const int g = (int)(row % hkv);
  const int lane = lane_id(), w = wave_id(), tid = threadIdx.x;
  const int lg = lane / 16, col = lane % 16;
  const int64_t p = kv_len - 1;
  const int e0 = split * bpw;
  const int n_e = top_k - e0 < bpw ? top_k - e0 : bpw;
  const int64_t kv_off = ((int64_t)b * hkv + g) * kv_cap;

  // rotated query heads (bf16), head h by wave h % 4
  const uint16_t* qh = q + (b * hq + (int64_t)g * G) * D;
  for (int h = w; h < G; h += NW) {
    float x[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) x[i] = bf16_to_f32(qh[(int64_t)h * D + lane + kWave * i]);
    fwht_wave<D>(x);
#pragma unroll
    for (int i = 0; i < EPL; ++i) qrot[h * D + lane + kWave * i] = f32_to_bf16(x[i]);
  }
  __syncthreads();
  u32x4_t qf[D / 32];
  load_q8_query_operands<D>(qrot, G, qf);  // the cache's dim order (attend_units' 8-bit loads)

  float m_run = -__builtin_inff(), l_run = 0.f;
  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int sel_mine = lane < n_e ? sel[row * top_k + e0 + lane] : -1;
  const Q8Cache cache{kq + kv_off * D, vq + kv_off * D, ks + kv_off * (D / 32), vs_ + kv_off * (D / 32)};
  // blocks shorter than a 32-key unit: the unit's rows gathered from several entries
  if (bs < kUnit)
    attend_units<D, true, true>(qf, nullptr, nullptr, sel_mine, n_e, bs, p, scale_log2, smem + w * kUnit * SM::RS, w,
                                NW, m_run, l_run, o, cache);
  else
    attend_units<D, false, true>(qf, nullptr, nullptr, sel_mine, n_e, bs, p, scale_log2, smem + w * kUnit * SM::RS,
                                 w, NW, m_run, l_run, o, cache);
  l_run = sum_col4(l_run);

  // combine the waves' states in LDS (wave order), rotate the combined O
  // back, then write the output (one slice) or the slice state
  __syncthreads();  // staging area becomes the combine area
  float* cm = reinterpret_cast<float*>(smem);  // [NW][16] running maxima
  float* cl = cm + NW * 16;                    // [NW][16] sums
  constexpr int CS = kCombStride<D>;           // padded row stride (conflict-free 16-byte writes)
  float* co = cl + NW * 16;                    // [NW][16][CS] unnormalised outputs
  if (lane < 16) {
    cm[w * 16 + col] = m_run;
    cl[w * 16 + col] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) co[(w * 16 + col) * CS + 16 * dt + 4 * lg + i] = o[dt][i];
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += NT) {
    const int h = idx / D, e = idx % D;
    float M = -__builtin_inff();
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, cm[ww * 16 + h]);
    float L = 0.f, O = 0.f;
    if (M != -__builtin_inff()) {  // a slice may hold no visible key
      for (int ww = 0; ww < NW; ++ww) {
        const float f = __builtin_amdgcn_exp2f(cm[ww * 16 + h] - M);
        L += f * cl[ww * 16 + h];
        O += f * co[(ww * 16 + h) * CS + e];
      }
    }
    if (e == 0) {
      comb_m[h] = M;
      comb_l[h] = L;
    }
    comb_o[idx] = O;
  }
  __syncthreads();
  constexpr float inv_d = 1.0f / D;  // exact: D is a power of two
  for (int h = w; h < G; h += NW) {
    float x[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) x[i] = comb_o[h * D + lane + kWave * i];
    fwht_wave<D>(x);
#pragma unroll
    for (int i = 0; i < EPL; ++i) comb_o[h * D + lane + kWave * i] = x[i] * inv_d;
  }
  __syncthreads();

  if (n_split == 1) {
    for (int idx = tid; idx < G * D; idx += NT) {
      const int h = idx / D, e = idx % D;
      out[(b * hq + (int64_t)g * G + h) * D + e] = f32_to_bf16(comb_o[idx] / comb_l[h]);
    }
    return;
  }
  // several slices: this slice's state with device-coherent stores, a
  // ticket, and the last workgroup of the row merges (as the bf16 decode)
  const int stride = 2 * G + G * D;
  const auto prs = __builtin_amdgcn_make_buffer_rsrc(part + row * (int64_t)n_split * stride, 0,
                                                     n_split * stride * 4, kBufferFlags);
  const int soff = split * stride;
  for (int idx = tid; idx < G * D; idx += NT) {
    const int h = idx / D, e = idx % D;
    if (e == 0) {
      store_coherent(prs, soff + h, __float_as_uint(comb_m[h]));
      store_coherent(prs, soff + G + h, __float_as_uint(comb_l[h]));
    }
    store_coherent(prs, soff + 2 * G + idx, __float_as_uint(comb_o[idx]));
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counters + row, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev == (uint32_t)(n_split - 1);
    if (last) __hip_atomic_store(counters + row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_wg = last ? 1 : 0;
  }
  __syncthreads();
  if (!last_wg) return;
  if (G * (D / 4) <= NT) merge_slices<D, 1, 16, NT>(prs, smem, out, b, g, hq, G, n_split, tid);
  else merge_slices<D, 2, 8, NT>(prs, smem, out, b, g, hq, G, n_split, tid);
}

// Prefill rows over the rotated quantized cache: one 8-wave workgroup per
// (sequence, query row, KV head), as the bf16 prefill runs the shapes its
// tiled kernel does not serve. The row's query heads are rotated into LDS,
// its whole selection is attended in chunks of 64 entries (one per lane)
// with the codes widened on load, causal at the row's own position, and the
// waves' combined output is rotated back (H O / d) and written.
template <int D>
__global__ __launch_bounds__(8 * kWave) void prefill_rows_q8_kernel(
    const uint16_t* __restrict__ q, const int8_t* __restrict__ kq, const int8_t* __restrict__ vq,
    const uint16_t* __restrict__ ks, const uint16_t* __restrict__ vs_, const int32_t* __restrict__ sel,
    uint16_t* __restrict__ out, int64_t q_len, int64_t q_pos0, int64_t kv_cap, int hq, int hkv, int G, int bs,
    int top_k, float scale_log2) {
  constexpr int NW = 8;
  constexpr int EPL = D / kWave;
  constexpr int DT = D / 16;
  constexpr int RS = kStageRowBytes<D>;
  constexpr int kStage = NW * kUnit * RS;
  constexpr int kComb = (NW + 1) * (32 + 16 * kCombStride<D>) * 4;  // waves' states, then the rotated-back row
  __shared__ __align__(16) unsigned char smem[kStage > kComb ? kStage : kComb];
  __shared__ __align__(16) uint16_t qrot[16 * D];
  __shared__ int last_wg;

  const int64_t row = blockIdx.x;  // ((b * q_len) + t) * hkv + g
  const int64_t bt = row / hkv;    // b * q_len + t
  const int g = (int)(row % hkv);
  const int64_t b = bt / q_len;
  const int64_t p = q_pos0 + bt % q_len;  // the row's absolute position
  const int lane = lane_id(), w = wave_id();
  const int64_t kv_off = ((int64_t)b * hkv + g) * kv_cap;

  const uint16_t* qh = q + (bt * hq + (int64_t)g * G) * D;
  for (int h = w; h < G; h += NW) {
    float x[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) x[i] = bf16_to_f32(qh[(int64_t)h * D + lane + kWave * i]);
    fwht_wave<D>(x);
#pragma unroll
    for (int i = 0; i < EPL; ++i) qrot[h * D + lane + kWave * i] = f32_to_bf16(x[i]);
  }
  __syncthreads();
  u32x4_t qf[D / 32];
  load_q8_query_operands<D>(qrot, G, qf);  // the cache's dim order (attend_units' 8-bit loads)

  float m_run = -__builtin_inff(), l_run = 0.f;
  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const Q8Cache cache{kq + kv_off * D, vq + kv_off * D, ks + kv_off * (D / 32), vs_ + kv_off * (D / 32)};
  const int32_t* sel_row = sel + row * top_k;
  for (int e0 = 0; e0 < top_k; e0 += kWave) {
    const int n_e = top_k - e0 < kWave ? top_k - e0 : kWave;
    const int sel_mine = lane < n_e ? sel_row[e0 + lane] : -1;
    if (bs < kUnit)  // rows gathered from several entries per unit
      attend_units<D, true, true>(qf, nullptr, nullptr, sel_mine, n_e, bs, p, scale_log2, smem + w * kUnit * RS, w,
                                  NW, m_run, l_run, o, cache);
    else
      attend_units<D, false, true>(qf, nullptr, nullptr, sel_mine, n_e, bs, p, scale_log2, smem + w * kUnit * RS, w,
                                   NW, m_run, l_run, o, cache);
  }
  l_run = sum_col4(l_run);
  finish_row_slice<D, NW, true>(m_run, l_run, o, smem, &last_wg, out, nullptr, nullptr, row, bt, g, hq, G, 0, 1);
}

// The 8-bit cache rotated back into bf16 rows, for prefill over the cache
// with the tiled bf16 kernel: position pos of every (sequence, KV head) of K
// and of V is dequantized (code x scale, exact in float32), transformed by H
// and divided by D (H H = D I, so this undoes the cache's rotation; the
// scores and the output of attention over these rows are those over the
// rotated rows with the query rotated and the output rotated back), and
// rounded to bf16. Rows [n_pos, n_pad) are written as zeros. One wave per
// row; lane l holds elements l (and l + 64).
template <int D>
__global__ __launch_bounds__(256) void dequant_unrotate_kernel(
    const int8_t* __restrict__ kq, const int8_t* __restrict__ vq, const uint16_t* __restrict__ ks,
    const uint16_t* __restrict__ vs, uint16_t* __restrict__ k_out, uint16_t* __restrict__ v_out, int64_t kv_cap,
    int64_t n_pos, int64_t n_pad, int64_t n_rows) {
  constexpr int EPL = D / kWave;
  const int64_t item = (int64_t)blockIdx.x * 4 + wave_id();  // tensor (K, then V), (sequence, KV head), position
  if (item >= 2 * n_rows * n_pad) return;
  const int tensor = (int)(item / (n_rows * n_pad));
  const int64_t rem = item % (n_rows * n_pad);
  const int64_t bg = rem / n_pad, pos = rem % n_pad;
  const int lane = lane_id();
  uint16_t* dst = (tensor ? v_out : k_out) + (bg * n_pad + pos) * D;
  if (pos >= n_pos) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) dst[lane + kWave * i] = 0;
    return;
  }
  const int8_t* codes = (tensor ? vq : kq) + (bg * kv_cap + pos) * D;
  const uint16_t* sc = (tensor ? vs : ks) + (bg * kv_cap + pos) * (D / 32);
  float x[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    x[i] = (float)codes[e] * f16_bits_to_f32(sc[e / 32]);
  }
  fwht_wave<D>(x);
  constexpr float inv_d = 1.0f / D;  // exact: D is a power of two
#pragma unroll
  for (int i = 0; i < EPL; ++i) dst[lane + kWave * i] = f32_to_bf16(x[i] * inv_d);
}

template <int D>
hipError_t launch_prefill_q8_d(const Dims& s, const void* q, const int8_t* kq, const int8_t* vq, const uint16_t* ks,
                               const uint16_t* vs, int64_t q_len, int64_t q_pos0, int64_t kv_cap, const int32_t* sel,
                               void* out, hipStream_t st) {
  const int64_t rows = (int64_t)s.batch * q_len * s.hkv;
  // (H q).(H k) = d q.k: the 1/d of the rotation is folded into the scale
  const float scale_log2 = s.scale * 1.4426950408889634f / (float)D;
  hipLaunchKernelGGL((prefill_rows_q8_kernel<D>), dim3((unsigned)rows), dim3(8 * kWave), 0, st,
                     static_cast<const uint16_t*>(q), kq, vq, ks, vs, sel, static_cast<uint16_t*>(out), q_len,
                     q_pos0, kv_cap, s.hq, s.hkv, s.group, s.bs, s.top_k, scale_log2);
  return hipGetLastError();
}

template <int D>
hipError_t launch_quant_d(const void* k, const void* v, int8_t* kq, int8_t* vq, uint16_t* ks, uint16_t* vs,
                          int64_t kv_cap, int64_t pos_begin, int64_t n_pos, int64_t rows, hipStream_t st) {
  const int64_t n_items = rows * n_pos;
  hipLaunchKernelGGL((kv_quantize_kernel<D>), dim3((unsigned)((2 * n_items + 3) / 4)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), kq, vq, ks, vs, kv_cap,
                     pos_begin, n_pos, n_items);
  return hipGetLastError();
}

template <int D>
hipError_t launch_q8_d(const Dims& s, const DecodePlan& plan, const void* q, const int8_t* kq, const int8_t* vq,
                       const uint16_t* ks, const uint16_t* vs, int64_t kv_len, int64_t kv_cap, const int32_t* sel,
                       void* out, void* counters_ws, void* part_ws, hipStream_t st) {
  const int64_t rows = (int64_t)s.batch * s.hkv;
  // (H q).(H k) = d q.k: the 1/d of the rotation is folded into the scale
  const float scale_log2 = s.scale * 1.4426950408889634f / (float)D;
  uint32_t* counters = static_cast<uint32_t*>(counters_ws);
  float* part = plan.n_split > 1 ? static_cast<float*>(part_ws) : nullptr;
  auto kern = plan.waves == 8 ? decode_attn_q8_kernel<D, 8> : decode_attn_q8_kernel<D, 4>;
  hipLaunchKernelGGL(kern, dim3((unsigned)(rows * plan.n_split)), dim3(plan.waves * kWave), 0, st,
                     static_cast<const uint16_t*>(q), kq, vq, ks, vs, sel, static_cast<uint16_t*>(out), part,
                     counters, kv_len, kv_cap, s.hq, s.hkv, s.group, s.bs, s.top_k, scale_log2, plan.blocks_per_wg,
                     plan.n_split);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_quantize(const Dims& s, const void* k, const void* v, int64_t kv_cap, int64_t pos_begin,
                              int64_t pos_end, int8_t* kq, int8_t* vq, uint16_t* ks, uint16_t* vs, hipStream_t st) {
  const int64_t n_pos = pos_end - pos_begin;
  if (n_pos <= 0) return hipSuccess;
  const int64_t rows = (int64_t)s.batch * s.hkv;
  return s.d == 64 ? launch_quant_d<64>(k, v, kq, vq, ks, vs, kv_cap, pos_begin, n_pos, rows, st)
                   : launch_quant_d<128>(k, v, kq, vq, ks, vs, kv_cap, pos_begin, n_pos, rows, st);
}

hipError_t launch_decode_q8(const Dims& s, const DecodePlan& plan, const void* q, const int8_t* kq, const int8_t* vq,
                            const uint16_t* ks, const uint16_t* vs, int64_t kv_len, int64_t kv_cap,
                            const int32_t* sel, void* out, void* counters, void* part, hipStream_t st) {
  return s.d == 64 ? launch_q8_d<64>(s, plan, q, kq, vq, ks, vs, kv_len, kv_cap, sel, out, counters, part, st)
                   : launch_q8_d<128>(s, plan, q, kq, vq, ks, vs, kv_len, kv_cap, sel, out, counters, part, st);
}

hipError_t launch_dequant_unrotate(const Dims& s, const int8_t* kq, const int8_t* vq, const uint16_t* ks,
                                  const uint16_t* vs, int64_t kv_cap, int64_t n_pos, int64_t n_pad, uint16_t* k_out,
                                  uint16_t* v_out, hipStream_t st) {
  const int64_t n_rows = (int64_t)s.batch * s.hkv;
  const unsigned grid = (unsigned)((2 * n_rows * n_pad + 3) / 4);
  if (s.d == 64)
    hipLaunchKernelGGL((dequant_unrotate_kernel<64>), dim3(grid), dim3(256), 0, st, kq, vq, ks, vs, k_out, v_out,
                       kv_cap, n_pos, n_pad, n_rows);
  else
    hipLaunchKernelGGL((dequant_unrotate_kernel<128>), dim3(grid), dim3(256), 0, st, kq, vq, ks, vs, k_out, v_out,
                       kv_cap, n_pos, n_pad, n_rows);
  return hipGetLastError();
}

hipError_t launch_prefill_q8(const Dims& s, const void* q, const int8_t* kq, const int8_t* vq, const uint16_t* ks,
                             const uint16_t* vs, int64_t q_len, int64_t q_pos0, int64_t kv_cap, const int32_t* sel,
                             void* out, hipStream_t st) {
  return s.d == 64 ? launch_prefill_q8_d<64>(s, q, kq, vq, ks, vs, q_len, q_pos0, kv_cap, sel, out, st)
                   : launch_prefill_q8_d<128>(s, q, kq, vq, ks, vs, q_len, q_pos0, kv_cap, sel, out, st);
}

}  // namespace qsa
