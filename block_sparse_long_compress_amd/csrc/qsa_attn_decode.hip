// Sparse attention for one query token per sequence over its selected blocks
// ("Qwen4 in llama.cpp: Dissecting PR #27742", section "QSA Is an
// Address-Selection Problem, Not a New Attention Equation": ordinary softmax
// attention restricted to the cells the selector returned).
//
// The per-wave unit loop (bf16 MFMA, float32 online softmax, gathered units
// for blocks shorter than 32 keys) is in qsa_decode_unit.h.
//
// Grid: one workgroup (4 waves) per (sequence, KV head, slice of the
// selection list). Waves take units round-robin; the workgroup merges its
// waves' partial softmax states in LDS and writes the output directly when a
// row has one slice. Otherwise it writes its partial state to the workspace
// at the device-coherent level and takes a ticket from the row's arrival
// counter; the last workgroup of the row merges all slices in slice order
// and resets the counter to zero. The merge order is fixed, so results are
// bitwise reproducible whichever workgroup arrives last.
#include "qsa_decode_unit.h"
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

template <int D>
struct DecodeSmem {
  static constexpr int RS = kStageRowBytes<D>;
  static constexpr int kStage = 4 * kUnit * RS;
  static constexpr int kComb = 4 * (32 + 16 * D) * 4;
  static constexpr int kBytes = kStage > kComb ? kStage : kComb;
};

template <int D, bool GATHER>
__global__ __launch_bounds__(256) void decode_attn_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v, const int32_t* __restrict__ sel,
                                                          uint16_t* __restrict__ out, float* __restrict__ part,
                                                          uint32_t* __restrict__ counters, int64_t kv_len,
                                                          int64_t kv_cap, int hq, int hkv, int G, int bs, int top_k,
                                                          float scale_log2, int bpw, int n_split) {
  using SM = DecodeSmem<D>;
  constexpr int RS = SM::RS;
  constexpr int KS = D / 32;  // 32-wide K steps of the QK^T product
  constexpr int DT = D / 16;  // 16-wide dim tiles of the PV product
  __shared__ __align__(16) unsigned char smem[SM::kBytes];
  __shared__ int last_wg;

  const int64_t row = blockIdx.x / n_split;
  const int split = blockIdx.x % n_split;
  const int64_t b = row / hkv;
  const int g = (int)(row % hkv);
  const int lane = lane_id(), w = wave_id(), tid = threadIdx.x;
  const int lg = lane / 16, col = lane % 16;
  const int64_t p = kv_len - 1;
  const int e0 = split * bpw;
  const int e1 = e0 + bpw < top_k ? e0 + bpw : top_k;
  const int n_e = e1 - e0;
  const int32_t* sel_row = sel + row * top_k;
  const int64_t kv_off = ((int64_t)b * hkv + g) * kv_cap;

  u32x4_t qf[KS];
  load_q_operands<D>(q + (b * hq + (int64_t)g * G) * D, G, qf);

  float m_run = -__builtin_inff(), l_run = 0.f;
  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  unsigned char* vs = smem + w * kUnit * RS;

  // The slice's block ids, one per lane (bpw <= 64), loaded with Q.
  const int sel_mine = lane < e1 - e0 ? sel_row[e0 + lane] : -1;

  attend_units<D, GATHER>(qf, k + kv_off * D, v + kv_off * D, sel_mine, n_e, bs, p, scale_log2, vs, w, 4, m_run,
                         l_run, o);

  l_run = sum_col4(l_run);
  __syncthreads();  // staging area becomes the combine area
  float* cm = reinterpret_cast<float*>(smem);  // [4][16] running maxima
  float* cl = cm + 4 * 16;                     // [4][16] sums
  float* co = cl + 4 * 16;                     // [4][16][D] unnormalised outputs
  if (lane < 16) {
    cm[w * 16 + col] = m_run;
    cl[w * 16 + col] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) co[(w * 16 + col) * D + 16 * dt + 4 * lg + i] = o[dt][i];
  __syncthreads();

  if (n_split == 1) {
    for (int idx = tid; idx < G * D; idx += 256) {
      const int h = idx / D, e = idx % D;
      float M = -__builtin_inff();
      for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, cm[ww * 16 + h]);
      float L = 0.f, O = 0.f;
      for (int ww = 0; ww < 4; ++ww) {
        const float f = __builtin_amdgcn_exp2f(cm[ww * 16 + h] - M);
        L += f * cl[ww * 16 + h];
        O += f * co[(ww * 16 + h) * D + e];
      }
      out[(b * hq + (int64_t)g * G + h) * D + e] = f32_to_bf16(O / L);
    }
    return;
  }

  // Several slices per row: this slice's state goes out with stores that
  // reach the device-coherent level (cache policy sc1: no L2 write-back
  // needed), then one ticket per workgroup; the last workgroup of the row
  // to arrive merges every slice in order and resets the row's counter.
  const int stride = 2 * G + G * D;  // floats per slice: maxima, sums, outputs
  const auto prs = __builtin_amdgcn_make_buffer_rsrc(part + row * (int64_t)n_split * stride, 0,
                                                     n_split * stride * 4, kBufferFlags);
  const int soff = split * stride;
  for (int idx = tid; idx < G * D; idx += 256) {
    const int h = idx / D, e = idx % D;
    float M = -__builtin_inff();
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, cm[ww * 16 + h]);
    float L = 0.f, O = 0.f;
    if (M != -__builtin_inff()) {  // a slice may hold no visible key
      for (int ww = 0; ww < 4; ++ww) {
        const float f = __builtin_amdgcn_exp2f(cm[ww * 16 + h] - M);
        L += f * cl[ww * 16 + h];
        O += f * co[(ww * 16 + h) * D + e];
      }
    }
    if (e == 0) {
      store_coherent(prs, soff + h, __float_as_uint(M));
      store_coherent(prs, soff + G + h, __float_as_uint(L));
    }
    store_coherent(prs, soff + 2 * G + h * D + e, __float_as_uint(O));
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

  // 64 registers of staged values per batch: 16 slices for one group of 4
  // dims per thread, 8 slices for two (G = 16 at d = 128)
  if (G * (D / 4) <= 256) merge_slices<D, 1, 16, 256>(prs, smem, out, b, g, hq, G, n_split, tid);
  else merge_slices<D, 2, 8, 256>(prs, smem, out, b, g, hq, G, n_split, tid);
}

template <int D>
hipError_t launch_d(const Dims& s, const DecodePlan& plan, const void* q, const void* k, const void* v,
                    int64_t kv_len, int64_t kv_cap, const int32_t* sel, void* out, uint32_t* counters, float* part,
                    hipStream_t st) {
  const int64_t rows = (int64_t)s.batch * s.hkv;
  const float scale_log2 = s.scale * 1.4426950408889634f;
  auto kern = s.bs < kUnit ? decode_attn_kernel<D, true> : decode_attn_kernel<D, false>;
  if (plan.n_split == 1) part = nullptr;
  hipLaunchKernelGGL(kern, dim3((unsigned)(rows * plan.n_split)), dim3(256), 0, st, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), sel,
                     static_cast<uint16_t*>(out), part, counters, kv_len, kv_cap, s.hq, s.hkv, s.group, s.bs, s.top_k,
                     scale_log2, plan.blocks_per_wg, plan.n_split);
  return hipGetLastError();
}

}  // namespace

DecodePlan plan_decode(const Dims& s, int64_t kv_len) {
  (void)kv_len;
  DecodePlan p{};
  const int64_t rows = (int64_t)s.batch * s.hkv;
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

hipError_t launch_decode(const Dims& s, const DecodePlan& plan, const void* q, const void* k, const void* v,
                         int64_t kv_len, int64_t kv_cap, const int32_t* sel, void* out, void* counters, void* part,
                         hipStream_t st) {
  uint32_t* c = static_cast<uint32_t*>(counters);
  float* pt = static_cast<float*>(part);
  return s.d == 64 ? launch_d<64>(s, plan, q, k, v, kv_len, kv_cap, sel, out, c, pt, st)
                   : launch_d<128>(s, plan, q, k, v, kv_len, kv_cap, sel, out, c, pt, st);
}

}  // namespace qsa
