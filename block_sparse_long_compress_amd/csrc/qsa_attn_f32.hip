// Float32 sparse attention (dtype QSA_F32), decode and prefill alike: one
// wave per (sequence, query row, KV head) walks the row's selected blocks
// in ascending order and runs an online softmax in float32 for each of the
// G query heads ("Qwen4 in llama.cpp: Dissecting PR #27742", section "QSA Is
// an Address-Selection Problem, Not a New Attention Equation"; the softmax
// form is the ordinary one of "Qwen Model Architecture: From Transformer to
// MoE", section "Attention: what the model is 'looking at'").
//
// Lane j scores key j of each 64-key slice (a full-precision dot product with
// the head's query, read from LDS), then every lane accumulates 1 or 2
// output dims over the slice's values. With kv_lens (a ragged decode batch,
// q_len = 1) sequence b's token sits at position kv_lens[b] - 1, clamped
// into [0, q_pos0]. The float32 path exists for exact
// parity on small fp32 workloads; the bf16 MFMA kernels are the fast path.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                      const float* __restrict__ v, const int32_t* __restrict__ sel,
                                                      float* __restrict__ out, int64_t q_len, int64_t q_pos0,
                                                      int64_t kv_cap, int hq, int hkv, int G, int bs, int top_k,
                                                      float scale, const int32_t* __restrict__ kv_lens) {
  constexpr int DPL = D / kWave;  // output dims per lane
  __shared__ float qh[D];
  const int64_t t = blockIdx.x;
  const int g = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int lane = lane_id();
  int64_t p = q_pos0 + t;
  if (kv_lens) {
    const int64_t n = kv_lens[b];
    p = (n < 1 ? 1 : (n > q_pos0 + 1 ? q_pos0 + 1 : n)) - 1;
  }
  const int64_t own = p / bs;
  const int32_t* srow = sel + ((b * q_len + t) * hkv + g) * top_k;
  const float* kb = k + ((b * hkv + g) * kv_cap) * D;
  const float* vb = v + ((b * hkv + g) * kv_cap) * D;

  for (int j = 0; j < G; ++j) {
    const int64_t h = (int64_t)g * G + j;
    const float* qsrc = q + ((b * q_len + t) * hq + h) * D;
    for (int e = lane; e < D; e += kWave) qh[e] = qsrc[e];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    float m = -__builtin_inff(), l = 0.f;
    float acc[DPL];
#pragma unroll
    for (int x = 0; x < DPL; ++x) acc[x] = 0.f;
    for (int e = 0; e < top_k; ++e) {
      const int64_t c = srow[e];
      if (c < 0) break;
      if (c > own) continue;  // not a visible block: never read past position p
      const int64_t len = c < own ? bs : p - own * bs + 1;
      for (int64_t k0 = 0; k0 < len; k0 += kWave) {
        const int64_t kk = k0 + lane;
        const bool ok = kk < len;
        float z = -__builtin_inff();
        if (ok) {
          const float* kr = kb + (c * bs + kk) * D;
          float dot = 0.f;
#pragma unroll 8
          for (int d = 0; d < D; ++d) dot = fmaf(qh[d], kr[d], dot);
          z = dot * scale;
        }
        const float m_new = fmaxf(m, wave_max_f32(z));
        const float alpha = m == -__builtin_inff() ? 0.f : expf(m - m_new);
        const float pz = ok ? expf(z - m_new) : 0.f;
        l = l * alpha + wave_sum_f32(pz);
#pragma unroll
        for (int x = 0; x < DPL; ++x) acc[x] *= alpha;
        const int64_t n = len - k0 < kWave ? len - k0 : kWave;
        for (int jj = 0; jj < n; ++jj) {
          const float pj = __shfl(pz, jj, kWave);
          const float* vr = vb + (c * bs + k0 + jj) * D;
#pragma unroll
          for (int x = 0; x < DPL; ++x) acc[x] = fmaf(pj, vr[lane + kWave * x], acc[x]);
        }
        m = m_new;
      }
    }
    float* dst = out + ((b * q_len + t) * hq + h) * D;
#pragma unroll
    for (int x = 0; x < DPL; ++x) dst[lane + kWave * x] = acc[x] / l;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

}  // namespace

hipError_t launch_attn_f32(const Dims& s, const float* q, const float* k, const float* v, int64_t q_len,
                           int64_t q_pos0, int64_t kv_cap, const int32_t* sel, float* out, hipStream_t st,
                           const int32_t* kv_lens) {
  dim3 grid((unsigned)q_len, (unsigned)s.hkv, (unsigned)s.batch);
  if (s.d == 64)
    hipLaunchKernelGGL((attn_f32_kernel<64>), grid, dim3(64), 0, st, q, k, v, sel, out, q_len, q_pos0, kv_cap, s.hq,
                       s.hkv, s.group, s.bs, s.top_k, s.scale, kv_lens);
  else
    hipLaunchKernelGGL((attn_f32_kernel<128>), grid, dim3(64), 0, st, q, k, v, sel, out, q_len, q_pos0, kv_cap, s.hq,
                       s.hkv, s.group, s.bs, s.top_k, s.scale, kv_lens);
  return hipGetLastError();
}

}  // namespace qsa
