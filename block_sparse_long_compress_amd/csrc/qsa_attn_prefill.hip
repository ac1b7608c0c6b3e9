// Causal sparse attention for a run of query tokens, each attending over its
// own selected blocks ("Qwen4 in llama.cpp: Dissecting PR #27742", section
// "QSA Is an Address-Selection Problem, Not a New Attention Equation":
// ordinary attention over the selected cells, causal inside the own block).
//
// bf16 MFMA (v_mfma_f32_16x16x32_bf16) with float32 online softmax.
//
// Shape of the work. Every (token, KV head) has its own selection, shared by
// the G query heads of the group, so one token supplies only G MFMA columns.
// A column group (CG) packs 16/G consecutive tokens into the 16 N-columns;
// for a key block that only some of a CG's tokens selected, the other
// columns are masked (their MFMA work is wasted, the cost of per-token
// selection with GQA). The keys form the 16-row M side: S^T = K Q^T, then
// O^T += V^T P^T, with P^T taken from the S^T accumulators without any lane
// exchange (see kkey()).
//
// A workgroup owns W*NCG CGs of consecutive tokens of one (sequence, KV head)
// and walks the union of their selections in ascending block order. Each
// block's K rows and V^T fragments are staged once in LDS (double-buffered,
// the next block's global loads in flight while the current one is
// computed) and reused by every CG of the workgroup that selected it. Each
// token tracks its position in its ascending selection list, so membership
// is one LDS compare per block.
//
// V^T operand fragments come from vt_pack_kernel, which writes V in exactly
// the lane order the PV product consumes (one 16-byte LDS read per fragment).
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kUnit = 32;

__device__ __forceinline__ int kkey(int lg, int j) { return j < 4 ? 4 * lg + j : 12 + 4 * lg + j; }

// vt[(bg * n_units + u) * (D/16) + dt][lane][j] = V[32u + kkey(lane/16, j)][16 dt + lane % 16]
// (zero past kv_total). One wave per 32-key unit.
template <int D>
__global__ __launch_bounds__(256) void vt_pack_kernel(const uint16_t* __restrict__ v, uint16_t* __restrict__ vt,
                                                      int64_t kv_cap, int64_t kv_total, int64_t n_units,
                                                      int64_t n_items) {
  constexpr int RS = 2 * D + 16;
  __shared__ __align__(16) unsigned char smem[4 * kUnit * RS];
  const int64_t item = (int64_t)blockIdx.x * 4 + wave_id();
  if (item >= n_items) return;
  const int64_t bg = item / n_units, u = item % n_units;
  const int lane = lane_id(), lg = lane / 16, col = lane % 16;
  unsigned char* vs = smem + wave_id() * kUnit * RS;
  const int64_t key0 = u * kUnit;
  const uint16_t* vb = v + (bg * kv_cap + key0) * D;
  constexpr int VCH = kUnit * D / 8 / kWave;
  u32x4_t vr[VCH];
#pragma unroll
  for (int j = 0; j < VCH; ++j) {
    const int ci = lane + kWave * j;
    const int r = ci / (D / 8), c8 = ci % (D / 8);
    vr[j] = key0 + r < kv_total ? *reinterpret_cast<const u32x4_t*>(vb + (int64_t)r * D + 8 * c8)
                                : u32x4_t{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int j = 0; j < VCH; ++j) {
    const int ci = lane + kWave * j;
    const int r = ci / (D / 8), c8 = ci % (D / 8);
    *reinterpret_cast<u32x4_t*>(vs + r * RS + 16 * c8) = vr[j];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint16_t* dst = vt + item * (D / 16) * kWave * 8;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const unsigned char* src = vs + 2 * (16 * dt + col);
    uint32_t wv[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t lo = *reinterpret_cast<const uint16_t*>(src + kkey(lg, 2 * h) * RS);
      const uint32_t hi = *reinterpret_cast<const uint16_t*>(src + kkey(lg, 2 * h + 1) * RS);
      wv[h] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4_t*>(dst + ((int64_t)dt * kWave + lane) * 8) = u32x4_t{wv[0], wv[1], wv[2], wv[3]};
  }
}

struct PrefillSmem {
  int k_bytes, vt_bytes, sel_off, mask_off, total;
};

template <int D>
__host__ __device__ inline PrefillSmem prefill_smem(int bs, int qt, int top_k, int n_words) {
  PrefillSmem s;
  s.k_bytes = bs * (2 * D + 16);
  s.vt_bytes = (bs / kUnit) * (D / 16) * kWave * 16;
  s.sel_off = 2 * s.k_bytes + 2 * s.vt_bytes;
  s.mask_off = s.sel_off + qt * top_k * 4;
  s.total = s.mask_off + n_words * 4;
  return s;
}

template <int D, int W, int NCG>
__global__ __launch_bounds__(W * 64) void prefill_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ vt,
    const int32_t* __restrict__ sel, uint16_t* __restrict__ out, int64_t q_len, int64_t q_pos0, int64_t kv_cap,
    int64_t n_units, int hq, int hkv, int G, int bs, int top_k, float scale_log2) {
  constexpr int KRS = 2 * D + 16;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int NT = W * 64;
  extern __shared__ __align__(16) unsigned char smem[];

  const int tpc = 16 / G;
  const int qt = W * NCG * tpc;
  const int64_t tile = (int64_t)gridDim.x - 1 - blockIdx.x;  // longest tiles (latest tokens) first
  const int64_t t0 = tile * qt;
  const int g = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int lg = lane / 16, col = lane % 16;
  const int64_t rows = q_len - t0 < qt ? q_len - t0 : qt;
  const int64_t kv_total = q_pos0 + q_len;
  const int64_t own_last = (q_pos0 + t0 + rows - 1) / bs;
  const int n_words = (int)(own_last / 32) + 1;
  const PrefillSmem L = prefill_smem<D>(bs, qt, top_k, n_words);
  int32_t* sel_lds = reinterpret_cast<int32_t*>(smem + L.sel_off);
  uint32_t* mask = reinterpret_cast<uint32_t*>(smem + L.mask_off);

  for (int i = tid; i < n_words; i += NT) mask[i] = 0u;
  __syncthreads();
  for (int64_t i = tid; i < rows * top_k; i += NT) {
    const int64_t r = i / top_k, e = i % top_k;
    const int32_t c = sel[((b * q_len + t0 + r) * hkv + g) * top_k + e];
    sel_lds[i] = c;
    if (c >= 0 && (int64_t)c <= (q_pos0 + t0 + r) / bs) atomicOr(&mask[c >> 5], 1u << (c & 31));
  }
  __syncthreads();

  // Per CG: this lane's column token, its position and selection cursor.
  u32x4_t qf[NCG][KS];
  f32x4_t o[NCG][DT];
  float m_run[NCG], l_run[NCG];
  int cursor[NCG];
  int64_t pos_q[NCG];
  bool row_ok[NCG];
  int rloc[NCG];
#pragma unroll
  for (int n = 0; n < NCG; ++n) {
    rloc[n] = (w * NCG + n) * tpc + col / G;
    row_ok[n] = rloc[n] < rows;
    pos_q[n] = q_pos0 + t0 + rloc[n];
    cursor[n] = 0;
    m_run[n] = -__builtin_inff();
    l_run[n] = 0.f;
    const uint16_t* qs = q + ((b * q_len + t0 + rloc[n]) * hq + (int64_t)g * G + col % G) * D + 8 * lg;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[n][s] = row_ok[n] ? *reinterpret_cast<const u32x4_t*>(qs + 32 * s) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[n][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  auto next_block = [&](int64_t after) -> int64_t {
    int64_t c = after + 1;
    int wd = (int)(c >> 5);
    if (wd >= n_words) return -1;
    uint32_t bits = mask[wd] & (~0u << (c & 31));
    while (bits == 0u) {
      if (++wd >= n_words) return -1;
      bits = mask[wd];
    }
    return (int64_t)wd * 32 + __builtin_ctz(bits);
  };

  const uint16_t* kg_base = k + ((b * hkv + g) * kv_cap) * D;
  const uint16_t* vt_base = vt + ((b * hkv + g) * n_units) * DT * kWave * 8;
  const int k_chunks = bs * D / 8;
  const int v_chunks = (bs / kUnit) * DT * kWave;
  constexpr int MAXCH = 4;  // per-thread staging chunks (checked on the host)
  u32x4_t kreg[MAXCH], vreg[MAXCH];

  auto stage_load = [&](int64_t c) {
#pragma unroll
    for (int j = 0; j < MAXCH; ++j) {
      const int ci = tid + NT * j;
      kreg[j] = u32x4_t{0u, 0u, 0u, 0u};
      if (ci < k_chunks) {
        const int r = ci / (D / 8), c8 = ci % (D / 8);
        const int64_t pos = c * bs + r;
        if (pos < kv_total) kreg[j] = *reinterpret_cast<const u32x4_t*>(kg_base + pos * D + 8 * c8);
      }
      if (ci < v_chunks)
        vreg[j] = *reinterpret_cast<const u32x4_t*>(vt_base + (c * (bs / kUnit) * DT * kWave + ci) * 8);
    }
  };
  auto stage_store = [&](int par) {
    unsigned char* kb = smem + par * L.k_bytes;
    unsigned char* vb = smem + 2 * L.k_bytes + par * L.vt_bytes;
#pragma unroll
    for (int j = 0; j < MAXCH; ++j) {
      const int ci = tid + NT * j;
      if (ci < k_chunks) {
        const int r = ci / (D / 8), c8 = ci % (D / 8);
        *reinterpret_cast<u32x4_t*>(kb + r * KRS + 16 * c8) = kreg[j];
      }
      if (ci < v_chunks) *reinterpret_cast<u32x4_t*>(vb + 16 * ci) = vreg[j];
    }
  };

  int64_t c = next_block(-1);
  if (c >= 0) stage_load(c);
  int par = 0;
  while (c >= 0) {
    stage_store(par);
    __syncthreads();
    const int64_t c_next = next_block(c);
    if (c_next >= 0) stage_load(c_next);

    const unsigned char* kb = smem + par * L.k_bytes;
    const unsigned char* vb = smem + 2 * L.k_bytes + par * L.vt_bytes;
    bool mem[NCG];
    bool any = false;
#pragma unroll
    for (int n = 0; n < NCG; ++n) {
      mem[n] = row_ok[n] && cursor[n] < top_k && sel_lds[rloc[n] * top_k + cursor[n]] == (int32_t)c;
      any |= __ballot(mem[n]) != 0;
    }
    if (any) {
      for (int u = 0; u < bs / kUnit; ++u) {
        const int64_t key0 = c * bs + (int64_t)u * kUnit;
        bool need[NCG];
        bool any_u = false;
#pragma unroll
        for (int n = 0; n < NCG; ++n) {
          need[n] = __ballot(mem[n] && key0 <= pos_q[n]) != 0;
          any_u |= need[n];
        }
        if (!any_u) continue;
        f32x4_t sacc[NCG][2];
#pragma unroll
        for (int n = 0; n < NCG; ++n) sacc[n][0] = sacc[n][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const unsigned char* kr = kb + (kUnit * u + col) * KRS + 2 * (32 * s + 8 * lg);
          const u32x4_t k0 = *reinterpret_cast<const u32x4_t*>(kr);
          const u32x4_t k1 = *reinterpret_cast<const u32x4_t*>(kr + 16 * KRS);
#pragma unroll
          for (int n = 0; n < NCG; ++n) {
            if (!need[n]) continue;
            sacc[n][0] = mfma_bf16(k0, qf[n][s], sacc[n][0]);
            sacc[n][1] = mfma_bf16(k1, qf[n][s], sacc[n][1]);
          }
        }
        u32x4_t pf[NCG];
#pragma unroll
        for (int n = 0; n < NCG; ++n) {
          if (!need[n]) continue;
          float x[2][4];
          float mloc = -__builtin_inff();
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bool ok = mem[n] && key0 + 16 * st + 4 * lg + i <= pos_q[n];
              x[st][i] = ok ? sacc[n][st][i] * scale_log2 : -__builtin_inff();
              mloc = fmaxf(mloc, x[st][i]);
            }
          mloc = fmaxf(mloc, shfl_xor_f32(mloc, 16));
          mloc = fmaxf(mloc, shfl_xor_f32(mloc, 32));
          const float m_new = fmaxf(m_run[n], mloc);
          if (__ballot(m_new > m_run[n]) != 0) {
            const float alpha = m_run[n] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_run[n] - m_new);
            l_run[n] *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[n][dt] *= alpha;
          }
          m_run[n] = m_new;
          const float ms = m_new == -__builtin_inff() ? 0.f : m_new;
          float pr[2][4];
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              pr[st][i] = __builtin_amdgcn_exp2f(x[st][i] - ms);
              l_run[n] += pr[st][i];
            }
          pf[n] = u32x4_t{pack_bf16x2(pr[0][0], pr[0][1]), pack_bf16x2(pr[0][2], pr[0][3]),
                          pack_bf16x2(pr[1][0], pr[1][1]), pack_bf16x2(pr[1][2], pr[1][3])};
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const u32x4_t vf = *reinterpret_cast<const u32x4_t*>(vb + ((u * DT + dt) * kWave + lane) * 16);
#pragma unroll
          for (int n = 0; n < NCG; ++n) {
            if (!need[n]) continue;
            o[n][dt] = mfma_bf16(vf, pf[n], o[n][dt]);
          }
        }
      }
#pragma unroll
      for (int n = 0; n < NCG; ++n) cursor[n] += mem[n] ? 1 : 0;
    }
    par ^= 1;
    c = c_next;
  }

#pragma unroll
  for (int n = 0; n < NCG; ++n) {
    float l = l_run[n];
    l += shfl_xor_f32(l, 16);
    l += shfl_xor_f32(l, 32);
    if (!row_ok[n]) continue;
    const float inv = 1.0f / l;
    uint16_t* dst = out + ((b * q_len + t0 + rloc[n]) * hq + (int64_t)g * G + col % G) * D + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const u32x2_t pk = {pack_bf16x2(o[n][dt][0] * inv, o[n][dt][1] * inv),
                          pack_bf16x2(o[n][dt][2] * inv, o[n][dt][3] * inv)};
      *reinterpret_cast<u32x2_t*>(dst + 16 * dt) = pk;
    }
  }
}

constexpr int kW = 8;
constexpr int kNCG = 2;

template <int D>
hipError_t launch_d(const Dims& s, const PrefillPlan& plan, const void* q, const void* k, const void* v,
                    int64_t q_len, int64_t q_pos0, int64_t kv_cap, const int32_t* sel, void* out, void* ws,
                    hipStream_t st) {
  const int64_t kv_total = q_pos0 + q_len;
  const int64_t n_blocks = (kv_total + s.bs - 1) / s.bs;
  const int64_t n_units = n_blocks * (s.bs / kUnit);
  const int64_t bg = (int64_t)s.batch * s.hkv;
  uint16_t* vt = static_cast<uint16_t*>(ws);
  const int64_t items = bg * n_units;
  hipLaunchKernelGGL((vt_pack_kernel<D>), dim3((unsigned)((items + 3) / 4)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(v), vt, kv_cap, kv_total, n_units, items);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int qt = plan.rows_per_wg;
  const int n_words = (int)(((kv_total - 1) / s.bs) / 32) + 1;
  const PrefillSmem L = prefill_smem<D>(s.bs, qt, s.top_k, n_words);
  const float scale_log2 = s.scale * 1.4426950408889634f;
  dim3 grid((unsigned)((q_len + qt - 1) / qt), (unsigned)s.hkv, (unsigned)s.batch);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&prefill_attn_kernel<D, kW, kNCG>), hipFuncAttributeMaxDynamicSharedMemorySize,
      160 * 1024);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((prefill_attn_kernel<D, kW, kNCG>), grid, dim3(kW * 64), L.total, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), vt, sel,
                     static_cast<uint16_t*>(out), q_len, q_pos0, kv_cap, n_units, s.hq, s.hkv, s.group, s.bs,
                     s.top_k, scale_log2);
  return hipGetLastError();
}

}  // namespace

PrefillPlan plan_prefill(const Dims& s, int64_t q_len, int64_t q_pos0) {
  PrefillPlan p{};
  p.rows_per_wg = kW * kNCG * (16 / s.group);
  if (s.dtype != 1) {
    p.ws_bytes = 0;
    return p;
  }
  const int64_t kv_total = q_pos0 + q_len;
  const int64_t n_blocks = (kv_total + s.bs - 1) / s.bs;
  p.ws_bytes = (size_t)s.batch * s.hkv * n_blocks * s.bs * s.d * sizeof(uint16_t);
  return p;
}

// Largest LDS footprint the prefill kernel may need for these sizes.
int prefill_smem_bytes(const Dims& s, int64_t q_len, int64_t q_pos0) {
  const int64_t kv_total = q_pos0 + q_len;
  const int n_words = (int)(((kv_total - 1) / s.bs) / 32) + 1;
  const int qt = kW * kNCG * (16 / s.group);
  return s.d == 64 ? prefill_smem<64>(s.bs, qt, s.top_k, n_words).total
                   : prefill_smem<128>(s.bs, qt, s.top_k, n_words).total;
}

hipError_t launch_prefill(const Dims& s, const PrefillPlan& plan, const void* q, const void* k, const void* v,
                          int64_t q_len, int64_t q_pos0, int64_t kv_cap, const int32_t* sel, void* out, void* ws,
                          hipStream_t st) {
  return s.d == 64 ? launch_d<64>(s, plan, q, k, v, q_len, q_pos0, kv_cap, sel, out, ws, st)
                   : launch_d<128>(s, plan, q, k, v, q_len, q_pos0, kv_cap, sel, out, ws, st);
}

}  // namespace qsa
