// Sparse attention for one query token per sequence over its selected blocks
// ("Qwen4 in llama.cpp: Dissecting PR #27742", section "QSA Is an
// Address-Selection Problem, Not a New Attention Equation": ordinary softmax
// attention restricted to the cells the selector returned).
//
// bf16 inputs, bf16 MFMA (v_mfma_f32_16x16x32_bf16), float32 softmax and
// accumulation. Work unit = 32 keys: 32 consecutive keys of one selected
// block, or for blocks shorter than 32 keys (Bs = 4, 8, 16) the keys of
// 32/Bs consecutive entries of the selection list, each row addressed on
// its own (the position of every key row is computed once per unit and
// shared across lanes with ds_bpermute).
// Per unit a wave computes S^T = K Q^T with the keys as the 16-row M operand
// and the G query heads of the KV head as the N columns (G <= 16; columns
// >= G are zero queries and are ignored), keeps an online softmax per column
// in the exp2 domain, and accumulates O^T = V^T P^T. K fragments are loaded
// straight from HBM in operand layout (16 contiguous bytes per lane). V rows
// are staged in the wave's own LDS slice with coalesced loads and read back
// transposed, two bytes at a time, into the V^T operand.
//
// Grid: one workgroup (4 waves) per (sequence, KV head, slice of the
// selection list). Waves take units round-robin; the workgroup merges its
// waves' partial softmax states in LDS and writes the output directly when a
// row has one slice, else a partial state that decode_combine_kernel merges
// in slice order. No atomics: results are bitwise reproducible.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kUnit = 32;

// Element j of a lane's 8-wide K-dimension operand slot, for lane group lg,
// is key kkey(lg, j) of the 32-key unit. S^T tiles 0 and 1 hold keys
// 4*lg+i and 16+4*lg+i in lane group lg (MFMA output layout), so P^T can be
// fed to the PV product without any lane exchange.
__device__ __forceinline__ int kkey(int lg, int j) { return j < 4 ? 4 * lg + j : 12 + 4 * lg + j; }

template <int D>
struct DecodeSmem {
  static constexpr int RS = 2 * D + 16;  // LDS row stride of staged V (bytes)
  static constexpr int kStage = 4 * kUnit * RS;
  static constexpr int kComb = 4 * (32 + 16 * D) * 4;
  static constexpr int kBytes = kStage > kComb ? kStage : kComb;
};

template <int D, bool GATHER>
__global__ __launch_bounds__(256) void decode_attn_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v, const int32_t* __restrict__ sel,
                                                          uint16_t* __restrict__ out, float* __restrict__ part,
                                                          int64_t kv_len, int64_t kv_cap, int hq, int hkv, int G,
                                                          int bs, int top_k, float scale_log2, int bpw, int n_split) {
  using SM = DecodeSmem<D>;
  constexpr int RS = SM::RS;
  constexpr int KS = D / 32;  // 32-wide K steps of the QK^T product
  constexpr int DT = D / 16;  // 16-wide dim tiles of the PV product
  __shared__ __align__(16) unsigned char smem[SM::kBytes];

  const int64_t row = blockIdx.x / n_split;
  const int split = blockIdx.x % n_split;
  const int64_t b = row / hkv;
  const int g = (int)(row % hkv);
  const int lane = lane_id(), w = wave_id(), tid = threadIdx.x;
  const int lg = lane / 16, col = lane % 16;
  const int64_t p = kv_len - 1;
  const int upb = GATHER ? 1 : bs / kUnit;   // units per block
  const int bpu = GATHER ? kUnit / bs : 1;   // blocks per unit
  const int e0 = split * bpw;
  const int e1 = e0 + bpw < top_k ? e0 + bpw : top_k;
  const int n_e = e1 - e0;
  const int n_units = GATHER ? (n_e + bpu - 1) / bpu : n_e * upb;
  const int32_t* sel_row = sel + row * top_k;
  const int64_t kv_off = ((int64_t)b * hkv + g) * kv_cap;

  u32x4_t qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qf[s] = u32x4_t{0u, 0u, 0u, 0u};
    if (col < G) qf[s] = *reinterpret_cast<const u32x4_t*>(q + ((b * hq + (int64_t)g * G + col) * D + 32 * s + 8 * lg));
  }

  float m_run = -__builtin_inff(), l_run = 0.f;
  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  unsigned char* vs = smem + w * kUnit * RS;

  // The slice's block ids, one per lane (bpw <= 64), loaded with Q.
  const int sel_mine = lane < e1 - e0 ? sel_row[e0 + lane] : -1;

  // A wave's units are idx = w, w + 4, ...
  constexpr int VCH = kUnit * D / 8 / kWave;  // 16-byte V chunks per lane
  struct Unit {
    u32x4_t kf[2][KS];
    u32x4_t vr[VCH];
    int64_t key0;  // contiguous units: position of key row 0
    int mpos[2];   // gathered units: position of key row 16*st + 4*lg (-1: not visible)
    bool ok;
  };
  auto fetch = [&](int idx, Unit& u) {
    u.ok = false;
    if (idx >= n_units) return;
    if constexpr (GATHER) {
      // Row r of the unit is key r % Bs of slice entry idx*bpu + r/Bs; lanes
      // r and r + 32 compute it, every other lane fetches it with bpermute.
      // idx*bpu + r/Bs < 64: the slice holds at most 64 entries and bpu
      // divides 64.
      const int r = lane & (kUnit - 1);
      const int slot = idx * bpu + r / bs;
      const int c = __builtin_amdgcn_ds_bpermute(slot << 2, sel_mine);
      const int64_t pos = (int64_t)c * bs + (r % bs);
      const int rowpos = (slot < n_e && c >= 0 && pos <= p) ? (int)pos : -1;
      if (__ballot(rowpos >= 0) == 0) return;
      u.ok = true;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int kp = __builtin_amdgcn_ds_bpermute((16 * st + col) << 2, rowpos);
        u.mpos[st] = __builtin_amdgcn_ds_bpermute((16 * st + 4 * lg) << 2, rowpos);
        const uint16_t* kb = k + (kv_off + (kp >= 0 ? kp : 0)) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s)
          u.kf[st][s] = kp >= 0 ? *reinterpret_cast<const u32x4_t*>(kb + 32 * s + 8 * lg) : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < VCH; ++j) {
        const int ci = lane + kWave * j;
        const int rr = ci / (D / 8), c8 = ci % (D / 8);
        const int vp = __builtin_amdgcn_ds_bpermute(rr << 2, rowpos);
        u.vr[j] = vp >= 0 ? *reinterpret_cast<const u32x4_t*>(v + (kv_off + (vp >= 0 ? vp : 0)) * D + 8 * c8)
                          : u32x4_t{0u, 0u, 0u, 0u};
      }
    } else {
      const int c = __builtin_amdgcn_readlane(sel_mine, idx / upb);
      if (c < 0) return;
      u.key0 = (int64_t)c * bs + (int64_t)(idx % upb) * kUnit;
      if (u.key0 > p) return;
      u.ok = true;
      const uint16_t* kb = k + (kv_off + u.key0) * D;
      const uint16_t* vb = v + (kv_off + u.key0) * D;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int kr = 16 * st + col;
        const bool ok = u.key0 + kr <= p;
#pragma unroll
        for (int s = 0; s < KS; ++s)
          u.kf[st][s] = ok ? *reinterpret_cast<const u32x4_t*>(kb + (int64_t)kr * D + 32 * s + 8 * lg)
                           : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < VCH; ++j) {
        const int ci = lane + kWave * j;
        const int r = ci / (D / 8), c8 = ci % (D / 8);
        u.vr[j] = u.key0 + r <= p ? *reinterpret_cast<const u32x4_t*>(vb + (int64_t)r * D + 8 * c8)
                                  : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  auto consume = [&](const Unit& u) {
    if (!u.ok) return;
#pragma unroll
    for (int j = 0; j < VCH; ++j) {
      const int ci = lane + kWave * j;
      const int r = ci / (D / 8), c8 = ci % (D / 8);
      *reinterpret_cast<u32x4_t*>(vs + r * RS + 16 * c8) = u.vr[j];
    }

    f32x4_t sacc[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      sacc[st] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) sacc[st] = mfma_bf16(u.kf[st][s], qf[s], sacc[st]);
    }
    float x[2][4];
    float mloc = -__builtin_inff();
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // rows 16*st + 4*lg + i (i < 4) lie in one block of >= 4 keys
        const bool ok = GATHER ? (u.mpos[st] >= 0 && u.mpos[st] + i <= p) : (u.key0 + 16 * st + 4 * lg + i <= p);
        x[st][i] = ok ? sacc[st][i] * scale_log2 : -__builtin_inff();
        mloc = fmaxf(mloc, x[st][i]);
      }
    mloc = max_col4(mloc);
    const float m_new = fmaxf(m_run, mloc);  // finite: the unit has a visible key
    if (__ballot(m_new > m_run) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
    m_run = m_new;
    float pr[2][4];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[st][i] = __builtin_amdgcn_exp2f(x[st][i] - m_new);
        l_run += pr[st][i];
      }
    const u32x4_t pf = {pack_bf16x2(pr[0][0], pr[0][1]), pack_bf16x2(pr[0][2], pr[0][3]),
                        pack_bf16x2(pr[1][0], pr[1][1]), pack_bf16x2(pr[1][2], pr[1][3])};

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const unsigned char* src = vs + 2 * (16 * dt + col);
      uint32_t wv[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t lo = *reinterpret_cast<const uint16_t*>(src + kkey(lg, 2 * h) * RS);
        const uint32_t hi = *reinterpret_cast<const uint16_t*>(src + kkey(lg, 2 * h + 1) * RS);
        wv[h] = lo | (hi << 16);
      }
      o[dt] = mfma_bf16(u32x4_t{wv[0], wv[1], wv[2], wv[3]}, pf, o[dt]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // One unit in flight per wave: a second register set would halve the
  // waves per SIMD, and more waves hide latency at least as well.
  for (int idx = w; idx < n_units; idx += 4) {
    Unit u;
    fetch(idx, u);
    consume(u);
  }

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

  for (int idx = tid; idx < G * D; idx += 256) {
    const int h = idx / D, e = idx % D;
    float M = -__builtin_inff();
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, cm[ww * 16 + h]);
    float L = 0.f, O = 0.f;
    if (M != -__builtin_inff()) {
      for (int ww = 0; ww < 4; ++ww) {
        const float f = __builtin_amdgcn_exp2f(cm[ww * 16 + h] - M);
        L += f * cl[ww * 16 + h];
        O += f * co[(ww * 16 + h) * D + e];
      }
    }
    if (n_split == 1) {
      out[(b * hq + (int64_t)g * G + h) * D + e] = f32_to_bf16(O / L);
    } else {
      float* pp = part + (row * n_split + split) * (int64_t)(2 * G + G * D);
      if (e == 0) {
        pp[h] = M;
        pp[G + h] = L;
      }
      pp[2 * G + h * D + e] = O;
    }
  }
}

// Merge the slices' partial softmax states of one (row, query head), one
// output dim per thread, slices in order.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const float* __restrict__ part, uint16_t* __restrict__ out,
                                                           int hq, int hkv, int G, int n_split) {
  const int64_t row = blockIdx.x / G;
  const int h = blockIdx.x % G;
  const int e = threadIdx.x;
  const int64_t b = row / hkv;
  const int g = (int)(row % hkv);
  const int64_t stride = 2 * G + G * D;
  const float* pr = part + row * n_split * stride;
  // Slices in batches of 32 whose loads all go out at once (one memory round
  // trip per batch), folded in slice order into a running state.
  constexpr int kBatch = 32;
  float M = -__builtin_inff(), L = 0.f, O = 0.f;
  for (int s0 = 0; s0 < n_split; s0 += kBatch) {
    float ms[kBatch], ls[kBatch], os[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const bool ok = s0 + j < n_split;
      const float* ps = pr + (int64_t)(s0 + j) * stride;
      ms[j] = ok ? ps[h] : -__builtin_inff();
      ls[j] = ok ? ps[G + h] : 0.f;
      os[j] = ok ? ps[2 * G + h * D + e] : 0.f;
    }
    float mb = M;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) mb = fmaxf(mb, ms[j]);
    if (mb == -__builtin_inff()) continue;  // no visible key so far
    const float a = __builtin_amdgcn_exp2f(M - mb);  // 0 while M = -inf
    L *= a;
    O *= a;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float f = __builtin_amdgcn_exp2f(ms[j] - mb);  // 0 for empty slices
      L += f * ls[j];
      O += f * os[j];
    }
    M = mb;
  }
  out[(b * hq + (int64_t)g * G + h) * D + e] = f32_to_bf16(O / L);
}

template <int D>
hipError_t launch_d(const Dims& s, const DecodePlan& plan, const void* q, const void* k, const void* v,
                    int64_t kv_len, int64_t kv_cap, const int32_t* sel, void* out, void* ws, hipStream_t st) {
  const int64_t rows = (int64_t)s.batch * s.hkv;
  const float scale_log2 = s.scale * 1.4426950408889634f;
  auto kern = s.bs < kUnit ? decode_attn_kernel<D, true> : decode_attn_kernel<D, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)(rows * plan.n_split)), dim3(256), 0, st, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), sel,
                     static_cast<uint16_t*>(out), static_cast<float*>(ws), kv_len, kv_cap, s.hq, s.hkv, s.group,
                     s.bs, s.top_k, scale_log2, plan.blocks_per_wg, plan.n_split);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.n_split == 1) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)(rows * s.group)), dim3(D), 0, st,
                     static_cast<const float*>(ws), static_cast<uint16_t*>(out), s.hq, s.hkv, s.group, plan.n_split);
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
  p.ws_bytes = p.n_split > 1 ? (size_t)rows * p.n_split * (2 * s.group + s.group * s.d) * sizeof(float) : 0;
  return p;
}

hipError_t launch_decode(const Dims& s, const DecodePlan& plan, const void* q, const void* k, const void* v,
                         int64_t kv_len, int64_t kv_cap, const int32_t* sel, void* out, void* ws, hipStream_t st) {
  return s.d == 64 ? launch_d<64>(s, plan, q, k, v, kv_len, kv_cap, sel, out, ws, st)
                   : launch_d<128>(s, plan, q, k, v, kv_len, kv_cap, sel, out, ws, st);
}

}  // namespace qsa
