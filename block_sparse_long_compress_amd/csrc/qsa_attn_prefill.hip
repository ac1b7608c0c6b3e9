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
// columns are masked (their MFMA work is wasted: the cost of per-token
// selection with GQA). The keys form the 16-row M side: S^T = K Q^T, then
// O^T += V^T P^T, with P^T taken from the S^T accumulators without any lane
// exchange (see kkey()).
//
// A workgroup of 4 waves owns NCG CGs per wave (a 64-token tile for G = 8)
// of one (sequence, KV head) and walks the union of their selections in
// ascending block order. Each block's K and V^T operand fragments are copied
// into a ring of NS LDS stages by direct global->LDS loads
// (global_load_lds_dwordx4: no VGPR staging), NS-1 blocks ahead of the one
// being computed; a stage is released with a plain s_barrier after an
// explicit vmcnt wait, so the copies of later stages stay in flight. Every
// fragment is one 16-byte LDS read per lane, shared by all CGs of the wave
// that selected the block. Accumulators (NCG x d/16 x 4 floats per lane) sit
// in AGPRs. Each token keeps a cursor into its ascending selection list, so
// membership is one LDS compare per block.
//
// V^T fragments come from vt_pack_kernel, which writes V in exactly the lane
// order the PV product consumes. K fragments are read straight from the
// cache in operand order by the DMA lane addresses.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kUnit = 32;
constexpr float kRescaleSlack = 8.0f;  // log2 headroom before the softmax offset is raised

__device__ __forceinline__ int kkey(int lg, int j) { return j < 4 ? 4 * lg + j : 12 + 4 * lg + j; }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that does not drain the DMA queue (the release fence of
// __syncthreads would wait for every outstanding global load); the asm
// statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

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

template <int D, int BS, int W>
struct Stage {
  static constexpr int kKFrags = (BS / 16) * (D / 32);  // 1 KiB each: 16 keys x 32 dims
  static constexpr int kVFrags = (BS / 32) * (D / 16);  // 1 KiB each: 16 dims x 32 keys
  static constexpr int kFrags = kKFrags + kVFrags;
  static constexpr int kPerWave = kFrags / W;           // DMA instructions per wave per block
  static constexpr int kBytes = kFrags * 1024;
  static constexpr int kMaxStages = (4 * kBytes <= 128 * 1024) ? 4 : ((3 * kBytes <= 128 * 1024) ? 3 : 2);
  static_assert(kFrags % W == 0, "fragments per block");
};

// LDS layout after the ring of `stages` x Stage::kBytes:
//   mask[n_words] (u32)  wprefix[n_words] (u32)  tokmask[u_cap] (u64)  ulist[u_cap] (i32)
struct PrefillLds {
  int mask, wprefix, tokmask, ulist, total;
};
__host__ __device__ inline PrefillLds prefill_lds(int stage_bytes, int stages, int n_words, int u_cap) {
  PrefillLds L;
  L.mask = stage_bytes * stages;
  L.wprefix = L.mask + n_words * 4;
  L.tokmask = (L.wprefix + n_words * 4 + 7) / 8 * 8;
  L.ulist = L.tokmask + u_cap * 8;
  L.total = L.ulist + u_cap * 4;
  return L;
}

template <int D, int BS, int W, int NCG>
__global__ __launch_bounds__(W * 64, 1) void prefill_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ vt,
    const int32_t* __restrict__ sel, uint16_t* __restrict__ out, int64_t q_len, int64_t q_pos0, int64_t kv_cap,
    int64_t n_units, int hq, int hkv, int G, int top_k, float scale_log2, int n_tiles, int xcd_groups, int stages,
    int n_words_max, int u_cap) {
  using ST = Stage<D, BS, W>;
  constexpr int NT = W * 64;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int UPB = BS / kUnit;
  // keys per softmax step: 64 when registers allow, else 32 (the K operands of a step stay in VGPRs)
  constexpr int CH = (W == 8) ? ((BS == 64 && D * NCG <= 256) ? 64 : 32) : ((D * NCG >= 512 || BS < 64) ? 32 : 64);
  constexpr int NCH = BS / CH;
  constexpr int SUB = CH / 16;           // 16-key S^T tiles per step
  constexpr int UPC = CH / kUnit;        // 32-key PV steps per softmax step
  extern __shared__ __align__(16) unsigned char smem[];

  // Work item: (sequence, KV head, tile). Workgroups go to the 8 XCDs
  // round-robin; when the (sequence, KV head) pairs split evenly over the
  // XCDs, each XCD serves one pair so that its L2 keeps that pair's K and V.
  int bg, tile;
  if (xcd_groups > 0) {
    const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const int per = 8 / xcd_groups;  // XCDs per pair
    bg = xcd / per;
    tile = slot * per + xcd % per;
  } else {
    bg = blockIdx.x / n_tiles;
    tile = blockIdx.x % n_tiles;
  }
  tile = n_tiles - 1 - tile;  // latest tokens (most blocks) first
  const int64_t b = bg / hkv;
  const int g = bg % hkv;
  const int tpc = 16 / G;
  const int qt = W * NCG * tpc;
  const int64_t t0 = (int64_t)tile * qt;
  const int tid = threadIdx.x, lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lg = lane / 16, col = lane % 16;
  const int rows = (int)(q_len - t0 < qt ? q_len - t0 : qt);
  const int64_t kv_total = q_pos0 + q_len;
  const int64_t pos_first = q_pos0 + t0;
  const int64_t own_last = (pos_first + rows - 1) / BS;
  const int n_words = (int)(own_last / 32) + 1;
  const PrefillLds L = prefill_lds(ST::kBytes, stages, n_words_max, u_cap);
  uint32_t* mask = reinterpret_cast<uint32_t*>(smem + L.mask);
  uint32_t* wprefix = reinterpret_cast<uint32_t*>(smem + L.wprefix);
  unsigned long long* tokmask = reinterpret_cast<unsigned long long*>(smem + L.tokmask);
  int32_t* ulist = reinterpret_cast<int32_t*>(smem + L.ulist);

  // ---- union of the tile's selections, ascending, with the token set of each block
  for (int i = tid; i < n_words; i += NT) mask[i] = 0u;
  for (int i = tid; i < u_cap; i += NT) tokmask[i] = 0ull;
  __syncthreads();
  const int32_t* sel_tile = sel + ((b * q_len + t0) * hkv + g) * top_k;
  for (int i = tid; i < rows * top_k; i += NT) {
    const int r = i / top_k, e = i % top_k;
    const int32_t c = sel_tile[(int64_t)r * hkv * top_k + e];
    if (c >= 0 && (int64_t)c <= (pos_first + r) / BS) atomicOr(&mask[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
  if (w == 0) {  // exclusive prefix of the per-word popcounts
    uint32_t carry = 0;
    for (int base = 0; base < n_words; base += kWave) {
      const uint32_t cnt = base + lane < n_words ? (uint32_t)__builtin_popcount(mask[base + lane]) : 0u;
      uint32_t incl = cnt;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)incl, d, kWave);
        incl += lane >= d ? y : 0u;
      }
      if (base + lane < n_words) wprefix[base + lane] = carry + incl - cnt;
      carry += (uint32_t)__shfl((int)incl, kWave - 1, kWave);
    }
  }
  __syncthreads();
  const int n_union = (int)(wprefix[n_words - 1] + (uint32_t)__builtin_popcount(mask[n_words - 1]));
  for (int i = tid; i < rows * top_k; i += NT) {
    const int r = i / top_k, e = i % top_k;
    const int32_t c = sel_tile[(int64_t)r * hkv * top_k + e];
    if (c >= 0 && (int64_t)c <= (pos_first + r) / BS) {
      const int idx = (int)(wprefix[c >> 5] + (uint32_t)__builtin_popcount(mask[c >> 5] & ((1u << (c & 31)) - 1u)));
      ulist[idx] = c;
      atomicOr(&tokmask[idx], 1ull << r);
    }
  }
  __syncthreads();

  // ---- per-wave DMA plan: fragment f = w + W*j of each block
  const uint16_t* kg = k + ((b * hkv + g) * kv_cap) * D;
  const uint16_t* vtg = vt + ((b * hkv + g) * n_units) * DT * kWave * 8;
  int src_off[ST::kPerWave];  // elements from the block's base (K rows or V^T units)
#pragma unroll
  for (int j = 0; j < ST::kPerWave; ++j) {
    const int f = w + W * j;
    if (f < ST::kKFrags) {
      const int su = f / KS, s = f % KS;
      src_off[j] = (16 * su + col) * D + 32 * s + 8 * lg;
    } else {
      src_off[j] = ((f - ST::kKFrags) * kWave + lane) * 8;
    }
  }
  auto issue = [&](int ui, int slot) {
    const int64_t c = ulist[ui];
    unsigned char* dst = smem + slot * ST::kBytes;
    const uint16_t* kbase = kg + c * BS * D;
    const uint16_t* vbase = vtg + c * (UPB * DT * kWave * 8);
    const bool tail = (c + 1) * BS > kv_total;  // block runs past the prefix: clamp K rows
#pragma unroll
    for (int j = 0; j < ST::kPerWave; ++j) {
      const int f = w + W * j;
      const uint16_t* src;
      if (f < ST::kKFrags) {
        src = kbase + src_off[j];
        if (tail) {
          const int su = f / KS, s = f % KS;
          int64_t key = c * BS + 16 * su + col;
          key = key < kv_total ? key : kv_total - 1;  // any finite row: masked out below
          src = kg + key * D + 32 * s + 8 * lg;
        }
      } else {
        src = vbase + src_off[j];
      }
      __builtin_amdgcn_global_load_lds(src, dst + f * 1024, 16, 0, 0);
    }
  };

  // ---- per CG: this lane's column token, its position, softmax state, Q operands
  u32x4_t qf[NCG][KS];
  f32x4_t o[NCG][DT];
  float m_run[NCG], l_run[NCG];
  int pos_q[NCG];  // absolute positions fit in int32 (checked on the host)
  bool row_ok[NCG];
  const int tau = col / G;
#pragma unroll
  for (int n = 0; n < NCG; ++n) {
    const int r = (w * NCG + n) * tpc + tau;
    row_ok[n] = r < rows;
    pos_q[n] = (int)(pos_first + r);
    m_run[n] = -__builtin_inff();
    l_run[n] = 0.f;
    const uint16_t* qs = q + ((b * q_len + t0 + r) * hq + (int64_t)g * G + col % G) * D + 8 * lg;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[n][s] = row_ok[n] ? *reinterpret_cast<const u32x4_t*>(qs + 32 * s) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[n][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  wait_vmcnt<0>();  // Q is in registers before the DMA queue starts counting

  const int wave_shift = w * NCG * tpc;
  const unsigned long long cg_mask = (1ull << tpc) - 1ull;

  // Consume the union in groups of `per_it` blocks per barrier (2 when four
  // stages fit: the next group's copies run during the current group's math),
  // which also averages the per-wave work of the group before the barrier.
  const int per_it = stages >= 4 ? 2 : 1;
  const int ring = per_it == 2 ? 4 : stages;
  if (per_it == 2) {
    for (int ui = 0; ui < 2 && ui < n_union; ++ui) issue(ui, ui);
  } else {
    for (int ui = 0; ui < stages - 1 && ui < n_union; ++ui) issue(ui, ui);
  }

  for (int u0 = 0; u0 < n_union; u0 += per_it) {
    if (per_it == 2) {
      wait_vmcnt<0>();
      stage_barrier();  // every wave is past the previous group: its stages may be refilled
      for (int a = 2; a < 4; ++a)
        if (u0 + a < n_union) issue(u0 + a, (u0 + a) % ring);
    } else {
      int ahead = n_union - 1 - u0;
      ahead = ahead < stages - 2 ? ahead : stages - 2;
      if (ahead >= 2) wait_vmcnt<2 * ST::kPerWave>();
      else if (ahead == 1) wait_vmcnt<ST::kPerWave>();
      else wait_vmcnt<0>();
      stage_barrier();
      if (u0 + stages - 1 < n_union) issue(u0 + stages - 1, (u0 + stages - 1) % stages);
    }
    for (int ui = u0; ui < u0 + per_it && ui < n_union; ++ui) {
    const int slot = ui % ring;
    const int64_t c = ulist[ui];
    const unsigned long long tm = tokmask[ui] >> wave_shift;
    unsigned need = 0u;
    bool mem[NCG];
#pragma unroll
    for (int n = 0; n < NCG; ++n) {
      const unsigned long long bits = (tm >> (n * tpc)) & cg_mask;
      need |= bits != 0ull ? (1u << n) : 0u;
      mem[n] = row_ok[n] && ((bits >> tau) & 1ull);
    }
    if (need == 0u) continue;
    const bool diag = (c + 1) * BS > pos_first;  // own block of some token of the tile: causal mask
    const int key_base = (int)(c * BS);          // positions fit in int32 (checked on the host)
    const unsigned char* kb = smem + slot * ST::kBytes;
    const unsigned char* vb = kb + ST::kKFrags * 1024;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const int key0 = key_base + ch * CH;
      u32x4_t kf[SUB][KS];
#pragma unroll
      for (int su = 0; su < SUB; ++su)
#pragma unroll
        for (int s = 0; s < KS; ++s)
          kf[su][s] = *reinterpret_cast<const u32x4_t*>(kb + (((ch * SUB + su) * KS + s) * kWave + lane) * 16);
      u32x4_t pf[NCG][UPC];
#pragma unroll
      for (int n = 0; n < NCG; ++n) {
        if (!((need >> n) & 1u)) continue;
        float x[SUB * 4];
#pragma unroll
        for (int su = 0; su < SUB; ++su) {
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s) acc = mfma_bf16(kf[su][s], qf[n][s], acc);
#pragma unroll
          for (int i = 0; i < 4; ++i) x[su * 4 + i] = acc[i];
        }
        if (diag) {
#pragma unroll
          for (int su = 0; su < SUB; ++su)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int pos = key0 + 16 * su + 4 * lg + i;
              x[su * 4 + i] = pos <= pos_q[n] ? x[su * 4 + i] : -__builtin_inff();
            }
        }
        float mx = x[0];
#pragma unroll
        for (int i = 1; i + 1 < SUB * 4; i += 2) mx = __builtin_fmaxf(mx, __builtin_fmaxf(x[i], x[i + 1]));
        if constexpr ((SUB * 4) % 2 == 0) mx = __builtin_fmaxf(mx, x[SUB * 4 - 1]);
        mx = max_col4(mx);
        // The exponent offset m_run is raised only when a score exceeds it by
        // more than 2^8: p stays <= 256 (exact in fp32, representable in
        // bf16) and the accumulators are rescaled rarely.
        const float m_old = m_run[n];
        const float cand = mx * scale_log2;
        const bool grow = mem[n] && cand > m_old + kRescaleSlack;
        const float m_new = grow ? cand : m_old;
        if (__ballot(grow && m_old != -__builtin_inff()) != 0) {
          const float alpha = grow ? __builtin_amdgcn_exp2f(m_old - m_new) : 1.0f;
          l_run[n] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[n][dt] *= alpha;
        }
        m_run[n] = m_new;
        const float negm = (mem[n] && m_new != -__builtin_inff()) ? -m_new : -__builtin_inff();
        float pv[SUB * 4];
#pragma unroll
        for (int i = 0; i < SUB * 4; ++i) {
          pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], scale_log2, negm));
          l_run[n] += pv[i];
        }
        // P^T operand of 32-key step u: tiles 2u, 2u+1 (see kkey())
#pragma unroll
        for (int u = 0; u < UPC; ++u) {
          const float* a = pv + 8 * u;
          pf[n][u] = u32x4_t{cvt_pk_bf16(a[0], a[1]), cvt_pk_bf16(a[2], a[3]), cvt_pk_bf16(a[4], a[5]),
                             cvt_pk_bf16(a[6], a[7])};
        }
      }
#pragma unroll
      for (int u = 0; u < UPC; ++u)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const u32x4_t vf = *reinterpret_cast<const u32x4_t*>(vb + (((ch * UPC + u) * DT + dt) * kWave + lane) * 16);
#pragma unroll
          for (int n = 0; n < NCG; ++n) {
            if (!((need >> n) & 1u)) continue;
            o[n][dt] = mfma_bf16(vf, pf[n][u], o[n][dt]);
          }
        }
    }
    }
  }

#pragma unroll
  for (int n = 0; n < NCG; ++n) {
    const float l = sum_col4(l_run[n]);
    if (!row_ok[n]) continue;
    const float inv = 1.0f / l;
    const int r = (w * NCG + n) * tpc + tau;
    uint16_t* dst = out + ((b * q_len + t0 + r) * hq + (int64_t)g * G + col % G) * D + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const u32x2_t pk = {cvt_pk_bf16(o[n][dt][0] * inv, o[n][dt][1] * inv),
                          cvt_pk_bf16(o[n][dt][2] * inv, o[n][dt][3] * inv)};
      *reinterpret_cast<u32x2_t*>(dst + 16 * dt) = pk;
    }
  }
}

// CGs per wave: tiles of at most 64 tokens, and for d = 128 at most 4 CGs
// (4 x 32 accumulator AGPRs plus the Q and K operands fill the register file).
inline int ncg_for(int G, int D) {
  const int cap = D == 128 ? 4 : 8;
  return G >= cap ? cap : G;
}
// Waves per workgroup: 8 (two per SIMD, 2 CGs each) where the CG count allows.
inline int waves_for(int G, int D) { return ncg_for(G, D) >= 4 ? 8 : 4; }
inline int ncg_per_wave(int G, int D) { return waves_for(G, D) == 8 ? ncg_for(G, D) / 2 : ncg_for(G, D); }

struct PrefillGeom {
  int qt, n_tiles, n_words, u_cap, stages, lds;
};

template <int D, int BS>
PrefillGeom prefill_geom(const Dims& s, int64_t q_len, int64_t q_pos0) {
  using ST = Stage<D, BS, 4>;  // stage bytes do not depend on the wave count
  PrefillGeom gm;
  const int64_t kv_total = q_pos0 + q_len;
  gm.qt = waves_for(s.group, D) * ncg_per_wave(s.group, D) * (16 / s.group);
  gm.n_tiles = (int)((q_len + gm.qt - 1) / gm.qt);
  gm.n_words = (int)(((kv_total - 1) / BS) / 32) + 1;
  const int64_t n_blocks = (kv_total + BS - 1) / BS;
  const int64_t cap = (int64_t)gm.qt * s.top_k;
  gm.u_cap = (int)(cap < n_blocks ? cap : n_blocks);
  gm.stages = ST::kMaxStages;
  gm.lds = prefill_lds(ST::kBytes, gm.stages, gm.n_words, gm.u_cap).total;
  while (gm.stages > 2 && gm.lds > 160 * 1024) {
    --gm.stages;
    gm.lds = prefill_lds(ST::kBytes, gm.stages, gm.n_words, gm.u_cap).total;
  }
  return gm;
}

template <int D, int BS, int W, int NCG>
hipError_t launch_kernel(const Dims& s, const PrefillGeom& gm, int64_t q_len, int64_t q_pos0, int64_t kv_cap,
                         int64_t n_units, const void* q, const void* k, const uint16_t* vt, const int32_t* sel,
                         void* out, hipStream_t st) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&prefill_attn_kernel<D, BS, W, NCG>), hipFuncAttributeMaxDynamicSharedMemorySize,
      160 * 1024);
  if (attr != hipSuccess) return attr;
  const int n_bg = s.batch * s.hkv;
  // one (sequence, KV head) pair per group of XCDs when pairs and tiles split evenly over the 8 XCDs
  int xcd_groups = 0;
  if (n_bg <= 8 && 8 % n_bg == 0 && gm.n_tiles % (8 / n_bg) == 0) xcd_groups = n_bg;
  const float scale_log2 = s.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((prefill_attn_kernel<D, BS, W, NCG>), dim3((unsigned)(gm.n_tiles * n_bg)), dim3(W * 64), gm.lds, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), vt, sel,
                     static_cast<uint16_t*>(out), q_len, q_pos0, kv_cap, n_units, s.hq, s.hkv, s.group, s.top_k,
                     scale_log2, gm.n_tiles, xcd_groups, gm.stages, gm.n_words, gm.u_cap);
  return hipGetLastError();
}

template <int D, int BS>
hipError_t launch_bs(const Dims& s, int64_t q_len, int64_t q_pos0, int64_t kv_cap, int64_t n_units, const void* q,
                     const void* k, const uint16_t* vt, const int32_t* sel, void* out, hipStream_t st) {
  const PrefillGeom gm = prefill_geom<D, BS>(s, q_len, q_pos0);
  switch (ncg_for(s.group, D)) {
    case 1:
      return launch_kernel<D, BS, 4, 1>(s, gm, q_len, q_pos0, kv_cap, n_units, q, k, vt, sel, out, st);
    case 2:
      return launch_kernel<D, BS, 4, 2>(s, gm, q_len, q_pos0, kv_cap, n_units, q, k, vt, sel, out, st);
    case 4:
      return launch_kernel<D, BS, 8, 2>(s, gm, q_len, q_pos0, kv_cap, n_units, q, k, vt, sel, out, st);
    default:  // 8 CGs (d = 64 only)
      if constexpr (D == 64) return launch_kernel<D, BS, 8, 4>(s, gm, q_len, q_pos0, kv_cap, n_units, q, k, vt, sel, out, st);
      else return launch_kernel<D, BS, 8, 2>(s, gm, q_len, q_pos0, kv_cap, n_units, q, k, vt, sel, out, st);
  }
}

template <int D>
hipError_t launch_d(const Dims& s, const PrefillPlan& plan, const void* q, const void* k, const void* v,
                    int64_t q_len, int64_t q_pos0, int64_t kv_cap, const int32_t* sel, void* out, void* ws,
                    hipStream_t st) {
  (void)plan;
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
  switch (s.bs) {
    case 32:
      return launch_bs<D, 32>(s, q_len, q_pos0, kv_cap, n_units, q, k, vt, sel, out, st);
    case 64:
      return launch_bs<D, 64>(s, q_len, q_pos0, kv_cap, n_units, q, k, vt, sel, out, st);
    default:
      return launch_bs<D, 128>(s, q_len, q_pos0, kv_cap, n_units, q, k, vt, sel, out, st);
  }
}

}  // namespace

PrefillPlan plan_prefill(const Dims& s, int64_t q_len, int64_t q_pos0) {
  PrefillPlan p{};
  p.rows_per_wg = waves_for(s.group, s.d) * ncg_per_wave(s.group, s.d) * (16 / s.group);
  if (s.dtype != 1) {
    p.ws_bytes = 0;
    return p;
  }
  const int64_t kv_total = q_pos0 + q_len;
  const int64_t n_blocks = (kv_total + s.bs - 1) / s.bs;
  p.ws_bytes = (size_t)s.batch * s.hkv * n_blocks * s.bs * s.d * sizeof(uint16_t);
  return p;
}

// LDS footprint of the prefill kernel for these sizes.
int prefill_smem_bytes(const Dims& s, int64_t q_len, int64_t q_pos0) {
  if (s.d == 64) {
    return s.bs == 32 ? prefill_geom<64, 32>(s, q_len, q_pos0).lds
                      : (s.bs == 64 ? prefill_geom<64, 64>(s, q_len, q_pos0).lds : prefill_geom<64, 128>(s, q_len, q_pos0).lds);
  }
  return s.bs == 32 ? prefill_geom<128, 32>(s, q_len, q_pos0).lds
                    : (s.bs == 64 ? prefill_geom<128, 64>(s, q_len, q_pos0).lds : prefill_geom<128, 128>(s, q_len, q_pos0).lds);
}

hipError_t launch_prefill(const Dims& s, const PrefillPlan& plan, const void* q, const void* k, const void* v,
                          int64_t q_len, int64_t q_pos0, int64_t kv_cap, const int32_t* sel, void* out, void* ws,
                          hipStream_t st) {
  return s.d == 64 ? launch_d<64>(s, plan, q, k, v, q_len, q_pos0, kv_cap, sel, out, ws, st)
                   : launch_d<128>(s, plan, q, k, v, q_len, q_pos0, kv_cap, sel, out, ws, st);
}

}  // namespace qsa
