// One wave's share of sparse decode attention over a slice of the selection
// list (shared by the decode kernel and the fused decode step).
//
// bf16 inputs, bf16 MFMA (v_mfma_f32_16x16x32_bf16), float32 softmax and
// accumulation. Work unit = 32 keys: 32 consecutive keys of one selected
// block, or for blocks shorter than 32 keys (Bs = 4, 8, 16) the keys of
// 32/Bs consecutive entries of the selection list, each row addressed on its
// own (the position of every key row is computed once per unit and shared
// across lanes with ds_bpermute). Per unit the wave computes S^T = K Q^T with
// the keys as the 16-row M operand and the G query heads of the KV head as
// the N columns (G <= 16; columns >= G are zero queries and are ignored),
// keeps an online softmax per column in the exp2 domain, and accumulates
// O^T = V^T P^T. K fragments are loaded straight from HBM in operand layout
// (16 contiguous bytes per lane). V rows are staged in the wave's own LDS
// slice with coalesced loads and read back transposed, two bytes at a time,
// into the V^T operand.
#pragma once

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

constexpr int kUnit = 32;

// Element j of a lane's 8-wide K-dimension operand slot, for lane group lg,
// is key kkey(lg, j) of the 32-key unit. S^T tiles 0 and 1 hold keys
// 4*lg+i and 16+4*lg+i in lane group lg (MFMA output layout), so P^T can be
// fed to the PV product without any lane exchange.
__device__ __forceinline__ int kkey(int lg, int j) { return j < 4 ? 4 * lg + j : 12 + 4 * lg + j; }

template <int D>
constexpr int kStageRowBytes = 2 * D + 16;  // LDS row stride of staged V (bytes)
// Row stride (floats) of the waves' unnormalised outputs when a workgroup
// combines them in LDS: one 16-byte slot past D, so that the 16 lanes of a
// lane group, which write 16 rows at one column, spread over the banks.
template <int D>
constexpr int kCombStride = D + 4;

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// 8 codes (two little-endian words) times one scale, as 4 packed bf16 pairs.
// The codes are biased to unsigned bytes (xor 0x80), widened one byte per
// instruction, and (c + 128 - 128) * scale is one fused multiply-add.
__device__ __forceinline__ u32x4_t dequant8_bf16(u32x2_t codes, float scale) {
  const float off = -128.0f * scale;
  uint32_t r[4];
#pragma unroll
  for (int wi = 0; wi < 2; ++wi) {
    const uint32_t w = codes[wi] ^ 0x80808080u;
    const float c0 = (float)(w & 0xFFu), c1 = (float)((w >> 8) & 0xFFu);  // one byte-to-float instruction each
    const float c2 = (float)((w >> 16) & 0xFFu), c3 = (float)(w >> 24);
    r[2 * wi] = pack_bf16x2(__builtin_fmaf(c0, scale, off), __builtin_fmaf(c1, scale, off));
    r[2 * wi + 1] = pack_bf16x2(__builtin_fmaf(c2, scale, off), __builtin_fmaf(c3, scale, off));
  }
  return u32x4_t{r[0], r[1], r[2], r[3]};
}

// Q operands of the row's G query heads (head j in column j; columns >= G zero).
template <int D>
__device__ __forceinline__ void load_q_operands(const uint16_t* __restrict__ q_heads, int G, u32x4_t (&qf)[D / 32]) {
  const int lane = lane_id(), lg = lane / 16, col = lane % 16;
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    qf[s] = u32x4_t{0u, 0u, 0u, 0u};
    if (col < G) qf[s] = *reinterpret_cast<const u32x4_t*>(q_heads + (int64_t)col * D + 32 * s + 8 * lg);
  }
}

// In-place unnormalised Walsh-Hadamard transform of a D-vector held by one
// wave, lane l holding elements l and l + 64 (D = 128) or l (D = 64).
template <int D>
__device__ __forceinline__ void fwht_wave(float (&v)[D / kWave]) {
  const int lane = lane_id();
#pragma unroll
  for (int h = 1; h < kWave && h < D; h <<= 1) {
#pragma unroll
    for (int i = 0; i < D / kWave; ++i) {
      const float other = shfl_xor_f32(v[i], h);
      v[i] = (lane & h) ? other - v[i] : v[i] + other;
    }
  }
  if constexpr (D == 2 * kWave) {
    const float a = v[0], b = v[1];
    v[0] = a + b;
    v[1] = a - b;
  }
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }

// One row of the rotated 8-bit cache, by one wave: the Walsh-Hadamard
// rotation of the bf16 row src, then for each 32 values a float16 scale (the
// largest magnitude / 127, rounded to float16) and codes
// round-half-even(value / scale) clamped to [-127, 127] (0 when the scale is
// 0), written to dq (D codes) and ds (D / 32 scales).
template <int D>
__device__ __forceinline__ void quantize_row_wave(const uint16_t* __restrict__ src, int8_t* __restrict__ dq,
                                                  uint16_t* __restrict__ ds) {
  constexpr int EPL = D / kWave;
  const int lane = lane_id();
  float x[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) x[i] = bf16_to_f32(src[lane + kWave * i]);
  fwht_wave<D>(x);
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    // the 32 lanes of element lane + 64 i that share a group
    float amax = fabsf(x[i]);
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) amax = fmaxf(amax, shfl_xor_f32(amax, m));
    const uint16_t sbits = f32_to_f16_bits(amax / 127.0f);
    const float scale = f16_bits_to_f32(sbits);
    float c = scale > 0.f ? __builtin_rintf(x[i] / scale) : 0.f;
    c = fminf(fmaxf(c, -127.f), 127.f);
    dq[lane + kWave * i] = (int8_t)(int)c;
    if ((lane & 31) == 0) ds[(lane + kWave * i) / 32] = sbits;
  }
}

// Q operands in the 8-bit cache's dim order: step s = 2t + h takes, in lane
// group lg, dims 64 t + 16 lg + 8 h .. +7 (a lane's 16-byte code load covers
// both steps of a pair). Any order of the dims gives the same dot products.
template <int D>
__device__ __forceinline__ void load_q8_query_operands(const uint16_t* __restrict__ q_heads, int G,
                                                       u32x4_t (&qf)[D / 32]) {
  const int lane = lane_id(), lg = lane / 16, col = lane % 16;
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    qf[s] = u32x4_t{0u, 0u, 0u, 0u};
    if (col < G)
      qf[s] = *reinterpret_cast<const u32x4_t*>(q_heads + (int64_t)col * D + 64 * (s / 2) + 16 * lg + 8 * (s % 2));
  }
}

// Units idx = first, first + stride, ... of a slice of n_e selection entries
// (entry j of the slice in lane j's sel_mine, -1 for padding), attended by
// one wave into (m_run, l_run, o). kbase, vbase point at position 0 of the
// row's keys and values; p is the query position; vs is the wave's 32-row
// staging slice. One unit in flight per wave: a second register set would
// halve the waves per SIMD, and more waves hide latency at least as well.
template <int D, bool GATHER, bool Q8 = false>
__device__ __forceinline__ void attend_units(const u32x4_t (&qf)[D / 32], const uint16_t* __restrict__ kbase,
                                             const uint16_t* __restrict__ vbase, int sel_mine, int n_e, int bs,
                                             int64_t p, float scale_log2, unsigned char* vs, int first, int stride,
                                             float& m_run, float& l_run, f32x4_t (&o)[D / 16],
                                             Q8Cache q8 = Q8Cache{nullptr, nullptr, nullptr, nullptr}) {
  constexpr int RS = kStageRowBytes<D>;
  constexpr int KS = D / 32;  // 32-wide K steps of the QK^T product
  constexpr int DT = D / 16;  // 16-wide dim tiles of the PV product
  const int lane = lane_id();
  const int lg = lane / 16, col = lane % 16;
  const int upb = GATHER ? 1 : bs / kUnit;  // units per block
  const int bpu = GATHER ? kUnit / bs : 1;  // blocks per unit
  const int n_units = GATHER ? (n_e + bpu - 1) / bpu : n_e * upb;
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
      if constexpr (Q8) {
        // the 8-bit cache, rows gathered: a lane's K codes are those of the
        // contiguous case (its row 16 st + col, bytes 64 t + 16 lg, scale
        // group 2 t + lg/2) at the row's own position, with that row's scale
        // read directly; V codes and scales likewise per staged row, widened
        // straight into the wave's staging slice. Rows past the causal bound
        // or of padding entries read as code 0 with scale 0, i.e. zero.
        static_assert(KS % 2 == 0, "two operand steps per 16-byte load");
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int kp = __builtin_amdgcn_ds_bpermute((16 * st + col) << 2, rowpos);
          u.mpos[st] = __builtin_amdgcn_ds_bpermute((16 * st + 4 * lg) << 2, rowpos);
          const int64_t kr = kp >= 0 ? kp : 0;
          u32x4_t kc[KS / 2];
          uint16_t ksc[KS / 2];
#pragma unroll
          for (int t = 0; t < KS / 2; ++t) {
            kc[t] = kp >= 0 ? *reinterpret_cast<const u32x4_t*>(q8.k + kr * D + 64 * t + 16 * lg)
                            : u32x4_t{0u, 0u, 0u, 0u};
            ksc[t] = kp >= 0 ? q8.ks[kr * (D / 32) + 2 * t + lg / 2] : (uint16_t)0;
          }
#pragma unroll
          for (int t = 0; t < KS / 2; ++t) {
            const float sc = f16_bits_to_f32(ksc[t]);
            u.kf[st][2 * t] = dequant8_bf16(u32x2_t{kc[t][0], kc[t][1]}, sc);
            u.kf[st][2 * t + 1] = dequant8_bf16(u32x2_t{kc[t][2], kc[t][3]}, sc);
          }
        }
        u32x2_t vc[VCH];
        uint16_t vsc[VCH];
        int vrow[VCH];
#pragma unroll
        for (int j = 0; j < VCH; ++j) {
          const int ci = lane + kWave * j;
          const int rr = ci / (D / 8), c8 = ci % (D / 8);
          const int vp = __builtin_amdgcn_ds_bpermute(rr << 2, rowpos);
          const int64_t vr = vp >= 0 ? vp : 0;
          vrow[j] = rr;
          vc[j] = vp >= 0 ? *reinterpret_cast<const u32x2_t*>(q8.v + vr * D + 8 * c8) : u32x2_t{0u, 0u};
          vsc[j] = vp >= 0 ? q8.vs[vr * (D / 32) + c8 / 4] : (uint16_t)0;
        }
        // (the previous unit's reads of the staging slice ended at its
        // closing wave barrier)
#pragma unroll
        for (int j = 0; j < VCH; ++j) {
          const int c8 = (lane + kWave * j) % (D / 8);
          *reinterpret_cast<u32x4_t*>(vs + vrow[j] * RS + 16 * c8) = dequant8_bf16(vc[j], f16_bits_to_f32(vsc[j]));
        }
        return;
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int kp = __builtin_amdgcn_ds_bpermute((16 * st + col) << 2, rowpos);
        u.mpos[st] = __builtin_amdgcn_ds_bpermute((16 * st + 4 * lg) << 2, rowpos);
        const uint16_t* kb = kbase + (int64_t)(kp >= 0 ? kp : 0) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s)
          u.kf[st][s] = kp >= 0 ? *reinterpret_cast<const u32x4_t*>(kb + 32 * s + 8 * lg) : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < VCH; ++j) {
        const int ci = lane + kWave * j;
        const int rr = ci / (D / 8), c8 = ci % (D / 8);
        const int vp = __builtin_amdgcn_ds_bpermute(rr << 2, rowpos);
        u.vr[j] = vp >= 0 ? *reinterpret_cast<const u32x4_t*>(vbase + (int64_t)(vp >= 0 ? vp : 0) * D + 8 * c8)
                          : u32x4_t{0u, 0u, 0u, 0u};
      }
    } else {
      const int c = __builtin_amdgcn_readlane(sel_mine, idx / upb);
      if (c < 0) return;
      u.key0 = (int64_t)c * bs + (int64_t)(idx % upb) * kUnit;
      if (u.key0 > p) return;
      u.ok = true;
      if constexpr (Q8) {
        // K from the codes, 16 per lane and load: the lane's row (16 st +
        // col) at bytes 64 t + 16 lg .. +15, which are the dims of operand
        // steps s = 2t (first 8) and 2t + 1 (last 8) in this cache's dim
        // order (load_q8_query_operands gives the query the same order), all
        // in scale group 2t + lg/2. The unit's 32 x D/32 key scales are
        // loaded once across the wave (lane l: bytes 4l .. 4l+3) and each
        // lane's scales fetched with bpermute.
        static_assert(KS % 2 == 0, "two operand steps per 16-byte load");
        u32x4_t kc16[2][KS / 2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int64_t key = u.key0 + 16 * st + col;
          const bool ok = key <= p;
#pragma unroll
          for (int t = 0; t < KS / 2; ++t)
            kc16[st][t] = ok ? *reinterpret_cast<const u32x4_t*>(q8.k + key * D + 64 * t + 16 * lg)
                             : u32x4_t{0u, 0u, 0u, 0u};
        }
        constexpr int KSW = kUnit * (D / 32) / 2;  // 32-bit words of the unit's key scales
        const uint32_t ksw_all = (lane < KSW && u.key0 + (2 * lane) / (D / 32) <= p)
                                     ? *reinterpret_cast<const uint32_t*>(q8.ks + u.key0 * (D / 32) + 2 * lane)
                                     : 0u;
        // V: the unit's 32 x D/32 scales loaded once across the wave (lane l:
        // row l * KS / 64, two scales), each lane's pair fetched with bpermute
        u32x2_t vc[VCH];
        constexpr int SPL = 2;  // scales per lane
        static_assert(kUnit * (D / 32) == SPL * kWave || kUnit * (D / 32) == kWave, "scale layout");
        const int sl_row = (lane * SPL) / (D / 32);
        const bool sl_ok = (kUnit * (D / 32) == SPL * kWave || lane < kUnit) && u.key0 + sl_row <= p;
        const uint32_t vsw =
            sl_ok ? (kUnit * (D / 32) == SPL * kWave ? *reinterpret_cast<const uint32_t*>(q8.vs + u.key0 * (D / 32) + SPL * lane)
                                                    : *reinterpret_cast<const uint32_t*>(q8.vs + (u.key0 + lane) * (D / 32)))
                  : 0u;
#pragma unroll
        for (int j = 0; j < VCH; ++j) {
          const int ci = lane + kWave * j;
          const int r = ci / (D / 8), c8 = ci % (D / 8);
          const int64_t key = u.key0 + r;
          vc[j] = key <= p ? *reinterpret_cast<const u32x2_t*>(q8.v + key * D + 8 * c8) : u32x2_t{0u, 0u};
        }
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int t = 0; t < KS / 2; ++t) {
            const int si = (16 * st + col) * (D / 32) + 2 * t + lg / 2;  // scale index within the unit
            const uint32_t w = (uint32_t)__builtin_amdgcn_ds_bpermute((si / 2) << 2, (int)ksw_all);
            const float sc = f16_bits_to_f32((uint16_t)(w >> (16 * (si % 2))));
            u.kf[st][2 * t] = dequant8_bf16(u32x2_t{kc16[st][t][0], kc16[st][t][1]}, sc);
            u.kf[st][2 * t + 1] = dequant8_bf16(u32x2_t{kc16[st][t][2], kc16[st][t][3]}, sc);
          }
        // widened V goes straight to the wave's staging slice (the previous
        // unit's reads of it ended at its closing wave barrier)
#pragma unroll
        for (int j = 0; j < VCH; ++j) {
          const int ci = lane + kWave * j;
          const int r = ci / (D / 8), c8 = ci % (D / 8);
          const int si = r * (D / 32) + c8 / 4;  // scale index within the unit
          const uint32_t wsrc = (uint32_t)__builtin_amdgcn_ds_bpermute((si / SPL) << 2, (int)vsw);
          const float sc = f16_bits_to_f32((uint16_t)(wsrc >> (16 * (si % SPL))));
          *reinterpret_cast<u32x4_t*>(vs + r * RS + 16 * c8) = dequant8_bf16(vc[j], sc);
        }
      } else {
      const uint16_t* kb = kbase + u.key0 * D;
      const uint16_t* vb = vbase + u.key0 * D;
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
    }
  };
  auto consume = [&](const Unit& u) {
    if (!u.ok) return;
    if constexpr (!Q8) {  // (the 8-bit fetch stages V itself)
#pragma unroll
      for (int j = 0; j < VCH; ++j) {
        const int ci = lane + kWave * j;
        const int r = ci / (D / 8), c8 = ci % (D / 8);
        *reinterpret_cast<u32x4_t*>(vs + r * RS + 16 * c8) = u.vr[j];
      }
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
  for (int idx = first; idx < n_units; idx += stride) {
    Unit u;
    fetch(idx, u);
    consume(u);
  }

}

// Merge of a row's slice states by its last workgroup: slices in batches of
// SB, each batch's loads all in flight (one memory round trip), folded in
// slice order into a running state per group of 4 output dims; GPT groups
// per thread (NT threads) cover the G * D / 4 groups of the row.
template <int D, int GPT, int SB, int NT>
__device__ __forceinline__ void merge_slices(__amdgpu_buffer_rsrc_t prs, unsigned char* smem, uint16_t* out,
                                             int64_t b, int g, int hq, int G, int n_split, int tid) {
  const int stride = 2 * G + G * D;
  const int n_g4 = G * (D / 4);
  float* st = reinterpret_cast<float*>(smem);  // [SB][2G] maxima and sums of the batch
  float Mr[GPT], Lr[GPT];
  f32x4_t Or[GPT];
#pragma unroll
  for (int q4 = 0; q4 < GPT; ++q4) {
    Mr[q4] = -__builtin_inff();
    Lr[q4] = 0.f;
    Or[q4] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  for (int s0 = 0; s0 < n_split; s0 += SB) {
    const int nb = n_split - s0 < SB ? n_split - s0 : SB;
    __syncthreads();  // the previous batch's statistics are consumed
    for (int i = tid; i < nb * 2 * G; i += NT) {
      const int sl = i / (2 * G), j = i % (2 * G);
      st[i] = __uint_as_float(load_coherent(prs, (s0 + sl) * stride + j));
    }
    f32x4_t ov[GPT][SB];
#pragma unroll
    for (int q4 = 0; q4 < GPT; ++q4) {
      const int gi = tid + NT * q4;
      const int h = gi / (D / 4), e4 = 4 * (gi % (D / 4));
#pragma unroll
      for (int j = 0; j < SB; ++j)
        ov[q4][j] = (gi < n_g4 && j < nb)
                        ? __builtin_bit_cast(f32x4_t, load4_coherent(prs, (s0 + j) * stride + 2 * G + h * D + e4))
                        : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();
#pragma unroll
    for (int q4 = 0; q4 < GPT; ++q4) {
      const int gi = tid + NT * q4;
      if (gi >= n_g4) continue;
      const int h = gi / (D / 4);
      float ms[SB];
      float mb = Mr[q4];
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        ms[j] = j < nb ? st[j * 2 * G + h] : -__builtin_inff();
        mb = fmaxf(mb, ms[j]);
      }
      if (mb == -__builtin_inff()) continue;  // no visible key so far
      const float a = __builtin_amdgcn_exp2f(Mr[q4] - mb);  // 0 while Mr = -inf
      Lr[q4] *= a;
      Or[q4] *= a;
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        const float f = __builtin_amdgcn_exp2f(ms[j] - mb);  // 0 for empty and missing slices
        Lr[q4] += j < nb ? f * st[j * 2 * G + G + h] : 0.f;
        Or[q4] += f * ov[q4][j];
      }
      Mr[q4] = mb;
    }
  }
#pragma unroll
  for (int q4 = 0; q4 < GPT; ++q4) {
    const int gi = tid + NT * q4;
    if (gi >= n_g4) continue;
    const int h = gi / (D / 4), e4 = 4 * (gi % (D / 4));
    const float inv = 1.f / Lr[q4];
    const u32x2_t v = {pack_bf16x2(Or[q4][0] * inv, Or[q4][1] * inv), pack_bf16x2(Or[q4][2] * inv, Or[q4][3] * inv)};
    *reinterpret_cast<u32x2_t*>(out + (b * hq + (int64_t)g * G + h) * D + e4) = v;
  }
}

// End of a row slice attended by the NW waves of a workgroup (call with every
// thread, after attend_units and sum_col4): the waves' softmax states merge
// in LDS in wave order; with one slice per row that is the output, else the
// slice's state goes to the workspace with device-coherent stores, the
// workgroup takes a ticket from the row's arrival counter, and the last one
// to arrive merges all slices in slice order and resets the counter.
//
// ROT (the rotated 8-bit cache): the workgroup's combined state is rotated
// back (H o / D per head, the float32 butterflies) before it is written or
// merged; the rotation is linear, so the slices' merge commutes with it.
// The combine area then needs (NW + 1) * (32 + 16 D) floats.
template <int D, int NW, bool ROT = false>
__device__ void finish_row_slice(float m_run, float l_run, const f32x4_t (&o)[D / 16], unsigned char* smem,
                                 int* last_flag, uint16_t* __restrict__ out, float* part, uint32_t* counters,
                                 int64_t row, int64_t b, int g, int hq, int G, int split, int n_split) {
  constexpr int NT = NW * kWave;
  constexpr int DT = D / 16;
  const int lane = lane_id(), w = wave_id(), tid = threadIdx.x;
  const int lg = lane / 16, col = lane % 16;
  __syncthreads();  // staging area becomes the combine area
  // row stride of co padded by 16 bytes: the 16 lanes of a lane group write
  // rows 16 bytes apart in the banks, not all into the same four banks
  constexpr int CS = kCombStride<D>;
  float* cm = reinterpret_cast<float*>(smem);  // [NW][16] running maxima
  float* cl = cm + NW * 16;                    // [NW][16] sums
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
  if constexpr (ROT) {
    constexpr int EPL = D / kWave;
    float* bm = co + NW * 16 * CS;  // [16] the workgroup's maxima
    float* bl = bm + 16;           // [16] sums
    float* bo = bl + 16;           // [16][D] outputs, rotated back below
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
        bm[h] = M;
        bl[h] = L;
      }
      bo[idx] = O;
    }
    __syncthreads();
    constexpr float inv_d = 1.0f / D;  // exact: D is a power of two
    for (int h = w; h < G; h += NW) {
      float x[EPL];
#pragma unroll
      for (int i = 0; i < EPL; ++i) x[i] = bo[h * D + lane + kWave * i];
      fwht_wave<D>(x);
#pragma unroll
      for (int i = 0; i < EPL; ++i) bo[h * D + lane + kWave * i] = x[i] * inv_d;
    }
    __syncthreads();
    if (n_split == 1) {
      for (int idx = tid; idx < G * D; idx += NT)
        out[(b * hq + (int64_t)g * G + idx / D) * D + idx % D] = f32_to_bf16(bo[idx] / bl[idx / D]);
      return;
    }
    const int stride = 2 * G + G * D;
    const auto prs = __builtin_amdgcn_make_buffer_rsrc(part + row * (int64_t)n_split * stride, 0,
                                                       n_split * stride * 4, kBufferFlags);
    const int soff = split * stride;
    for (int idx = tid; idx < G * D; idx += NT) {
      if (idx % D == 0) {
        store_coherent(prs, soff + idx / D, __float_as_uint(bm[idx / D]));
        store_coherent(prs, soff + G + idx / D, __float_as_uint(bl[idx / D]));
      }
      store_coherent(prs, soff + 2 * G + idx, __float_as_uint(bo[idx]));
    }
    __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
    __syncthreads();
    if (tid == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(counters + row, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool last = prev == (uint32_t)(n_split - 1);
      if (last) __hip_atomic_store(counters + row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *last_flag = last ? 1 : 0;
    }
    __syncthreads();
    if (!*last_flag) return;
    if (G * (D / 4) <= NT) merge_slices<D, 1, 16, NT>(prs, smem, out, b, g, hq, G, n_split, tid);
    else merge_slices<D, 2, 8, NT>(prs, smem, out, b, g, hq, G, n_split, tid);
    return;
  }
  if (n_split == 1) {
    for (int idx = tid; idx < G * D; idx += NT) {
      const int h = idx / D, e = idx % D;
      float M = -__builtin_inff();
      for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, cm[ww * 16 + h]);
      float L = 0.f, O = 0.f;
      for (int ww = 0; ww < NW; ++ww) {
        const float f = __builtin_amdgcn_exp2f(cm[ww * 16 + h] - M);  // 0 for waves without a unit
        L += f * cl[ww * 16 + h];
        O += f * co[(ww * 16 + h) * CS + e];
      }
      out[(b * hq + (int64_t)g * G + h) * D + e] = f32_to_bf16(O / L);
    }
    return;
  }
  const int stride = 2 * G + G * D;
  const auto prs = __builtin_amdgcn_make_buffer_rsrc(part + row * (int64_t)n_split * stride, 0,
                                                     n_split * stride * 4, kBufferFlags);
  const int soff = split * stride;
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
    *last_flag = last ? 1 : 0;
  }
  __syncthreads();
  if (!*last_flag) return;
  if (G * (D / 4) <= NT) merge_slices<D, 1, 16, NT>(prs, smem, out, b, g, hq, G, n_split, tid);
  else merge_slices<D, 2, 8, NT>(prs, smem, out, b, g, hq, G, n_split, tid);
}

}  // namespace qsa
