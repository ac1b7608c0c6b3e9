// Device helpers shared by the QSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Keeps a value in a VGPR at this point: stops the optimiser from fusing
// lane-dependent selects across steps of a butterfly into index chains.
__device__ __forceinline__ void reg_fence(float& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round-to-nearest-even float -> bf16 (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Element loads of the two supported storage types, widened to float.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
};

// Four consecutive elements widened to float (one 8- or 16-byte load).
__device__ __forceinline__ f32x4_t load4_f32(const float* p) { return *reinterpret_cast<const f32x4_t*>(p); }
__device__ __forceinline__ f32x4_t load4_f32(const uint16_t* p) {
  const u32x2_t w = *reinterpret_cast<const u32x2_t*>(p);
  return f32x4_t{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
}

// Sum over the G (<= 16) query heads of a group of four consecutive dims:
// p points at head 0, heads are `stride` elements apart. The sum runs in
// head order from 0.
template <int GC, typename T>
__device__ __forceinline__ f32x4_t group_sum4_n(const T* p, int64_t stride) {
  // keeps the loads (head 0's, common to every case) from being hoisted
  // above the dispatch, where the compiler would wait for it on its own
  asm volatile("" ::: "memory");
  f32x4_t v[GC];
#pragma unroll
  for (int j = 0; j < GC; ++j) v[j] = load4_f32(p + j * stride);
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < GC; ++j) s += v[j];
  return s;
}
// group_sum4_n for NR rows at once (row r's head 0 at p[r]): every load of
// the NR rows is issued before the first add, so the rows cost one memory
// round trip together; sums in head order as above.
template <int GC, int NR, typename T>
__device__ __forceinline__ void group_sum4_rows(const T* const (&p)[NR], int64_t stride, f32x4_t (&out)[NR]) {
  asm volatile("" ::: "memory");
  f32x4_t v[NR][GC];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int j = 0; j < GC; ++j) v[r][j] = load4_f32(p[r] + j * stride);
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < GC; ++j) s += v[r][j];
    out[r] = s;
  }
}
// G is one of 1, 2, 4, 8, 16 (uniform over the wave). Each case issues all
// its loads before the first add: with a runtime bound on the head loop the
// compiler guards every load with a branch and waits for it inside the
// branch, which makes the G loads one memory round trip each.
template <typename T>
__device__ __forceinline__ f32x4_t group_sum4(const T* p, int G, int64_t stride) {
  switch (G) {
    case 1: return group_sum4_n<1>(p, stride);
    case 2: return group_sum4_n<2>(p, stride);
    case 4: return group_sum4_n<4>(p, stride);
    case 8: return group_sum4_n<8>(p, stride);
    default: return group_sum4_n<16>(p, stride);
  }
}

// ---------------------------------------------------------------- shuffles

__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int mask) {
  return (uint32_t)__shfl_xor((int)v, mask, kWave);
}
__device__ __forceinline__ float shfl_xor_f32(float v, int mask) { return __shfl_xor(v, mask, kWave); }
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  uint32_t lo = shfl_xor_u32((uint32_t)v, mask);
  uint32_t hi = shfl_xor_u32((uint32_t)(v >> 32), mask);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = (uint32_t)__shfl((int)(uint32_t)v, src, kWave);
  uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), src, kWave);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ float wave_max_f32(float v) {
  for (int m = 32; m > 0; m >>= 1) v = fmaxf(v, shfl_xor_f32(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  for (int m = 32; m > 0; m >>= 1) v += shfl_xor_f32(v, m);
  return v;
}

// ---------------------------------------------------------------- selection keys
//
// A candidate block is ranked by (score descending, block id ascending).
// Both go into one 64-bit key so that a larger key is a better candidate:
// high word = order-preserving image of the float score (-0 folded onto +0),
// low word = ~id. Key 0 is below every real key and marks "no candidate".

__device__ __forceinline__ uint32_t score_order_bits(float s) {
  uint32_t u = (s == 0.0f) ? 0u : __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t make_key(float score, int id) {
  return ((uint64_t)score_order_bits(score) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}
__device__ __forceinline__ int key_id(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }
__device__ __forceinline__ float key_score(uint64_t key) {
  uint32_t o = (uint32_t)(key >> 32);
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

// v_permlane16_swap / v_permlane32_swap with both operands = v: element 0
// holds v of the lower half of each 32-lane (resp. 64-lane) group in both
// halves, element 1 the upper half. So lane l sees v[l & ~16] and v[l | 16]
// (resp. v[l & ~32] and v[l | 32]) in one VALU instruction.
__device__ __forceinline__ uint32_t xor16_u32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return (lane_id() & 16) ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t xor32_u32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (lane_id() & 32) ? r[0] : r[1];
}
// max / sum over the four lanes {l, l^16, l^32, l^48} (one MFMA output column).
__device__ __forceinline__ float max_col4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_col4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Lane exchange with lane ^ j for a compile-time j (after unrolling).
// xor 1, 2: DPP quad permutes; xor 4: two DPP row rotations (row_ror:N
// moves lane i to lane i+N within its row of 16); xor 8: DPP row_ror:8;
// xor 16, 32: permlane swaps.
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t v, int j) {
  const int x = (int)v;
  switch (j) {
    case 1:
      return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);
    case 2:
      return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);
    case 4: {
      const int up = __builtin_amdgcn_mov_dpp(x, 0x12C, 0xF, 0xF, false);    // lane i <- i+4
      const int down = __builtin_amdgcn_mov_dpp(x, 0x124, 0xF, 0xF, false);  // lane i <- i-4
      return (uint32_t)((lane_id() & 4) ? down : up);
    }
    case 8:
      return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);
    case 16:
      return xor16_u32(v);
    case 32:
      return xor32_u32(v);
    default:
      return (uint32_t)__builtin_amdgcn_ds_bpermute((lane_id() ^ j) << 2, x);
  }
}
__device__ __forceinline__ uint64_t xor_lane_u64(uint64_t v, int j) {
  const uint32_t lo = xor_lane_u32((uint32_t)v, j);
  const uint32_t hi = xor_lane_u32((uint32_t)(v >> 32), j);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ float xor_lane_f32(float v, int j) {
  return __uint_as_float(xor_lane_u32(__float_as_uint(v), j));
}

// Lane sums with xor butterflies (DPP and permlane steps, no LDS round trips):
// total over the wave, inclusive prefix (lanes <= l) and inclusive suffix
// (lanes >= l). At step j every lane holds the total of its aligned group of
// j lanes; the partner group is the other half of the group of 2j.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int j = 1; j < kWave; j <<= 1) v += xor_lane_u32(v, j);
  return v;
}
__device__ __forceinline__ uint32_t wave_prefix_sum_u32(uint32_t v) {
  const int lane = lane_id();
  uint32_t total = v;
#pragma unroll
  for (int j = 1; j < kWave; j <<= 1) {
    const uint32_t t = xor_lane_u32(total, j);
    if (lane & j) v += t;
    total += t;
  }
  return v;
}
__device__ __forceinline__ uint32_t wave_suffix_sum_u32(uint32_t v) {
  const int lane = lane_id();
  uint32_t total = v;
#pragma unroll
  for (int j = 1; j < kWave; j <<= 1) {
    const uint32_t t = xor_lane_u32(total, j);
    if (!(lane & j)) v += t;
    total += t;
  }
  return v;
}

// Compare-exchange of a bitonic network: the larger of x and its partner y
// where take_max holds, else the smaller. One comparison decides which to
// keep (x == y: either, the same key); written this way the compiler emits
// one 64-bit compare, a lane-mask operation and two selects, rather than
// both a maximum and a minimum and a select between them.
__device__ __forceinline__ uint64_t cas_u64(uint64_t x, uint64_t y, bool take_max) {
  return ((x > y) == take_max) ? x : y;
}

__device__ __forceinline__ uint32_t cas_u32(uint32_t x, uint32_t y, bool take_max) {
  return ((x > y) == take_max) ? x : y;
}

// Bitonic sort of one 32-bit value per lane across the wave, descending.
__device__ __forceinline__ uint32_t wave_sort_desc_u32(uint32_t x) {
  const int lane = lane_id();
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint32_t y = xor_lane_u32(x, j);
      const bool lower = (lane & j) == 0;
      const bool desc = (lane & k) == 0;
      x = cas_u32(x, y, lower == desc);
    }
  }
  return x;
}

// Bitonic sort of one key per lane across the wave, descending (lane 0 = largest).
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t x) {
  const int lane = lane_id();
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      uint64_t y = xor_lane_u64(x, j);
      bool lower = (lane & j) == 0;
      bool desc = (lane & k) == 0;
      bool take_max = (lower == desc);
      x = cas_u64(x, y, take_max);
    }
  }
  return x;
}

// Same network restricted to groups of N lanes (N = 16, 32 or 64): the first
// group is sorted descending (groups alternate direction after it).
template <int N>
__device__ __forceinline__ uint64_t wave_sort_desc_n(uint64_t x) {
  const int lane = lane_id();
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      uint64_t y = xor_lane_u64(x, j);
      bool lower = (lane & j) == 0;
      bool desc = (lane & k) == 0;
      bool take_max = (lower == desc);
      x = cas_u64(x, y, take_max);
    }
  }
  return x;
}

// ------------------------------------------------------------ threshold select
//
// Exact selection of the m largest of the keys held P per lane (key 0 =
// empty slot, never selected) without sorting: the m-th largest key is found
// bit by bit from the most significant end, counting keys at or above each
// trial value with ballots. Keys are distinct (the low word is the
// complemented block id), so exactly min(m, #keys) keys are >= the result.

__device__ __forceinline__ int lanes_set(bool pred) { return __builtin_popcountll(__ballot(pred)); }

// Smallest key value T with exactly min(m, #nonzero keys) keys >= T
// (1 when there are fewer than m keys).
template <int P>
__device__ __forceinline__ uint64_t kth_largest_key(const uint64_t (&x)[P], int m) {
  uint32_t h[P], l[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    h[p] = (uint32_t)(x[p] >> 32);
    l[p] = (uint32_t)x[p];
  }
  // Largest th with #(high word >= th) >= m. Real keys have a nonzero high
  // word (the order image of a finite float), so th = 0 means < m keys.
  uint32_t th = 0;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = th | (1u << bit);
    int n = 0;
#pragma unroll
    for (int p = 0; p < P; ++p) n += lanes_set(h[p] >= c);
    th = n >= m ? c : th;
  }
  if (th == 0) return 1ull;
  int n_gt = 0, n_ge = 0;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    n_gt += lanes_set(h[p] > th);
    n_ge += lanes_set(h[p] >= th);
  }
  if (n_ge == m) return (uint64_t)th << 32;
  // High words tie at th: keep the (m - n_gt) largest low words among them.
  const int need = m - n_gt;
  uint32_t tl = 0;
#pragma unroll 4
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = tl | (1u << bit);
    int n = 0;
#pragma unroll
    for (int p = 0; p < P; ++p) n += lanes_set(h[p] == th && l[p] >= c);
    tl = n >= need ? c : tl;
  }
  return ((uint64_t)th << 32) | tl;
}

// Keys >= t (t >= 1) packed into lanes 0 .. count-1 in no particular order;
// `scratch` is 64 keys of LDS owned by the calling wave.
template <int P>
__device__ __forceinline__ uint64_t gather_keys_ge(const uint64_t (&x)[P], uint64_t t, uint64_t* scratch, int& count) {
  int base = 0;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const bool s = x[p] >= t;
    const uint64_t msk = __ballot(s);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(msk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)msk, 0));
    if (s) scratch[base + below] = x[p];
    base += __builtin_popcountll(msk);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint64_t r = lane_id() < base ? scratch[lane_id()] : 0ull;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  count = base;
  return r;
}

// Running top-m set of one row kept by one wave: `keys` in lanes < count,
// unordered; `thr` = the last selection threshold (every kept key is >= it).
struct TopSet {
  uint64_t keys;
  int count;
  uint64_t thr;
};

// Absorb P fresh keys per lane into the set (skipped when the set is full
// and no fresh key beats its threshold).
template <int P>
__device__ __forceinline__ void topset_absorb(TopSet& s, const uint64_t (&fresh)[P], int m, uint64_t* scratch) {
  if (s.count == m) {
    bool any = false;
#pragma unroll
    for (int p = 0; p < P; ++p) any |= fresh[p] > s.thr;
    if (__ballot(any) == 0) return;
  }
  uint64_t x[P + 1];
#pragma unroll
  for (int p = 0; p < P; ++p) x[p] = fresh[p];
  x[P] = s.keys;
  s.thr = kth_largest_key<P + 1>(x, m);
  s.keys = gather_keys_ge<P + 1>(x, s.thr, scratch, s.count);
}

// Top-64 of two descending lists held one key per lane; result descending.
__device__ __forceinline__ uint64_t wave_merge_desc(uint64_t cur, uint64_t fresh_desc) {
  const int lane = lane_id();
  uint64_t rev = shfl_u64(fresh_desc, kWave - 1 - lane);
  uint64_t x = cur > rev ? cur : rev;  // bitonic sequence holding the top 64
#pragma unroll
  for (int j = kWave / 2; j > 0; j >>= 1) {
    uint64_t y = xor_lane_u64(x, j);
    bool lower = (lane & j) == 0;
    x = cas_u64(x, y, lower);
  }
  return x;
}

// Value of `v` in lane `src` (wave-uniform src), via the scalar unit.
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int src) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

// LDS written by some lanes of a wave made visible to the others (the wave's
// LDS operations run in order; this keeps the compiler from reordering them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The 16 largest of 256 keys held four per lane (0 = empty; the others
// distinct), descending in lanes 0..15 (0 in the other lanes).
// Cut: the 16th largest lane maximum M bounds the 16th largest key from
// below (the 16 largest maxima are keys >= M), so every one of the 16 best
// keys has a high word (score image) >= th, the 16th largest high word of
// the lane maxima. When exactly 16 lanes have a maximum whose high word
// reaches th, the keys above the cut lie in those lanes: at most 64. (When
// high words tie at th the cut is M itself, from a sort of the whole keys;
// with fewer than 16 non-empty lanes every key survives, at most 60.)
// Order: the survivors are gathered (scratch: 64 keys of LDS owned by the
// calling wave), each lane counts the survivors above its own key, and the
// keys of rank < 16 are placed by that rank. The cut sorts 32-bit words and
// the order needs no sort: about half the instructions of two 64-bit sorts.
__device__ __forceinline__ uint64_t top16_of_256(const uint64_t (&x)[4], uint64_t* scratch) {
  const int lane = lane_id();
  const uint64_t m01 = x[0] > x[1] ? x[0] : x[1];
  const uint64_t m23 = x[2] > x[3] ? x[2] : x[3];
  const uint64_t m = m01 > m23 ? m01 : m23;
  const uint32_t mh = (uint32_t)(m >> 32);
  const uint32_t th = (uint32_t)__builtin_amdgcn_readlane((int)wave_sort_desc_u32(mh), 15);
  uint64_t t;
  if (th == 0u)
    t = 1ull;  // fewer than 16 non-empty lanes (real keys have a nonzero high word)
  else if (lanes_set(mh >= th) == 16)
    t = (uint64_t)th << 32;
  else
    t = readlane_u64(wave_sort_desc(m), 15);
  // survivors (keys >= t) into scratch[0, c), zeros in scratch[c, 64)
  int c = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const bool s = x[p] >= t;
    const uint64_t msk = __ballot(s);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(msk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)msk, 0));
    if (s) scratch[c + below] = x[p];
    c += __builtin_popcountll(msk);
  }
  if (lane >= c) scratch[lane] = 0ull;
  wave_lds_sync();
  const uint64_t r = scratch[lane];
  uint32_t rank = 0u;  // survivors above r
  const int n8 = ((c < kWave ? c : kWave) + 7) & ~7;
  for (int j0 = 0; j0 < n8; j0 += 8) {
    uint64_t y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = scratch[j0 + i];
#pragma unroll
    for (int i = 0; i < 8; ++i) rank += y[i] > r ? 1u : 0u;
  }
  wave_lds_sync();
  // the key of rank i < 16 to scratch[i]; lanes c .. 15 clear theirs (ranks
  // are below c, so the two sets of addresses are disjoint)
  const bool put = r != 0ull && rank < 16u;
  const bool clear = lane >= c && lane < 16;
  if (put || clear) scratch[put ? (int)rank : lane] = put ? r : 0ull;
  wave_lds_sync();
  const uint64_t out = lane < 16 ? scratch[lane] : 0ull;
  wave_lds_sync();
  return out;
}

// Fold one lane-per-candidate batch into a running descending top list
// (`cur`, lane j = j-th best). Only the first `m` entries of `cur` matter;
// the batch is skipped when no key beats the current m-th best.
__device__ __forceinline__ uint64_t topk_fold(uint64_t cur, uint64_t fresh, int m) {
  const uint64_t thr = readlane_u64(cur, m - 1);
  if (__ballot(fresh > thr) == 0) return cur;
  return wave_merge_desc(cur, wave_sort_desc(fresh));
}

// Same for a batch that is already a descending list.
__device__ __forceinline__ uint64_t topk_fold_sorted(uint64_t cur, uint64_t fresh_desc, int m) {
  const uint64_t thr = readlane_u64(cur, m - 1);
  if (readlane_u64(fresh_desc, 0) <= thr) return cur;
  return wave_merge_desc(cur, fresh_desc);
}

// ---------------------------------------------------------------- device-coherent access
//
// Buffer loads and stores with cache policy sc1 reach the device-coherent
// level directly (no L2 write-back or invalidate of other data), so workgroups
// of one kernel on different XCDs can hand data over once the stores have
// completed. Offsets are in 4-byte words from the resource base.

constexpr int kBufferFlags = 0x00020000;  // raw buffer resource word 3 for gfx950
constexpr int kPolicySc1 = 16;

__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t rs, int word, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, rs, word * 4, 0, kPolicySc1);
}
__device__ __forceinline__ uint32_t load_coherent(__amdgpu_buffer_rsrc_t rs, int word) {
  return __builtin_amdgcn_raw_buffer_load_b32(rs, word * 4, 0, kPolicySc1);
}
__device__ __forceinline__ u32x4_t load4_coherent(__amdgpu_buffer_rsrc_t rs, int word) {
  return __builtin_amdgcn_raw_buffer_load_b128(rs, word * 4, 0, kPolicySc1);
}
__device__ __forceinline__ u32x2_t load2_coherent(__amdgpu_buffer_rsrc_t rs, int word) {
  return __builtin_amdgcn_raw_buffer_load_b64(rs, word * 4, 0, kPolicySc1);
}
__device__ __forceinline__ void store2_coherent(__amdgpu_buffer_rsrc_t rs, int word, uint32_t lo, uint32_t hi) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{lo, hi}, rs, word * 4, 0, kPolicySc1);
}

// ---------------------------------------------------------------- MFMA

__device__ __forceinline__ f32x4_t mfma_bf16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

}  // namespace qsa
