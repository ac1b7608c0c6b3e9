// The large-k selection's cutoff and id extraction (k > 64), shared by the
// selection kernels and the fused pick-and-attend kernel of the decode step.
// See qsa_select.hip for the method.
#pragma once

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

constexpr int kLargeChunk = 256;   // candidates per score workgroup (4 waves x 64)
constexpr int kLargeList = 16;     // best keys kept per chunk
constexpr int kPickThreads = 512;
constexpr int kListPerThread = 8;   // keys per pick thread in the pool of chunk lists
constexpr int kPoolPerThread = 24;  // keys per pick thread in a pool of whole chunks
constexpr int kPoolCap = kPickThreads * kPoolPerThread;
static_assert(kPickThreads * kListPerThread == kLargeList * (kMaxCandLarge / kLargeChunk), "list pool");
constexpr int kBitmapWords = (int)(kMaxCandLarge / 32);
// A re-expanded chunk has all 16 list keys at or above the pool cutoff, so at
// most (top_k - 1) / 16 chunks expand: the second pool stays within capacity.
static_assert(kLargeList * (kMaxCandLarge / kLargeChunk) +
                  (kLargeChunk - kLargeList) * ((kMaxTopKLarge - 1) / kLargeList) <= kPoolCap,
              "pool capacity");

__device__ __forceinline__ float order_to_float(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

struct PickSmem {
  uint32_t bitmap[kBitmapWords];    // kept candidates
  uint32_t word_pre[kBitmapWords];  // kept candidates in the words before
  static_assert(kBitmapWords % kPickThreads == 0, "bitmap words per thread");
  uint32_t hist[2][256];            // radix histograms (alternating)
  uint64_t red_max[kPickThreads / kWave], red_min[kPickThreads / kWave];
  int red_cnt[kPickThreads / kWave];
  uint32_t wave_tot[kPickThreads / kWave];
  uint32_t digit[3];                // chosen digit, keys above its bin, keys in its bin
  uint64_t last[kMaxCandLarge / kLargeChunk];  // 16th list key of every chunk
  uint32_t sat_mask[8];             // re-expanded chunks
  int sat_list[kMaxCandLarge / kLargeChunk];
  int n_sat;
};

__device__ __forceinline__ uint64_t high_bits(uint64_t x, int n_low) { return n_low >= 64 ? 0ull : x >> n_low; }

// Smallest key value T such that exactly min(m, #keys) of the nonzero keys
// held by the workgroup (KP per thread, distinct) are >= T; 1 when there are
// none. Most-significant-digit radix descent with 8-bit digits, starting at
// the highest bit in which the largest and smallest key differ, and stopping
// as soon as the remaining keys of the chosen bin are all needed.
template <int KP>
__device__ uint64_t block_kth_largest(const uint64_t (&x)[KP], int m, PickSmem& sm) {
  constexpr int NW = kPickThreads / kWave;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  __syncthreads();  // shared state of an earlier call fully consumed
  uint64_t mx = 0ull, mn = ~0ull;
  int cnt = 0;
#pragma unroll
  for (int p = 0; p < KP; ++p) {
    if (x[p] != 0ull) {
      mx = x[p] > mx ? x[p] : mx;
      mn = x[p] < mn ? x[p] : mn;
      ++cnt;
    }
  }
#pragma unroll
  for (int j = 1; j < kWave; j <<= 1) {
    const uint64_t a = xor_lane_u64(mx, j), c = xor_lane_u64(mn, j);
    mx = a > mx ? a : mx;
    mn = c < mn ? c : mn;
  }
  cnt = (int)wave_sum_u32((uint32_t)cnt);
  if (lane == 0) {
    sm.red_max[w] = mx;
    sm.red_min[w] = mn;
    sm.red_cnt[w] = cnt;
  }
  if (tid < 256) sm.hist[0][tid] = 0u;
  __syncthreads();
  mx = 0ull;
  mn = ~0ull;
  cnt = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    mx = sm.red_max[i] > mx ? sm.red_max[i] : mx;
    mn = sm.red_min[i] < mn ? sm.red_min[i] : mn;
    cnt += sm.red_cnt[i];
  }
  if (cnt == 0) return 1ull;
  if (cnt <= m) return mn;

  int cur = 64 - __builtin_clzll(mx ^ mn);  // low bits still open (mx != mn: >= 2 distinct keys)
  uint64_t prefix = high_bits(mx, cur);
  int need = m;
  int buf = 0;
  while (true) {
    const int wd = cur < 8 ? cur : 8;
    const int shift = cur - wd;
    const uint32_t dmask = (1u << wd) - 1u;
#pragma unroll
    for (int p = 0; p < KP; ++p)
      if (x[p] != 0ull && high_bits(x[p], cur) == prefix)
        atomicAdd(&sm.hist[buf][(uint32_t)(x[p] >> shift) & dmask], 1u);
    __syncthreads();
    if (w == 0) {
      uint32_t h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = sm.hist[buf][4 * lane + i];
      const uint32_t own = h[0] + h[1] + h[2] + h[3];
      // keys in the bins of higher lanes (higher digits)
      uint32_t above = wave_suffix_sum_u32(own) - own;
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if (above < (uint32_t)need && (uint32_t)need <= above + h[i]) {
          sm.digit[0] = 4 * lane + i;
          sm.digit[1] = above;
          sm.digit[2] = h[i];
        }
        above += h[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.hist[buf ^ 1][4 * lane + i] = 0u;
    }
    __syncthreads();
    const uint32_t d = sm.digit[0];
    need -= (int)sm.digit[1];
    const int in_bin = (int)sm.digit[2];
    prefix = (prefix << wd) | d;
    cur = shift;
    if (need == in_bin || cur == 0) return prefix << cur;
    buf ^= 1;
  }
}

// Cutoff and kept ids (ascending) of one row from its stored scores (order
// images, candidate c at sc_row[c]) and chunk lists; forced block and padding
// after them. sel_row / score_row may be null; ids_lds, when given, receives
// the top_k ids as well. Called by all kPickThreads threads of a workgroup.
static __device__ void pick_row(PickSmem& sm, const uint32_t* __restrict__ sc_row, const uint64_t* __restrict__ ls_row,
                         int n_cand, int slots, int forced, int top_k, int32_t* sel_row, float* score_row,
                         int* ids_lds) {
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  // forced block right after the kept ids, then padding
  for (int i = slots + tid; i < top_k; i += kPickThreads) {
    const bool f = i == slots && forced >= 0;
    if (sel_row) sel_row[i] = f ? forced : -1;
    if (score_row) score_row[i] = f ? __builtin_inff() : -__builtin_inff();
    if (ids_lds) ids_lds[i] = f ? forced : -1;
  }
  if (slots == 0) return;
  if (slots == n_cand) {  // every candidate kept
    for (int c = tid; c < n_cand; c += kPickThreads) {
      if (sel_row) sel_row[c] = c;
      if (score_row) score_row[c] = order_to_float(sc_row[c]);
      if (ids_lds) ids_lds[c] = c;
    }
    return;
  }
  const int n_words = (n_cand + 31) / 32;
  for (int i = tid; i < n_words; i += kPickThreads) sm.bitmap[i] = 0u;
  auto key_of = [&](int c) -> uint64_t {
    return ((uint64_t)sc_row[c] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)c);
  };

  uint64_t x[kPoolPerThread];  // the pool the cutoff is taken over (0 = empty)
  uint64_t cut;
  if (n_cand <= kPoolCap) {
#pragma unroll
    for (int p = 0; p < kPoolPerThread; ++p) {
      const int c = tid + kPickThreads * p;
      x[p] = c < n_cand ? key_of(c) : 0ull;
    }
    cut = block_kth_largest<kPoolPerThread>(x, slots, sm);
  } else {
    // first pool: the chunk lists (every chunk's 16 best)
    const int nch = (n_cand + kLargeChunk - 1) / kLargeChunk;
    const int n_list = nch * kLargeList;
    uint64_t y[kListPerThread];
#pragma unroll
    for (int p = 0; p < kListPerThread; ++p) {
      const int i = tid + kPickThreads * p;
      y[p] = i < n_list ? ls_row[i] : 0ull;
      if (i < n_list && i % kLargeList == kLargeList - 1) sm.last[i / kLargeList] = y[p];
    }
#pragma unroll
    for (int p = 0; p < kPoolPerThread; ++p) x[p] = p < kListPerThread ? y[p] : 0ull;
    if (tid < 8) sm.sat_mask[tid] = 0u;
    if (tid == 0) sm.n_sat = 0;
    cut = block_kth_largest<kListPerThread>(y, slots, sm);
    // A chunk whose 16th key reaches the cutoff may hold more kept keys than
    // its list shows; every other chunk's unlisted keys lie below the cutoff.
    for (int c = tid; c < nch; c += kPickThreads) {
      const uint64_t last = sm.last[c];
      if (last != 0ull && last >= cut) {
        sm.sat_list[atomicAdd(&sm.n_sat, 1)] = c;
        atomicOr(&sm.sat_mask[c >> 5], 1u << (c & 31));
      }
    }
    __syncthreads();
    const int n_sat = sm.n_sat;
    if (n_sat > 0) {
      // second pool: lists of the other chunks plus every key of the expanded ones
#pragma unroll
      for (int p = 0; p < kPoolPerThread; ++p) {
        const int i = tid + kPickThreads * p;
        uint64_t v = 0ull;
        if (i < n_list) {
          const int c = i / kLargeList;
          if (!((sm.sat_mask[c >> 5] >> (c & 31)) & 1u)) v = ls_row[i];
        } else if (i < n_list + n_sat * kLargeChunk) {
          const int j = i - n_list;
          const int c = sm.sat_list[j / kLargeChunk] * kLargeChunk + j % kLargeChunk;
          if (c < n_cand) v = key_of(c);
        }
        x[p] = v;
      }
      cut = block_kth_largest<kPoolPerThread>(x, slots, sm);
    }
  }

  // kept = keys >= cut (exactly `slots` of them); positions from the bitmap
#pragma unroll
  for (int p = 0; p < kPoolPerThread; ++p)
    if (x[p] != 0ull && x[p] >= cut) {
      const int id = key_id(x[p]);
      atomicOr(&sm.bitmap[id >> 5], 1u << (id & 31));
    }
  __syncthreads();
  // exclusive prefix of the kept counts over the bitmap words; thread t owns
  // words WPT*t .. WPT*t + WPT-1
  constexpr int WPT = kBitmapWords / kPickThreads;
  uint32_t cnt[WPT];
  uint32_t own = 0u;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int wi = WPT * tid + i;
    cnt[i] = wi < n_words ? (uint32_t)__builtin_popcount(sm.bitmap[wi]) : 0u;
    own += cnt[i];
  }
  const uint32_t incl = wave_prefix_sum_u32(own);
  if (lane == kWave - 1) sm.wave_tot[w] = incl;
  __syncthreads();
  uint32_t before = incl - own;
  for (int i = 0; i < w; ++i) before += sm.wave_tot[i];
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int wi = WPT * tid + i;
    if (wi < n_words) sm.word_pre[wi] = before;
    before += cnt[i];
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < kPoolPerThread; ++p)
    if (x[p] != 0ull && x[p] >= cut) {
      const int id = key_id(x[p]);
      const int pos = (int)(sm.word_pre[id >> 5] + __builtin_popcount(sm.bitmap[id >> 5] & ((1u << (id & 31)) - 1u)));
      if (pos < slots) {  // always true for distinct keys
        if (sel_row) sel_row[pos] = id;
        if (score_row) score_row[pos] = key_score(x[p]);
        if (ids_lds) ids_lds[pos] = id;
      }
    }
}


}  // namespace qsa
