// Wave-level pieces of the block selection shared by the selection kernels
// and the fused decode step: the row frame, streaming dot products of 64
// compressed keys, the final id-ordered write of a row, and the merge of the
// waves' top lists. See qsa_select.hip for the method and its sources.
#pragma once

#include "qsa_device.h"

namespace qsa {

// Candidates 0 .. n_cand-1 and the always-kept block (-1: none) of a row
// whose query sits at absolute position p.
struct Frame {
  int n_cand;
  int forced;
};
__device__ __forceinline__ Frame row_frame(int64_t p, int bs, int keep_tail) {
  if (!keep_tail) {
    const int own = (int)(p / bs);
    return Frame{own, own};
  }
  const int n = (int)((p + 1) / bs);
  return Frame{n, ((p + 1) % bs) ? n : -1};
}
__device__ __forceinline__ int frame_slots(const Frame& f, int top_k) {
  return f.n_cand < top_k - 1 ? f.n_cand : top_k - 1;
}

// Write one row's selection from the kept keys held one per lane (lanes <
// slots valid, any order): ids ascending, forced block last, -1 padding.
// ids_lds, when given, receives the same ids (LDS, top_k entries); sel_row
// may then be null.
__device__ __forceinline__ void finalize_row(uint64_t cur, int slots, int forced, int top_k, int32_t* sel_row,
                                             float* score_row, int* ids_lds = nullptr) {
  const int lane = lane_id();
  const int n_real = slots + (forced >= 0 ? 1 : 0);
  int id = lane < slots ? key_id(cur) : forced;
  float sc = lane < slots ? key_score(cur) : __builtin_inff();
  // Sort the n_real entries by ascending id: descending on the complemented
  // id, with the smallest network that holds them.
  uint64_t k2 = lane < n_real ? (((uint64_t)(0xFFFFFFFFu - (uint32_t)id) << 32) | __float_as_uint(sc)) : 0ull;
  if (n_real <= 16) k2 = wave_sort_desc_n<16>(k2);
  else if (n_real <= 32) k2 = wave_sort_desc_n<32>(k2);
  else k2 = wave_sort_desc_n<64>(k2);
  const bool real = lane < n_real;
  const int out_id = real ? (int)(0xFFFFFFFFu - (uint32_t)(k2 >> 32)) : -1;
  const float out_sc = real ? __uint_as_float((uint32_t)k2) : -__builtin_inff();
  if (lane < top_k) {
    if (sel_row) sel_row[lane] = out_id;
    if (score_row) score_row[lane] = out_sc;
    if (ids_lds) ids_lds[lane] = out_id;
  }
}

// Merge the descending lists of the NW waves of a workgroup (lists[w][lane]
// holds wave w's list) in a tree; wave 0 returns the merged list (other
// waves return their partial lists). Every wave must call it.
template <int NW = 4>
__device__ uint64_t merge_wave_lists(uint64_t (*lists)[kWave], uint64_t cur, int m) {
  const int lane = lane_id(), w = wave_id();
  lists[w][lane] = cur;
  __syncthreads();
#pragma unroll
  for (int span = 1; span < NW; span *= 2) {
    if (w % (2 * span) == 0) {
      cur = topk_fold_sorted(cur, lists[w + span][lane], m);
      lists[w][lane] = cur;
    }
    __syncthreads();
  }
  return cur;
}


// Dot products of 64 consecutive compressed keys with qbar, one per lane.
// Lane l reads the 16-byte column slice (l % LPR) of its rows, so every load
// instruction covers 1 KiB of consecutive keys. A pass issues 16 loads; a
// transpose-reduce butterfly over lane bits 3..0 leaves each lane one row of
// the pass summed over 16 lanes, and plain xor-reductions over the remaining
// lane bits of the row finish the sum. Row held by lane l: see dot64_row().
template <int D>
__device__ __forceinline__ int dot64_row(int lane) {
  constexpr int LPR = D / 4;
  constexpr int RPL = kWave / LPR;
  constexpr int ROWS_PASS = 16 * RPL;
  const int pass = (kWave / ROWS_PASS == 2) ? ((lane >> 4) & 1) : 0;
  return pass * ROWS_PASS + RPL * (lane % 16) + lane / LPR;
}

// BATCH: every load of the 64 rows is issued before the first product
// (PASSES x 16 per lane in flight; measured faster for the selection scans
// at 1M and 256K positions); otherwise the compiler interleaves loads and
// products (measured faster inside the fused decode step).
template <int D, bool BATCH = false>
__device__ __forceinline__ float dot64_rows(const float* __restrict__ rows_base, int64_t n_valid, const f32x4_t& qv) {
  constexpr int LPR = D / 4;               // lanes covering one key row
  constexpr int RPL = kWave / LPR;         // rows per load instruction
  constexpr int ROWS_PASS = 16 * RPL;      // rows per pass of 16 loads
  constexpr int PASSES = kWave / ROWS_PASS;
  const int lane = lane_id();
  // Rows past n_valid (>= 1) re-read the last valid row, so the loads need
  // no branches; the caller drops those rows' results.
  f32x4_t raw[PASSES][16];
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int row = pass * ROWS_PASS + RPL * j + lane / LPR;
      const int64_t r = row < n_valid ? row : n_valid - 1;
      raw[pass][j] = *reinterpret_cast<const f32x4_t*>(rows_base + r * D + 4 * (lane % LPR));
    }
  if constexpr (BATCH) __builtin_amdgcn_sched_barrier(0);  // every load above the products
  float res[PASSES];
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    float vals[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      vals[j] = raw[pass][j][0] * qv[0] + raw[pass][j][1] * qv[1] + raw[pass][j][2] * qv[2] + raw[pass][j][3] * qv[3];
    }
#pragma unroll
    for (int half = 8; half >= 1; half /= 2) {
      const bool upper = (lane & half) != 0;
#pragma unroll
      for (int v = 0; v < half; ++v) {
        float lo = vals[v], hi = vals[v + half];
        reg_fence(lo);  // opaque operands: keeps the selects from becoming indexed array reads
        reg_fence(hi);
        const float send = upper ? lo : hi;
        const float keep = upper ? hi : lo;
        vals[v] = keep + xor_lane_f32(send, half);
      }
    }
#pragma unroll
    for (int m = 16; m < LPR; m <<= 1) vals[0] += xor_lane_f32(vals[0], m);
    res[pass] = vals[0];
    reg_fence(res[pass]);
  }
  if constexpr (PASSES == 2) return ((lane >> 4) & 1) ? res[1] : res[0];
  return res[0];
}

// Mean of the bs keys of one block (src: the block's first key) by one wave,
// in the compression kernel's order: each lane accumulates its 16-byte column
// slice over the rows it visits (16 loads in flight at a time), then a
// butterfly over the lanes that share a slice finishes the sum. The D floats
// go to dst and, when given, to dst2.
template <typename T, int D>
__device__ __forceinline__ void compress_block_wave(const T* __restrict__ src, int bs, float* dst, float* dst2) {
  constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte load
  constexpr int LPR = D / VEC;         // lanes covering one key row
  constexpr int RPL = kWave / LPR;     // rows per wave-wide load
  const int lane = lane_id();
  const int row0 = lane / LPR;
  const int col = (lane % LPR) * VEC;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  for (int r0 = 0; r0 < bs; r0 += 16 * RPL) {
    u32x4_t raw[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = r0 + j * RPL + row0;
      raw[j] = r < bs ? *reinterpret_cast<const u32x4_t*>(src + (int64_t)r * D + col) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          acc[2 * h] += bf16_lo(raw[j][h]);
          acc[2 * h + 1] += bf16_hi(raw[j][h]);
        }
      } else {
#pragma unroll
        for (int h = 0; h < 4; ++h) acc[h] += __uint_as_float(raw[j][h]);
      }
    }
  }
#pragma unroll
  for (int m = LPR; m < kWave; m <<= 1)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += shfl_xor_f32(acc[e], m);
  if (row0 == 0) {
    const float inv = 1.0f / (float)bs;  // exact: bs is a power of two
#pragma unroll
    for (int e = 0; e < VEC; e += 4) {
      const f32x4_t v = {acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
      if (dst) *reinterpret_cast<f32x4_t*>(dst + col + e) = v;
      if (dst2) *reinterpret_cast<f32x4_t*>(dst2 + col + e) = v;
    }
  }
}

}  // namespace qsa
