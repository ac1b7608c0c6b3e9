// Indexer scoring and top-k block selection ("Qwen4 in llama.cpp: Dissecting
// PR #27742", section "QSA Is an Address-Selection Problem, Not a New
// Attention Equation": compressed blocks are scored, the top-k kept and
// turned into cache addresses).
//
// Score of candidate c for (token, KV head g): scale * <qbar, kc[c]> with
// qbar the float32 sum of the group's G query heads (equal to the sum of the
// per-head scores). Selection keeps the query's own block plus the
// min(k-1, i) best candidates, ranked by the 64-bit key of qsa_device.h
// (score descending, id ascending), and writes ids ascending.
//
// Two paths:
//  * tile path (many query rows, prefill): a workgroup takes 16 consecutive
//    rows of one (b, g), which share the candidate prefix. Candidate chunks
//    of 64 compressed keys are staged in LDS and scored with fp32 MFMA
//    (16x16x4, full fp32 products); every 128 candidates each wave updates
//    four rows' running top sets by threshold selection (the m-th largest
//    key found bit by bit with ballot counts, no sorting), and the final set
//    is sorted by id once.
//  * split path (few rows, decode): the candidates of a row are cut into
//    chunks spread over the whole GPU. Each wave streams 64 compressed keys
//    per step with fully coalesced 16-byte loads (1 KiB per instruction),
//    finishes the dot products with a transpose-reduce butterfly, and keeps a
//    running top list; the chunk's list goes to the workspace and a merge
//    kernel reduces the lists of a row, skipping every key below the best
//    chunk-local cutoff (a valid lower bound of the row's cutoff); when all
//    the lists of a row hold at most 256 keys, one wave takes them at once.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

// Write one row's selection from the kept keys held one per lane (lanes <
// slots valid, any order): ids ascending, own block last, -1 padding.
__device__ void finalize_row(uint64_t cur, int slots, int own, int top_k, int32_t* sel_row, float* score_row) {
  const int lane = lane_id();
  int id = lane < slots ? key_id(cur) : own;
  float sc = lane < slots ? key_score(cur) : __builtin_inff();
  // Sort lanes 0..slots by ascending id: descending on the complemented id,
  // with the smallest network that holds slots + 1 entries.
  uint64_t k2 = lane <= slots ? (((uint64_t)(0xFFFFFFFFu - (uint32_t)id) << 32) | __float_as_uint(sc)) : 0ull;
  if (slots < 16) k2 = wave_sort_desc_n<16>(k2);
  else if (slots < 32) k2 = wave_sort_desc_n<32>(k2);
  else k2 = wave_sort_desc_n<64>(k2);
  const bool real = lane <= slots;
  const int out_id = real ? (int)(0xFFFFFFFFu - (uint32_t)(k2 >> 32)) : -1;
  const float out_sc = real ? __uint_as_float((uint32_t)k2) : -__builtin_inff();
  if (lane < top_k) {
    sel_row[lane] = out_id;
    if (score_row) score_row[lane] = out_sc;
  }
}

// Merge the descending lists of the 4 waves of a workgroup (lists[w][lane]
// holds wave w's list); wave 0 returns the merged list, other waves return 0.
__device__ uint64_t merge_wave_lists(uint64_t (*lists)[kWave], uint64_t cur, int m) {
  const int lane = lane_id(), w = wave_id();
  lists[w][lane] = cur;
  __syncthreads();
  if (w == 0 || w == 2) {
    cur = topk_fold_sorted(cur, lists[w + 1][lane], m);
    lists[w][lane] = cur;
  }
  __syncthreads();
  if (w == 0) cur = topk_fold_sorted(cur, lists[2][lane], m);
  return cur;
}

// ------------------------------------------------------------------ tile path

constexpr int kTileRows = 16;
constexpr int kTileCands = 64;   // candidates staged and scored per pass
constexpr int kTilePasses = 2;   // passes per selection step (128 candidates, 2 per lane)

template <typename T, int D>
__global__ __launch_bounds__(256) void select_tile_kernel(const T* __restrict__ q, const float* __restrict__ k_comp,
                                                          int32_t* __restrict__ sel, float* __restrict__ sel_scores,
                                                          int64_t q_len, int64_t q_pos0, int64_t nb_cap, int hq,
                                                          int hkv, int G, int bs, int top_k, float scale) {
  constexpr int QP = D + 4;  // padded row strides (floats): conflict-free 16-byte reads
  constexpr int SPAN = kTileCands * kTilePasses;
  __shared__ float qbar[kTileRows][QP];
  __shared__ float kc[kTileCands][QP];
  __shared__ float sc[kTileRows][SPAN + 4];
  __shared__ uint64_t scratch[4][kWave];

  const int64_t t0 = (int64_t)blockIdx.x * kTileRows;
  const int g = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int64_t rows = q_len - t0 < kTileRows ? q_len - t0 : kTileRows;

  for (int idx = tid; idx < kTileRows * D / 4; idx += 256) {
    const int r = idx / (D / 4), e4 = (idx % (D / 4)) * 4;
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    if (r < rows) v = group_sum4(q + ((b * q_len + t0 + r) * hq + (int64_t)g * G) * D + e4, G, D);
    *reinterpret_cast<f32x4_t*>(&qbar[r][e4]) = v;
  }

  const int64_t own_last = (q_pos0 + t0 + rows - 1) / bs;  // candidates of every row are < own_last
  const float* kc_src = k_comp + ((b * hkv + g) * nb_cap) * D;
  TopSet set[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) set[rr] = TopSet{0ull, 0, 0ull};

  for (int64_t c0 = 0; c0 < own_last; c0 += SPAN) {
    // score SPAN candidates for all 16 rows, one staged pass of 64 at a time
#pragma unroll
    for (int pass = 0; pass < kTilePasses; ++pass) {
      const int64_t p0 = c0 + pass * kTileCands;
      __syncthreads();  // kc (and sc) of the previous pass fully consumed
      for (int idx = tid; idx < kTileCands * D / 4; idx += 256) {
        const int r = idx / (D / 4), e4 = (idx % (D / 4)) * 4;
        f32x4_t v = {0.f, 0.f, 0.f, 0.f};
        if (p0 + r < own_last) v = *reinterpret_cast<const f32x4_t*>(kc_src + (p0 + r) * D + e4);
        *reinterpret_cast<f32x4_t*>(&kc[r][e4]) = v;
      }
      __syncthreads();
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      const int m = lane % 16, kg = lane / 16;
#pragma unroll
      for (int u = 0; u < D / 16; ++u) {
        const f32x4_t a = *reinterpret_cast<const f32x4_t*>(&qbar[m][16 * u + 4 * kg]);
        const f32x4_t bv = *reinterpret_cast<const f32x4_t*>(&kc[16 * w + m][16 * u + 4 * kg]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mfma_f32(a[e], bv[e], acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[4 * kg + i][pass * kTileCands + 16 * w + m] = acc[i] * scale;
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = 4 * w + rr;
      if (r >= rows) continue;
      const int64_t own = (q_pos0 + t0 + r) / bs;
      const int slots = own < top_k - 1 ? (int)own : top_k - 1;
      if (slots == 0) continue;
      uint64_t fresh[kTilePasses];
#pragma unroll
      for (int pass = 0; pass < kTilePasses; ++pass) {
        const int64_t cand = c0 + pass * kTileCands + lane;
        fresh[pass] = cand < own ? make_key(sc[r][pass * kTileCands + lane], (int)cand) : 0ull;
      }
      topset_absorb<kTilePasses>(set[rr], fresh, slots, scratch[w]);
    }
  }
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int r = 4 * w + rr;
    if (r >= rows) continue;
    const int64_t t = t0 + r;
    const int own = (int)((q_pos0 + t) / bs);
    const int slots = own < top_k - 1 ? own : top_k - 1;
    const int64_t off = ((b * q_len + t) * hkv + g) * top_k;
    finalize_row(set[rr].keys, slots, own, top_k, sel + off, sel_scores ? sel_scores + off : nullptr);
  }
}

// ------------------------------------------------------------------ split path

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

template <int D>
__device__ __forceinline__ float dot64_rows(const float* __restrict__ rows_base, int64_t n_valid, const f32x4_t& qv) {
  constexpr int LPR = D / 4;               // lanes covering one key row
  constexpr int RPL = kWave / LPR;         // rows per load instruction
  constexpr int ROWS_PASS = 16 * RPL;      // rows per pass of 16 loads
  constexpr int PASSES = kWave / ROWS_PASS;
  const int lane = lane_id();
  float res[PASSES];
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    f32x4_t raw[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int row = pass * ROWS_PASS + RPL * j + lane / LPR;
      raw[j] = row < n_valid ? *reinterpret_cast<const f32x4_t*>(rows_base + (int64_t)row * D + 4 * (lane % LPR))
                             : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    float vals[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      vals[j] = raw[j][0] * qv[0] + raw[j][1] * qv[1] + raw[j][2] * qv[2] + raw[j][3] * qv[3];
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

template <typename T, int D>
__global__ __launch_bounds__(256) void select_split_kernel(const T* __restrict__ q, const float* __restrict__ k_comp,
                                                           int32_t* __restrict__ sel, float* __restrict__ sel_scores,
                                                           uint64_t* __restrict__ ws, int64_t q_len, int64_t q_pos0,
                                                           int64_t nb_cap, int hq, int hkv, int G, int bs, int top_k,
                                                           float scale, int chunk, int64_t n_chunks) {
  constexpr int LPR = D / 4;
  __shared__ uint64_t lists[4][kWave];

  const int64_t row = blockIdx.x / n_chunks;
  const int64_t ch = blockIdx.x % n_chunks;
  const int64_t b = row / (q_len * hkv);
  const int64_t t = (row / hkv) % q_len;
  const int g = (int)(row % hkv);
  const int lane = lane_id(), w = wave_id(), tid = threadIdx.x;
  const int own = (int)((q_pos0 + t) / bs);
  const int slots = own < top_k - 1 ? own : top_k - 1;

  if (slots == 0) {  // nothing to score: the own block alone
    if (ch == 0 && w == 0) {
      const int64_t off = ((b * q_len + t) * hkv + g) * top_k;
      finalize_row(0ull, 0, own, top_k, sel + off, sel_scores ? sel_scores + off : nullptr);
    }
    return;
  }
  // Each lane sums its own 4 dims of the group's queries: no barrier, so the
  // first compressed-key loads go out together with the query loads.
  const f32x4_t qv = group_sum4(q + ((b * q_len + t) * hq + (int64_t)g * G) * D + 4 * (lane % LPR), G, D);

  const int64_t c_begin = ch * chunk;
  const int64_t c_end = c_begin + chunk < own ? c_begin + chunk : own;
  const float* kc_src = k_comp + ((b * hkv + g) * nb_cap) * D;
  uint64_t cur = 0ull;
  for (int64_t base = c_begin + (int64_t)kWave * w; base < c_end; base += 4 * kWave) {
    const float s = dot64_rows<D>(kc_src + base * D, c_end - base, qv);
    const int64_t cand = base + dot64_row<D>(lane);
    const uint64_t key = cand < c_end ? make_key(s * scale, (int)cand) : 0ull;
    cur = topk_fold(cur, key, slots);
  }
  cur = merge_wave_lists(lists, cur, slots);
  if (w != 0) return;
  if (n_chunks == 1) {
    const int64_t off = ((b * q_len + t) * hkv + g) * top_k;
    finalize_row(cur, slots, own, top_k, sel + off, sel_scores ? sel_scores + off : nullptr);
  } else if (lane < slots) {
    ws[(row * n_chunks + ch) * (top_k - 1) + lane] = cur;
  }
}

// One workgroup per row: reduce the row's chunk lists (each descending) to
// the final top list. The slots-th largest of the chunk maxima is a key that
// at least `slots` real keys reach, so every key below it can be dropped:
// only a short prefix of each list survives (on noise-like scores a few keys
// beyond `slots` in total). Survivors are folded in groups of 64.
constexpr int kMergeCap = 2048;  // survivors kept in LDS; more go straight from memory

__global__ __launch_bounds__(256) void select_merge_kernel(int32_t* __restrict__ sel, float* __restrict__ sel_scores,
                                                           const uint64_t* __restrict__ ws, int64_t q_len,
                                                           int64_t q_pos0, int hkv, int bs, int top_k,
                                                           int64_t n_chunks) {
  __shared__ uint64_t lists[4][kWave];
  __shared__ uint64_t surv[kMergeCap];
  __shared__ uint64_t bound_s;
  __shared__ int n_surv;
  const int64_t row = blockIdx.x;
  const int64_t b = row / (q_len * hkv);
  const int64_t t = (row / hkv) % q_len;
  const int g = (int)(row % hkv);
  const int lane = lane_id(), w = wave_id(), tid = threadIdx.x;
  const int own = (int)((q_pos0 + t) / bs);
  const int slots = own < top_k - 1 ? own : top_k - 1;
  if (slots == 0) return;  // written by the split kernel
  const int sm = top_k - 1;
  const uint64_t* lst = ws + row * n_chunks * sm;

  // bound = slots-th largest chunk maximum (0 when there are fewer chunks)
  if (w == 0) {
    uint64_t cur = 0ull;
    for (int64_t base = 0; base < n_chunks; base += kWave) {
      const uint64_t x = base + lane < n_chunks ? lst[(base + lane) * sm] : 0ull;
      cur = topk_fold(cur, x, slots);
    }
    if (lane == 0) {
      bound_s = n_chunks >= slots ? readlane_u64(cur, slots - 1) : 0ull;
      n_surv = 0;
    }
  }
  __syncthreads();
  const uint64_t bound = bound_s;
  // survivors: the prefix of each list at or above the bound
  for (int64_t c = tid; c < n_chunks; c += 256) {
    for (int j = 0; j < slots; ++j) {
      const uint64_t x = lst[c * sm + j];
      if (x < bound) break;
      const int at = atomicAdd(&n_surv, 1);
      if (at < kMergeCap) surv[at] = x;
    }
  }
  __syncthreads();
  const int total = n_surv;
  uint64_t cur = 0ull;
  if (total <= kMergeCap) {
    for (int base = kWave * w; base < total; base += 4 * kWave) {
      const uint64_t x = base + lane < total ? surv[base + lane] : 0ull;
      cur = topk_fold(cur, x, slots);
    }
  } else {  // adversarial inputs: fold every key at or above the bound from memory
    const int64_t n_keys = n_chunks * sm;
    for (int64_t base = (int64_t)kWave * w; base < n_keys; base += 4 * kWave) {
      const int64_t idx = base + lane;
      uint64_t key = 0ull;
      if (idx < n_keys && (int)(idx % sm) < slots) key = lst[idx];
      cur = topk_fold(cur, key >= bound ? key : 0ull, slots);
    }
  }
  cur = merge_wave_lists(lists, cur, slots);
  if (w != 0) return;
  const int64_t off = ((b * q_len + t) * hkv + g) * top_k;
  finalize_row(cur, slots, own, top_k, sel + off, sel_scores ? sel_scores + off : nullptr);
}

// Merge for rows whose chunk lists hold at most 256 keys in total: one wave
// loads every key at once (4 per lane) and takes the top set directly.
constexpr int kSmallMergeKeys = 4 * kWave;

__global__ __launch_bounds__(64) void select_merge_small_kernel(int32_t* __restrict__ sel,
                                                                float* __restrict__ sel_scores,
                                                                const uint64_t* __restrict__ ws, int64_t q_len,
                                                                int64_t q_pos0, int hkv, int bs, int top_k,
                                                                int64_t n_chunks) {
  __shared__ uint64_t scratch[kWave];
  const int64_t row = blockIdx.x;
  const int64_t b = row / (q_len * hkv);
  const int64_t t = (row / hkv) % q_len;
  const int g = (int)(row % hkv);
  const int lane = lane_id();
  const int own = (int)((q_pos0 + t) / bs);
  const int slots = own < top_k - 1 ? own : top_k - 1;
  if (slots == 0) return;  // written by the split kernel
  const int sm = top_k - 1;
  const uint64_t* lst = ws + row * n_chunks * sm;
  const int n_keys = (int)n_chunks * slots;  // the first `slots` entries of each list
  uint64_t x[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int i = lane + kWave * p;
    x[p] = i < n_keys ? lst[(int64_t)(i / slots) * sm + i % slots] : 0ull;
  }
  TopSet set{0ull, 0, 0ull};
  topset_absorb<4>(set, x, slots, scratch);
  const int64_t off = ((b * q_len + t) * hkv + g) * top_k;
  finalize_row(set.keys, slots, own, top_k, sel + off, sel_scores ? sel_scores + off : nullptr);
}

template <typename T, int D>
hipError_t launch_typed(const Dims& s, const SelectPlan& plan, const void* qv, int64_t q_len, int64_t q_pos0,
                        const float* k_comp, int64_t kv_cap, int32_t* sel, float* sel_scores, void* ws,
                        hipStream_t st) {
  const T* q = static_cast<const T*>(qv);
  const int64_t nb_cap = kv_cap / s.bs;
  if (plan.tiled) {
    dim3 grid((unsigned)((q_len + kTileRows - 1) / kTileRows), (unsigned)s.hkv, (unsigned)s.batch);
    hipLaunchKernelGGL((select_tile_kernel<T, D>), grid, dim3(256), 0, st, q, k_comp, sel, sel_scores, q_len, q_pos0,
                       nb_cap, s.hq, s.hkv, s.group, s.bs, s.top_k, s.scale);
    return hipGetLastError();
  }
  const int64_t rows = (int64_t)s.batch * q_len * s.hkv;
  uint64_t* wsk = static_cast<uint64_t*>(ws);
  hipLaunchKernelGGL((select_split_kernel<T, D>), dim3((unsigned)(rows * plan.n_chunks)), dim3(256), 0, st, q,
                     k_comp, sel, sel_scores, wsk, q_len, q_pos0, nb_cap, s.hq, s.hkv, s.group, s.bs, s.top_k,
                     s.scale, plan.chunk, plan.n_chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.n_chunks == 1) return e;
  if (plan.n_chunks * (s.top_k - 1) <= kSmallMergeKeys)
    hipLaunchKernelGGL(select_merge_small_kernel, dim3((unsigned)rows), dim3(64), 0, st, sel, sel_scores, wsk, q_len,
                       q_pos0, s.hkv, s.bs, s.top_k, plan.n_chunks);
  else
    hipLaunchKernelGGL(select_merge_kernel, dim3((unsigned)rows), dim3(256), 0, st, sel, sel_scores, wsk, q_len,
                       q_pos0, s.hkv, s.bs, s.top_k, plan.n_chunks);
  return hipGetLastError();
}

}  // namespace

SelectPlan plan_select(const Dims& s, int64_t q_len, int64_t q_pos0) {
  SelectPlan p{};
  const int64_t kv_len = q_pos0 + q_len;
  const int64_t max_cand = (kv_len - 1) / s.bs;  // candidates of the last row
  p.tiled = q_len >= kTileRows;
  p.chunk = 256;
  p.n_chunks = 1;
  p.ws_bytes = 0;
  if (p.tiled || max_cand <= 0) return p;
  const int64_t rows = (int64_t)s.batch * q_len * s.hkv;
  if (rows * max_cand <= 8192 && max_cand <= 2048) {
    // small problem: one workgroup per row, no merge launch
    p.chunk = (int)((max_cand + 255) / 256 * 256);
  } else {
    // 4 waves x 64 keys x u per workgroup; the largest u that still spreads
    // the scan over >= 512 workgroups (two per CU)
    int u = 8;
    while (u > 1 && rows * ((max_cand + 256 * u - 1) / (256 * u)) < 512) u /= 2;
    p.chunk = 256 * u;
  }
  p.n_chunks = (max_cand + p.chunk - 1) / p.chunk;
  if (p.n_chunks > 1) p.ws_bytes = (size_t)rows * p.n_chunks * (s.top_k - 1) * sizeof(uint64_t);
  return p;
}

hipError_t launch_select(const Dims& s, const SelectPlan& plan, const void* q, int64_t q_len, int64_t q_pos0,
                         const float* k_comp, int64_t kv_cap, int32_t* sel, float* sel_scores, void* ws,
                         hipStream_t st) {
  if (s.dtype == 1)
    return s.d == 64 ? launch_typed<uint16_t, 64>(s, plan, q, q_len, q_pos0, k_comp, kv_cap, sel, sel_scores, ws, st)
                     : launch_typed<uint16_t, 128>(s, plan, q, q_len, q_pos0, k_comp, kv_cap, sel, sel_scores, ws, st);
  return s.d == 64 ? launch_typed<float, 64>(s, plan, q, q_len, q_pos0, k_comp, kv_cap, sel, sel_scores, ws, st)
                   : launch_typed<float, 128>(s, plan, q, q_len, q_pos0, k_comp, kv_cap, sel, sel_scores, ws, st);
}

}  // namespace qsa
