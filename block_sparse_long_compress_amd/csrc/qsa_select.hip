// Indexer scoring and top-k block selection ("Qwen4 in llama.cpp: Dissecting
// PR #27742", section "QSA Is an Address-Selection Problem, Not a New
// Attention Equation": compressed blocks are scored, the top-k kept and
// turned into cache addresses).
//
// Score of candidate c for (token, KV head g): scale * <qbar, kc[c]> with
// qbar the float32 sum of the group's G query heads (equal to the sum of the
// per-head scores). A row's frame gives its candidates and its forced block:
// by default the complete blocks before the own block i = p / Bs, with block
// i forced; in the keep-tail frame (the released budget of the same page,
// visible width bounded by budget + ratio - 1) all (p+1)/Bs complete blocks,
// with the block of the positions past them forced when there are such
// positions. Selection keeps the forced block plus the min(k-1, n_cand) best
// candidates, ranked by the 64-bit key of qsa_device.h (score descending, id
// ascending), and writes ids ascending.
//
// Four paths:
//  * row path (many query rows, top_k <= 16: prefill): a workgroup takes 64
//    consecutive rows of one (b, g), which share the candidate prefix.
//    Rounds of 128 compressed keys are staged in LDS and scored with fp32
//    MFMA (16x16x4, full fp32 products) against the group-summed queries held
//    in registers; the product layout leaves each lane 16 scores of one row,
//    which it sorts in registers (bitonic network) and merges into its own
//    running top-16 list. At the end the lists of a row (4 lanes, 2 waves)
//    merge pairwise and each lane writes a quarter of the row's selection.
//  * tile path (many query rows, larger top_k): a workgroup takes 16
//    consecutive rows of one (b, g). Candidate chunks of 64 compressed keys
//    are staged in LDS and scored with fp32 MFMA as above; every 128
//    candidates each wave updates four rows' running top sets by threshold
//    selection (the m-th largest key found bit by bit with ballot counts, no
//    sorting), and the final set is sorted by id once.
//  * split path (few rows, decode): the candidates of a row are cut into
//    chunks spread over the whole GPU. Each wave streams 64 compressed keys
//    per step with fully coalesced 16-byte loads (1 KiB per instruction),
//    finishes the dot products with a transpose-reduce butterfly, and keeps a
//    running top list; the chunk's list goes to the workspace with
//    device-coherent stores, and the last workgroup of the row to finish
//    (an arrival counter per row) reduces the lists, skipping every key below
//    the best chunk-local cutoff (a valid lower bound of the row's cutoff);
//    when all the lists of a row hold at most 256 keys, one wave takes them
//    at once.
//  * large path (k > 64, the released budget of 512 blocks): a score pass
//    (per row, or, for 16 or more query rows, per tile of 16 rows sharing a
//    chunk's compressed keys) writes every candidate's score and, per chunk
//    of 256 candidates, the chunk's 16 best keys in order; one workgroup per
//    row then finds the cutoff by radix selection over the union of those
//    lists, re-expands the few chunks whose 16th key still reaches the cutoff
//    (only they can hide more kept keys), and emits the kept ids in ascending
//    order straight from an LDS bitmap of the candidates.
#include "qsa_device.h"
#include "qsa_internal.h"
#include "qsa_select_large.h"
#include "qsa_select_wave.h"

namespace qsa {
namespace {

// ------------------------------------------------------------------ tile path

constexpr int kTileRows = 16;
constexpr int kTileCands = 64;   // candidates staged and scored per pass
constexpr int kTilePasses = 2;   // passes per selection step (128 candidates, 2 per lane)

template <typename T, int D>
__global__ __launch_bounds__(256) void select_tile_kernel(const T* __restrict__ q, const float* __restrict__ k_comp,
                                                          int32_t* __restrict__ sel, float* __restrict__ sel_scores,
                                                          int64_t q_len, int64_t q_pos0, int64_t nb_cap, int hq,
                                                          int hkv, int G, int bs, int top_k, float scale,
                                                          int keep_tail) {
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

  // candidates of every row are below the last row's candidate count
  const int64_t cand_end = row_frame(q_pos0 + t0 + rows - 1, bs, keep_tail).n_cand;
  const float* kc_src = k_comp + ((b * hkv + g) * nb_cap) * D;
  TopSet set[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) set[rr] = TopSet{0ull, 0, 0ull};

  for (int64_t c0 = 0; c0 < cand_end; c0 += SPAN) {
    // score SPAN candidates for all 16 rows, one staged pass of 64 at a time
#pragma unroll
    for (int pass = 0; pass < kTilePasses; ++pass) {
      const int64_t p0 = c0 + pass * kTileCands;
      __syncthreads();  // kc (and sc) of the previous pass fully consumed
      for (int idx = tid; idx < kTileCands * D / 4; idx += 256) {
        const int r = idx / (D / 4), e4 = (idx % (D / 4)) * 4;
        f32x4_t v = {0.f, 0.f, 0.f, 0.f};
        if (p0 + r < cand_end) v = *reinterpret_cast<const f32x4_t*>(kc_src + (p0 + r) * D + e4);
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
      const Frame fr = row_frame(q_pos0 + t0 + r, bs, keep_tail);
      const int slots = frame_slots(fr, top_k);
      if (slots == 0) continue;
      uint64_t fresh[kTilePasses];
#pragma unroll
      for (int pass = 0; pass < kTilePasses; ++pass) {
        const int64_t cand = c0 + pass * kTileCands + lane;
        fresh[pass] = cand < fr.n_cand ? make_key(sc[r][pass * kTileCands + lane], (int)cand) : 0ull;
      }
      topset_absorb<kTilePasses>(set[rr], fresh, slots, scratch[w]);
    }
  }
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int r = 4 * w + rr;
    if (r >= rows) continue;
    const int64_t t = t0 + r;
    const Frame fr = row_frame(q_pos0 + t, bs, keep_tail);
    const int64_t off = ((b * q_len + t) * hkv + g) * top_k;
    finalize_row(set[rr].keys, frame_slots(fr, top_k), fr.forced, top_k, sel + off,
                 sel_scores ? sel_scores + off : nullptr);
  }
}

// ------------------------------------------------------------------ row path

constexpr int kRowsPerWg = 64;  // 4 groups of 16 query rows, two waves per group
constexpr int kRowKeep = 16;    // keys a lane keeps (the path serves top_k <= 16)
constexpr int kRowRound = 128;  // candidates staged per round: 64 for each wave of a group

template <int D>
constexpr int rows_lds_bytes() {
  return (kRowsPerWg + kRowRound) * (D + 4) * (int)sizeof(float);
}

// Compare-exchange that leaves the larger key in a.
__device__ __forceinline__ void cx_desc(uint64_t& a, uint64_t& b) {
  const bool swap = b > a;
  const uint64_t hi = swap ? b : a;
  const uint64_t lo = swap ? a : b;
  a = hi;
  b = lo;
}

// Bitonic sort of N keys held in registers, descending.
template <int N>
__device__ __forceinline__ void sort_desc(uint64_t (&x)[N]) {
#pragma unroll
  for (int k = 2; k <= N; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int l = i ^ j;
        if (l > i) {
          if ((i & k) == 0) cx_desc(x[i], x[l]);
          else cx_desc(x[l], x[i]);
        }
      }
}

// a := the N largest of two descending lists a and b, descending. The
// elementwise maximum of a and reversed b holds them and is bitonic, so one
// bitonic merge sorts it.
template <int N>
__device__ __forceinline__ void merge_top_desc(uint64_t (&a)[N], const uint64_t (&b)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) a[i] = a[i] > b[N - 1 - i] ? a[i] : b[N - 1 - i];
#pragma unroll
  for (int j = N >> 1; j > 0; j >>= 1)
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int l = i ^ j;
      if (l > i) cx_desc(a[i], a[l]);
    }
}

template <typename T, int D>
__global__ __launch_bounds__(512) void select_rows_kernel(const T* __restrict__ q, const float* __restrict__ k_comp,
                                                          int32_t* __restrict__ sel, float* __restrict__ sel_scores,
                                                          int64_t q_len, int64_t q_pos0, int64_t nb_cap, int hq,
                                                          int hkv, int G, int bs, int top_k, float scale,
                                                          int keep_tail) {
  constexpr int QP = D + 4;  // padded row stride (floats): conflict-free 16-byte reads
  extern __shared__ __align__(16) unsigned char smem[];
  float(*qbar)[QP] = reinterpret_cast<float(*)[QP]>(smem);
  float(*kc)[QP] = reinterpret_cast<float(*)[QP]>(smem + kRowsPerWg * QP * sizeof(float));
  // after the last round the staging area carries the second waves' lists
  uint64_t(*xl)[kRowKeep] = reinterpret_cast<uint64_t(*)[kRowKeep]>(smem + kRowsPerWg * QP * sizeof(float));

  const int64_t t0 = (int64_t)blockIdx.x * kRowsPerWg;
  const int g = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int rg = w & 3, half = w >> 2;  // row group, half of each round's candidates
  const int m = lane & 15, kg = lane >> 4;
  const int rows = (int)(q_len - t0 < kRowsPerWg ? q_len - t0 : kRowsPerWg);

  // Group-summed queries: a thread's 16-byte chunks (up to two at a time,
  // every head's load issued before the first add), summed in head order.
  {
    constexpr int EPL = 16 / (int)sizeof(T);  // elements per chunk
    constexpr int CPR = D / EPL;              // chunks per row
    constexpr int NCH = kRowsPerWg * CPR / 512;
    constexpr int NB = NCH < 2 ? NCH : 2;
#pragma unroll
    for (int c0 = 0; c0 < NCH; c0 += NB) {
      u32x4_t raw[NB][16];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int idx = tid + 512 * (c0 + i);
        const int r = idx / CPR, e = (idx % CPR) * EPL;
        const T* src = q + ((b * q_len + t0 + r) * hq + (int64_t)g * G) * D + e;
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (j < G && r < rows) raw[i][j] = *reinterpret_cast<const u32x4_t*>(src + (int64_t)j * D);
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int idx = tid + 512 * (c0 + i);
        const int r = idx / CPR, e = (idx % CPR) * EPL;
        float acc[EPL];
#pragma unroll
        for (int x = 0; x < EPL; ++x) acc[x] = 0.f;
        if (r < rows) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            if (j < G) {
#pragma unroll
              for (int x = 0; x < 4; ++x) {
                if constexpr (EPL == 8) {
                  acc[2 * x] += bf16_lo(raw[i][j][x]);
                  acc[2 * x + 1] += bf16_hi(raw[i][j][x]);
                } else {
                  acc[x] += __uint_as_float(raw[i][j][x]);
                }
              }
            }
          }
        }
#pragma unroll
        for (int x = 0; x < EPL; x += 4)
          *reinterpret_cast<f32x4_t*>(&qbar[r][e + x]) = f32x4_t{acc[x], acc[x + 1], acc[x + 2], acc[x + 3]};
      }
    }
  }
  // candidates of every row are below the last row's candidate count
  const int64_t cand_end = row_frame(q_pos0 + t0 + rows - 1, bs, keep_tail).n_cand;
  const int r = 16 * rg + m;  // this lane's row
  const bool row_ok = r < rows;
  const Frame fr = row_frame(q_pos0 + t0 + (row_ok ? r : 0), bs, keep_tail);
  const int64_t n_cand = row_ok ? fr.n_cand : 0;
  const float* kc_src = k_comp + ((b * hkv + g) * nb_cap) * D;

  uint64_t top[kRowKeep];
#pragma unroll
  for (int i = 0; i < kRowKeep; ++i) top[i] = 0ull;
  float qr[D / 4];  // the row's query sum, dims 16u + 4kg + e at qr[4u + e]
  for (int64_t c0 = 0; c0 < cand_end; c0 += kRowRound) {
    if (c0 > 0) __syncthreads();  // the previous round's keys fully read
    {
      constexpr int NK = kRowRound * D / 4 / 512;  // 16-byte chunks per thread, all loads first
      f32x4_t v[NK];
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const int idx = tid + 512 * i;
        const int c = idx / (D / 4), e4 = (idx % (D / 4)) * 4;
        v[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (c0 + c < cand_end) v[i] = *reinterpret_cast<const f32x4_t*>(kc_src + (c0 + c) * D + e4);
      }
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const int idx = tid + 512 * i;
        *reinterpret_cast<f32x4_t*>(&kc[idx / (D / 4)][(idx % (D / 4)) * 4]) = v[i];
      }
    }
    __syncthreads();
    if (c0 == 0) {
#pragma unroll
      for (int u = 0; u < D / 16; ++u) {
        const f32x4_t a = *reinterpret_cast<const f32x4_t*>(&qbar[r][16 * u + 4 * kg]);
#pragma unroll
        for (int e = 0; e < 4; ++e) qr[4 * u + e] = a[e];
      }
    }
    // scores of candidates c0 + 64 half + 16 ct + 4 kg + v for this lane's row
    // (keys as operand A, queries as operand B: output column = query row)
    uint64_t x[kRowKeep];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < D / 16; ++u) {
        const f32x4_t a = *reinterpret_cast<const f32x4_t*>(&kc[64 * half + 16 * ct + m][16 * u + 4 * kg]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mfma_f32(a[e], qr[4 * u + e], acc);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t cand = c0 + 64 * half + 16 * ct + 4 * kg + v;
        x[4 * ct + v] = cand < n_cand ? make_key(acc[v] * scale, (int)cand) : 0ull;
      }
    }
    sort_desc<kRowKeep>(x);
    merge_top_desc<kRowKeep>(top, x);
  }
  // the row's four lanes, then its two waves, to one list
#pragma unroll
  for (int j = 16; j <= 32; j <<= 1) {
    uint64_t o[kRowKeep];
#pragma unroll
    for (int i = 0; i < kRowKeep; ++i) o[i] = xor_lane_u64(top[i], j);
    merge_top_desc<kRowKeep>(top, o);
  }
  __syncthreads();  // every wave is done with the staging area
  if (half == 1 && kg == 0) {
#pragma unroll
    for (int i = 0; i < kRowKeep; ++i) xl[r][i] = top[i];
  }
  __syncthreads();
  if (half == 1 || !row_ok) return;
  {
    uint64_t o[kRowKeep];
#pragma unroll
    for (int i = 0; i < kRowKeep; ++i) o[i] = xl[r][i];
    merge_top_desc<kRowKeep>(top, o);
  }

  // Selection in ascending id order: entry i < slots is kept key i, entry
  // slots the forced block; lane kg places entries 4kg .. 4kg+3 at their
  // rank among the ids and pads positions past the real entries with -1.
  const int slots = frame_slots(fr, top_k);
  const int n_real = slots + (fr.forced >= 0 ? 1 : 0);
  int ids[kRowKeep];
#pragma unroll
  for (int i = 0; i < kRowKeep; ++i)
    ids[i] = i < slots ? key_id(top[i]) : ((i == slots && fr.forced >= 0) ? fr.forced : 0x7FFFFFFF);
  const int64_t off = ((b * q_len + t0 + r) * hkv + g) * top_k;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int j = 4 * kg + v;
    uint64_t key_j = 0ull;
    int id_j = 0x7FFFFFFF;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (kg == c) {
        key_j = top[4 * c + v];
        id_j = ids[4 * c + v];
      }
    }
    const float sc_j = j < slots ? key_score(key_j) : __builtin_inff();
    if (j < n_real) {
      int rank = 0;
#pragma unroll
      for (int i = 0; i < kRowKeep; ++i) rank += ids[i] < id_j ? 1 : 0;
      sel[off + rank] = id_j;
      if (sel_scores) sel_scores[off + rank] = sc_j;
    } else if (j < top_k) {
      sel[off + j] = -1;
      if (sel_scores) sel_scores[off + j] = -__builtin_inff();
    }
  }
}

// ------------------------------------------------------------------ split path

constexpr int kMergeCap = 2048;              // survivors kept in LDS; more go straight from memory
constexpr int kSmallMergeKeys = 4 * kWave;   // lists this small are merged by one wave at once

struct SplitSmem {
  uint64_t lists[4][kWave];
  uint64_t surv[kMergeCap];
  uint64_t bound;
  int n_surv;
  int last_wg;
};

// Key i of a row's chunk lists in the workspace (device-coherent read; the
// lists were written by other workgroups of the same kernel).
__device__ __forceinline__ uint64_t list_key(__amdgpu_buffer_rsrc_t rs, int64_t i) {
  const u32x2_t v = load2_coherent(rs, (int)(2 * i));
  return ((uint64_t)v[1] << 32) | v[0];
}

// Merge of lists that hold at most 256 keys in all (the first `slots`
// entries of each of the n_chunks lists, stride sm): wave 0 loads every key
// at once (4 per lane) and takes the top set directly.
__device__ void merge_lists_small(__amdgpu_buffer_rsrc_t rs, int64_t n_chunks, int sm, int slots, int forced,
                                  int top_k, uint64_t* scratch, int32_t* sel_row, float* score_row) {
  const int lane = lane_id();
  const int n_keys = (int)n_chunks * slots;
  uint64_t x[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int i = lane + kWave * p;
    x[p] = i < n_keys ? list_key(rs, (int64_t)(i / slots) * sm + i % slots) : 0ull;
  }
  TopSet set{0ull, 0, 0ull};
  topset_absorb<4>(set, x, slots, scratch);
  finalize_row(set.keys, slots, forced, top_k, sel_row, score_row);
}

// Merge of a row's chunk lists (each descending) by one workgroup. The
// slots-th largest of the chunk maxima is a key that at least `slots` real
// keys reach, so every key below it can be dropped: only a short prefix of
// each list survives (on noise-like scores a few keys beyond `slots` in
// total). Survivors are folded in groups of 64.
__device__ void merge_lists(__amdgpu_buffer_rsrc_t rs, int64_t n_chunks, int sm, int slots, int forced, int top_k,
                            SplitSmem& smem, int32_t* sel_row, float* score_row) {
  const int lane = lane_id(), w = wave_id(), tid = threadIdx.x;
  // The first 4 entries of this thread's first chunk list load together with
  // the chunk maxima below (survivors rarely go deeper on noise-like scores).
  constexpr int kPre = 4;
  uint64_t pre[kPre];
#pragma unroll
  for (int j = 0; j < kPre; ++j) pre[j] = (tid < n_chunks && j < slots) ? list_key(rs, (int64_t)tid * sm + j) : 0ull;
  // bound = slots-th largest chunk maximum (0 when there are fewer chunks)
  if (w == 0) {
    uint64_t cur = 0ull;
    for (int64_t base = 0; base < n_chunks; base += kWave) {
      const uint64_t x = base + lane < n_chunks ? list_key(rs, (base + lane) * sm) : 0ull;
      cur = topk_fold(cur, x, slots);
    }
    if (lane == 0) {
      smem.bound = n_chunks >= slots ? readlane_u64(cur, slots - 1) : 0ull;
      smem.n_surv = 0;
    }
  }
  __syncthreads();
  const uint64_t bound = smem.bound;
  // survivors: the prefix of each list at or above the bound, read in groups
  // of 4 independent loads
  for (int64_t c = tid; c < n_chunks; c += 256) {
    for (int j0 = 0; j0 < slots; j0 += kPre) {
      uint64_t x[kPre];
#pragma unroll
      for (int j = 0; j < kPre; ++j)
        x[j] = (c == tid && j0 == 0) ? pre[j] : (j0 + j < slots ? list_key(rs, c * sm + j0 + j) : 0ull);
      bool more = true;
#pragma unroll
      for (int j = 0; j < kPre; ++j) {
        if (more && j0 + j < slots && x[j] >= bound) {
          const int at = atomicAdd(&smem.n_surv, 1);
          if (at < kMergeCap) smem.surv[at] = x[j];
        } else {
          more = false;
        }
      }
      if (!more) break;
    }
  }
  __syncthreads();
  const int total = smem.n_surv;
  uint64_t cur = 0ull;
  if (total <= kMergeCap) {
    for (int base = kWave * w; base < total; base += 4 * kWave) {
      const uint64_t x = base + lane < total ? smem.surv[base + lane] : 0ull;
      cur = topk_fold(cur, x, slots);
    }
  } else {  // adversarial inputs: fold every key at or above the bound from memory
    const int64_t n_keys = n_chunks * sm;
    for (int64_t base = (int64_t)kWave * w; base < n_keys; base += 4 * kWave) {
      const int64_t idx = base + lane;
      uint64_t key = 0ull;
      if (idx < n_keys && (int)(idx % sm) < slots) key = list_key(rs, idx);
      cur = topk_fold(cur, key >= bound ? key : 0ull, slots);
    }
  }
  cur = merge_wave_lists(smem.lists, cur, slots);
  if (w == 0) finalize_row(cur, slots, forced, top_k, sel_row, score_row);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void select_split_kernel(const T* __restrict__ q, const float* k_comp,
                                                           const T* __restrict__ k_cache, float* k_comp_w, int64_t kv_cap,
                                                           int32_t* __restrict__ sel, float* __restrict__ sel_scores,
                                                           uint32_t* __restrict__ counters, uint64_t* __restrict__ ws,
                                                           int64_t q_len, int64_t q_pos0, int64_t nb_cap, int hq,
                                                           int hkv, int G, int bs, int top_k, float scale,
                                                           int keep_tail, int chunk, int64_t n_chunks,
                                                           int64_t close_block) {
  constexpr int LPR = D / 4;
  __shared__ SplitSmem smem;

  const int64_t row = blockIdx.x / n_chunks;
  const int64_t ch = blockIdx.x % n_chunks;
  const int64_t b = row / (q_len * hkv);
  const int64_t t = (row / hkv) % q_len;
  const int g = (int)(row % hkv);
  const int lane = lane_id(), w = wave_id(), tid = threadIdx.x;
  const Frame fr = row_frame(q_pos0 + t, bs, keep_tail);
  const int slots = frame_slots(fr, top_k);
  const int64_t off = ((b * q_len + t) * hkv + g) * top_k;
  int32_t* sel_row = sel + off;
  float* score_row = sel_scores ? sel_scores + off : nullptr;
  // A decode step's closed block: with keep_tail it is this row's last
  // candidate, compressed by the last chunk before it scores; in the default
  // frame it is the token's own block, never a candidate, and the first
  // workgroup of the row to post its list stores it (below), off the path
  // to the merge.
  auto compress_closed = [&]() {
    compress_block_wave<T, D>(k_cache + ((b * hkv + g) * kv_cap + close_block * bs) * D, bs,
                              k_comp_w + ((b * hkv + g) * nb_cap + close_block) * D, nullptr);
  };
  const bool close_first = close_block >= 0 && keep_tail;
  if (close_first && ch == n_chunks - 1) {
    if (w == 0) compress_closed();
    __syncthreads();
  }

  if (slots == 0) {  // nothing to score: the forced block alone
    if (ch == 0 && w == 0) {
      finalize_row(0ull, 0, fr.forced, top_k, sel_row, score_row);
      if (close_block >= 0 && !close_first) compress_closed();
    }
    return;
  }
  // Each lane sums its own 4 dims of the group's queries: no barrier, so the
  // first compressed-key loads go out together with the query loads.
  const f32x4_t qv = group_sum4(q + ((b * q_len + t) * hq + (int64_t)g * G) * D + 4 * (lane % LPR), G, D);

  const int64_t c_begin = ch * chunk;
  const int64_t c_end = c_begin + chunk < fr.n_cand ? c_begin + chunk : fr.n_cand;
  const float* kc_src = k_comp + ((b * hkv + g) * nb_cap) * D;
  uint64_t cur = 0ull;
  for (int64_t base = c_begin + (int64_t)kWave * w; base < c_end; base += 4 * kWave) {
    const float s = dot64_rows<D, true>(kc_src + base * D, c_end - base, qv);
    const int64_t cand = base + dot64_row<D>(lane);
    const uint64_t key = cand < c_end ? make_key(s * scale, (int)cand) : 0ull;
    cur = topk_fold(cur, key, slots);
  }
  cur = merge_wave_lists(smem.lists, cur, slots);
  if (n_chunks == 1) {
    if (w == 0) {
      finalize_row(cur, slots, fr.forced, top_k, sel_row, score_row);
      if (close_block >= 0 && !close_first) compress_closed();
    }
    return;
  }
  // Several chunks per row: the chunk's list goes out with device-coherent
  // stores, then one ticket per workgroup; the last workgroup of the row to
  // arrive merges the lists and resets the row's counter.
  const int sm = top_k - 1;
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(ws + row * n_chunks * sm, 0, (int)(n_chunks * sm * 8),
                                                    kBufferFlags);
  if (w == 0 && lane < slots) store2_coherent(rs, (int)(2 * (ch * sm + lane)), (uint32_t)cur, (uint32_t)(cur >> 32));
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counters + row, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev == (uint32_t)(n_chunks - 1);
    if (last) __hip_atomic_store(counters + row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    smem.last_wg = last ? 1 : (prev == 0u ? 2 : 0);  // 2: the first to arrive (never the last: n_chunks > 1)
  }
  __syncthreads();
  if (smem.last_wg != 1) {
    if (smem.last_wg == 2 && w == 0 && close_block >= 0 && !close_first) compress_closed();
    return;
  }
  if (n_chunks * slots <= kSmallMergeKeys) {
    if (w == 0) merge_lists_small(rs, n_chunks, sm, slots, fr.forced, top_k, smem.lists[0], sel_row, score_row);
  } else {
    merge_lists(rs, n_chunks, sm, slots, fr.forced, top_k, smem, sel_row, score_row);
  }
}

// ------------------------------------------------------------------ large path
// (constants, the radix cutoff and pick_row: qsa_select_large.h)


// Score pass: one workgroup per (row, chunk of 256 candidates). Writes the
// order image of every candidate's score (ws_scores, row stride n_chunks*256)
// and, for rows with more candidates than the pick kernel holds at once, the
// chunk's 16 best keys in descending order (ws_lists, 0 = empty).
template <typename T, int D>
__global__ __launch_bounds__(256) void select_large_score_kernel(
    const T* __restrict__ q, const float* k_comp, uint32_t* __restrict__ ws_scores,
    uint64_t* __restrict__ ws_lists, int64_t q_len, int64_t q_pos0, int64_t nb_cap, int hq, int hkv, int G, int bs,
    float scale, int keep_tail, int64_t n_chunks, const T* __restrict__ k_cache, float* k_comp_w, int64_t kv_cap,
    int64_t close_block, const int32_t* __restrict__ kv_lens) {
  constexpr int LPR = D / 4;
  __shared__ uint64_t tops[4][kLargeList];
  const int64_t row = blockIdx.x / n_chunks;
  const int64_t ch = blockIdx.x % n_chunks;
  const int64_t b = row / (q_len * hkv);
  const int64_t t = (row / hkv) % q_len;
  const int g = (int)(row % hkv);
  const int lane = lane_id(), w = wave_id();
  int64_t p = q_pos0 + t;
  if (kv_lens) {
    // a ragged decode batch (q_len = 1): sequence b's own length, clamped
    // into [1, q_pos0 + 1], and the block its new token closes, if any
    int64_t n = kv_lens[b];
    n = n < 1 ? 1 : (n > q_pos0 + 1 ? q_pos0 + 1 : n);
    p = n - 1;
    // the block its token closes, compressed when the keys are given (the
    // decode step); the selection call alone reads k_comp as it stands
    close_block = k_cache && n % bs == 0 ? n / bs - 1 : -1;
  }
  const int n_cand = row_frame(p, bs, keep_tail).n_cand;
  const int64_t c_begin = ch * kLargeChunk;
  const int64_t last_ch = n_cand > 0 ? (n_cand - 1) / kLargeChunk : 0;
  if (close_block >= 0 && ch == last_ch) {
    // a decode step's closed block, compressed before it is scored (with
    // keep_tail it is this chunk's last candidate)
    if (w == 0)
      compress_block_wave<T, D>(k_cache + ((b * hkv + g) * kv_cap + close_block * bs) * D, bs,
                                k_comp_w + ((b * hkv + g) * nb_cap + close_block) * D, nullptr);
    __syncthreads();
  }
  if (c_begin >= n_cand) return;  // uniform over the workgroup

  const f32x4_t qv = group_sum4(q + ((b * q_len + t) * hq + (int64_t)g * G) * D + 4 * (lane % LPR), G, D);
  const int64_t base = c_begin + (int64_t)kWave * w;
  uint64_t key = 0ull;
  if (base < n_cand) {
    const float sc = dot64_rows<D, true>(k_comp + ((b * hkv + g) * nb_cap + base) * D, n_cand - base, qv);
    const int64_t cand = base + dot64_row<D>(lane);
    if (cand < n_cand) {
      key = make_key(sc * scale, (int)cand);
      ws_scores[row * n_chunks * kLargeChunk + cand] = (uint32_t)(key >> 32);
    }
  }
  if (n_cand <= kPoolCap) return;  // the pick kernel takes every score directly
  key = wave_sort_desc(key);
  if (lane < kLargeList) tops[w][lane] = key;
  __syncthreads();
  if (w == 0) {
    uint64_t x = tops[lane / kLargeList][lane % kLargeList];
    x = wave_sort_desc(x);
    if (lane < kLargeList) ws_lists[(row * n_chunks + ch) * kLargeList + lane] = x;
  }
}

// The score pass for many query rows (prefill): a workgroup takes a tile of
// 32 consecutive rows of one (b, g) and one chunk of 256 candidates, which
// the rows share (k_comp is read once per tile instead of once per row).
// Scores come from fp32 MFMA as in the tile path; wave w scores candidates
// 16w .. 16w + 15 of each pass of 64 for both 16-row halves of the tile (one
// load of their compressed keys feeds two products), and as no other wave
// needs them it loads those keys straight into its operand registers, two
// passes ahead. Outputs are those of the per-row pass:
// every score of every row, and per (row, chunk) the chunk's 16 best keys in
// descending order when the row's candidates exceed the pick pool.
// Workgroups go to the 8 XCDs round-robin; the grid is laid out so that
// every (sequence, KV head, chunk) goes to one XCD (XCD x takes the chunks
// x, x + 8, ... of the flattened (sequence, KV head, chunk) order) and its
// tiles are dispatched there one after another: they run together and read
// the chunk's compressed keys from that XCD's L2, which fetches them once.
constexpr int kLargeTileRows = 32;

// Grid of select_large_tile_kernel: 8 XCD lanes of ceil(n_bg * n_chunks / 8)
// chunks of n_tiles workgroups each.
inline int64_t large_tile_grid(int64_t n_bg, int64_t n_chunks, int64_t n_tiles) {
  return 8 * n_tiles * ((n_bg * n_chunks + 7) / 8);
}

template <typename T, int D>
__global__ __launch_bounds__(256, 3) void select_large_tile_kernel(
    const T* __restrict__ q, const float* __restrict__ k_comp, uint32_t* __restrict__ ws_scores,
    uint64_t* __restrict__ ws_lists, int64_t q_len, int64_t q_pos0, int64_t nb_cap, int hq, int hkv, int G, int bs,
    float scale, int keep_tail, int64_t n_chunks, int64_t n_tiles, int64_t n_bg) {
  constexpr int TR = kLargeTileRows;
  constexpr int QP = D + 4;  // padded row strides (floats): conflict-free 16-byte reads
  constexpr int PASSES = kLargeChunk / kTileCands;
  constexpr int DU = D / 16;  // 16-byte operand loads per lane and pass
  __shared__ float qbar[TR][QP];
  __shared__ uint32_t sc[TR][kLargeChunk + 4];  // order images of the scaled scores
  __shared__ int ncand[TR];  // candidates of each row of the tile
  __shared__ uint64_t gather[4][kWave];  // each wave's scratch for its chunk lists
  static_assert(kLargeChunk == 256, "one thread per candidate of the chunk");

  const int64_t xcd = blockIdx.x % 8, j = blockIdx.x / 8;
  const int64_t tile = j % n_tiles;
  const int64_t gc = xcd + 8 * (j / n_tiles);  // flattened (sequence, KV head, chunk)
  if (gc >= n_bg * n_chunks) return;           // spare slots of the last round
  const int64_t ch = gc % n_chunks;
  const int64_t bg = gc / n_chunks;
  const int64_t b = bg / hkv;
  const int g = (int)(bg % hkv);
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int64_t t0 = tile * TR;
  const int rows = (int)(q_len - t0 < TR ? q_len - t0 : TR);
  const int64_t c_begin = ch * kLargeChunk;
  // the tile's last row has the most candidates
  const int64_t cand_end = row_frame(q_pos0 + t0 + rows - 1, bs, keep_tail).n_cand;
  if (c_begin >= cand_end) return;  // uniform over the workgroup
  if (tid < TR) ncand[tid] = tid < rows ? row_frame(q_pos0 + t0 + tid, bs, keep_tail).n_cand : 0;

  const float* kc_src = k_comp + (bg * nb_cap) * D;
  const int m = lane % 16, kg = lane / 16;
  // B operands of pass p: candidate c_begin + 64p + 16w + m, dims 16u + 4kg .. + 3
  // (candidates past the tile's last reach are read as zero)
  auto load_pass = [&](int pass, f32x4_t (&kb)[DU]) {
    const int64_t cand = c_begin + pass * kTileCands + 16 * w + m;
#pragma unroll
    for (int u = 0; u < DU; ++u)
      kb[u] = cand < cand_end ? *reinterpret_cast<const f32x4_t*>(kc_src + cand * D + 16 * u + 4 * kg)
                              : f32x4_t{0.f, 0.f, 0.f, 0.f};
  };
  {
    // the tile's group-summed queries: thread tid sums dims e4 .. e4 + 3 of
    // rows r0 + RS * i (rows past the tile's end read its last row and store
    // zeros), all rows' loads issued before the first add (with the first
    // passes' keys also in flight the kernel would need 232 registers)
    constexpr int NR = TR * D / 4 / 256, RS = 256 / (D / 4);
    const int e4 = (tid % (D / 4)) * 4, r0 = tid / (D / 4);
    const T* p[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int r = r0 + RS * i < rows ? r0 + RS * i : rows - 1;
      p[i] = q + ((b * q_len + t0 + r) * hq + (int64_t)g * G) * D + e4;
    }
    f32x4_t v[NR];
    switch (G) {
      case 1: group_sum4_rows<1, NR>(p, D, v); break;
      case 2: group_sum4_rows<2, NR>(p, D, v); break;
      case 4: group_sum4_rows<4, NR>(p, D, v); break;
      case 8: group_sum4_rows<8, NR>(p, D, v); break;
      default:
#pragma unroll
        for (int i = 0; i < NR; ++i) v[i] = group_sum4_n<16>(p[i], D);
    }
#pragma unroll
    for (int i = 0; i < NR; ++i)
      *reinterpret_cast<f32x4_t*>(&qbar[r0 + RS * i][e4]) =
          r0 + RS * i < rows ? v[i] : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  f32x4_t kb[2][DU];
  load_pass(0, kb[0]);
  load_pass(1, kb[1]);
  __syncthreads();  // qbar written
  // A operands, both halves: row 16h + m, dims 16u + 4kg .. + 3
  f32x4_t qa[2][DU];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int u = 0; u < DU; ++u) qa[h][u] = *reinterpret_cast<const f32x4_t*>(&qbar[16 * h + m][16 * u + 4 * kg]);
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    f32x4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int u = 0; u < DU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int h = 0; h < 2; ++h) acc[h] = mfma_f32(qa[h][u][e], kb[pass % 2][u][e], acc[h]);
    if (pass + 2 < PASSES) load_pass(pass + 2, kb[pass % 2]);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sc[16 * h + 4 * kg + i][pass * kTileCands + 16 * w + m] = score_order_bits(acc[h][i] * scale);
  }
  __syncthreads();
  // every row's scores of the chunk (thread tid: candidate c_begin + tid of
  // each row, coalesced along the candidates)
  {
    const int cand = (int)c_begin + tid;  // below kMaxCandLarge
    const int64_t stride = (int64_t)hkv * n_chunks * kLargeChunk;  // from one row of the tile to the next
    uint32_t* dst = ws_scores + ((b * q_len + t0) * hkv + g) * n_chunks * kLargeChunk + cand;
    // every row's value and count read first (one LDS round trip), then the
    // stores; rows past the tile's end have no candidates
    uint32_t v[TR];
    int nc[TR];
#pragma unroll
    for (int r = 0; r < TR; ++r) {
      v[r] = sc[r][tid];
      nc[r] = ncand[r];
    }
#pragma unroll
    for (int r = 0; r < TR; ++r)
      if (cand < nc[r]) dst[r * stride] = v[r];
  }
  // the chunk's 16 best keys of each row that needs them (wave w: rows 8w .. 8w + 7)
  for (int rr = 0; rr < TR / 4; ++rr) {
    const int r = (TR / 4) * w + rr;
    if (r >= rows) break;
    const int n_cand = ncand[r];
    if (n_cand <= kPoolCap || c_begin >= n_cand) continue;  // uniform over the wave
    static_assert(kLargeChunk == 4 * kWave && kLargeList == 16, "top16_of_256");
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) o[p] = sc[r][p * kWave + lane];
    uint64_t x[4];  // keys as make_key forms them (order image : complemented id)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int cand = (int)c_begin + p * kWave + lane;
      x[p] = cand < n_cand ? ((uint64_t)o[p] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)cand) : 0ull;
    }
    const uint64_t top = top16_of_256(x, gather[w]);
    const int64_t row = (b * q_len + t0 + r) * hkv + g;
    if (lane < kLargeList) ws_lists[(row * n_chunks + ch) * kLargeList + lane] = top;
  }
}

// Per (row, chunk of 256 candidates) of a score pass that wrote scores
// only: the chunk's 16 best keys in descending order, rebuilt from the
// written score bits (key = score bits : complemented id, as everywhere).
// One wave per (row, chunk); only rows whose candidates exceed the pick pool
// need them, the others return at once.
__global__ __launch_bounds__(kWave) void select_large_lists_kernel(const uint32_t* __restrict__ ws_scores,
                                                                   uint64_t* __restrict__ ws_lists, int64_t q_len,
                                                                   int64_t q_pos0, int hkv, int bs, int keep_tail,
                                                                   int64_t n_chunks) {
  const int64_t row = blockIdx.x / n_chunks;
  const int64_t ch = blockIdx.x % n_chunks;
  const int64_t t = (row / hkv) % q_len;
  const int64_t n_cand = row_frame(q_pos0 + t, bs, keep_tail).n_cand;
  const int64_t c_begin = ch * kLargeChunk;
  if (n_cand <= kPoolCap || c_begin >= n_cand) return;
  __shared__ uint64_t gather[kWave];
  const int lane = lane_id();
  static_assert(kLargeChunk == 4 * kWave && kLargeList == 16, "top16_of_256");
  uint64_t x[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int64_t cand = c_begin + p * kWave + lane;
    x[p] = cand < n_cand ? ((uint64_t)ws_scores[row * n_chunks * kLargeChunk + cand] << 32) |
                               (uint64_t)(0xFFFFFFFFu - (uint32_t)cand)
                         : 0ull;
  }
  const uint64_t top = top16_of_256(x, gather);
  if (lane < kLargeList) ws_lists[(row * n_chunks + ch) * kLargeList + lane] = top;
}

// One workgroup per row: cutoff, then the kept ids in ascending order.
// kv_lens (a ragged decode batch, q_len = 1): sequence b's token sits at
// position kv_lens[b] - 1, clamped as the score pass clamps it.
__global__ __launch_bounds__(kPickThreads) void select_large_pick_kernel(
    int32_t* __restrict__ sel, float* __restrict__ sel_scores, const uint32_t* __restrict__ ws_scores,
    const uint64_t* __restrict__ ws_lists, int64_t q_len, int64_t q_pos0, int hkv, int bs, int top_k, int keep_tail,
    int64_t n_chunks, const int32_t* __restrict__ kv_lens) {
  __shared__ PickSmem sm;
  const int64_t row = blockIdx.x;
  const int64_t b = row / (q_len * hkv);
  const int64_t t = (row / hkv) % q_len;
  const int g = (int)(row % hkv);
  int64_t p = q_pos0 + t;
  if (kv_lens) {
    const int64_t n = kv_lens[b];
    p = (n < 1 ? 1 : (n > q_pos0 + 1 ? q_pos0 + 1 : n)) - 1;
  }
  const Frame fr = row_frame(p, bs, keep_tail);
  const int64_t off = ((b * q_len + t) * hkv + g) * top_k;
  pick_row(sm, ws_scores + row * n_chunks * kLargeChunk, ws_lists + row * n_chunks * kLargeList, fr.n_cand,
           frame_slots(fr, top_k), fr.forced, top_k, sel + off, sel_scores ? sel_scores + off : nullptr, nullptr);
}

template <typename T, int D>
hipError_t launch_typed(const Dims& s, const SelectPlan& plan, const void* qv, int64_t q_len, int64_t q_pos0,
                        const float* k_comp, int64_t kv_cap, int32_t* sel, float* sel_scores, void* ws,
                        hipStream_t st, const void* k_cache, int64_t close_block, bool pick, const int32_t* kv_lens) {
  const T* q = static_cast<const T*>(qv);
  const T* kc = static_cast<const T*>(k_cache);
  float* kcw = const_cast<float*>(k_comp);
  const int64_t nb_cap = kv_cap / s.bs;
  const int64_t rows = (int64_t)s.batch * q_len * s.hkv;
  if (plan.large) {
    uint32_t* wss = static_cast<uint32_t*>(ws);
    uint64_t* wsl = reinterpret_cast<uint64_t*>(wss + rows * plan.n_chunks * kLargeChunk);
    if (plan.n_chunks > 0 && plan.tiled) {
      // prefill rows (close_block < 0: nothing to compress)
      const int64_t n_tiles = (q_len + kLargeTileRows - 1) / kLargeTileRows;
      const int64_t n_bg = (int64_t)s.batch * s.hkv;
      hipLaunchKernelGGL((select_large_tile_kernel<T, D>), dim3((unsigned)large_tile_grid(n_bg, plan.n_chunks, n_tiles)),
                         dim3(256), 0, st, q, k_comp, wss, wsl, q_len, q_pos0, nb_cap, s.hq, s.hkv, s.group, s.bs,
                         s.scale, s.keep_tail, plan.n_chunks, n_tiles, n_bg);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess || !pick) return e;
    } else if (plan.n_chunks > 0) {
      hipLaunchKernelGGL((select_large_score_kernel<T, D>), dim3((unsigned)(rows * plan.n_chunks)), dim3(256), 0, st,
                         q, k_comp, wss, wsl, q_len, q_pos0, nb_cap, s.hq, s.hkv, s.group, s.bs, s.scale,
                         s.keep_tail, plan.n_chunks, kc, kcw, kv_cap, close_block, kv_lens);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess || !pick) return e;
    } else if (close_block >= 0) {
      // no candidate to score (default frame, the new token closes block 0):
      // the score pass that would compress the closed block does not run, so
      // compress it here; later steps score it
      const hipError_t e = launch_compress(s, k_cache, kv_cap, close_block, close_block + 1, kcw, st);
      if (e != hipSuccess || !pick) return e;
    }
    if (!pick) return hipSuccess;
    hipLaunchKernelGGL(select_large_pick_kernel, dim3((unsigned)rows), dim3(kPickThreads), 0, st, sel, sel_scores,
                       wss, wsl, q_len, q_pos0, s.hkv, s.bs, s.top_k, s.keep_tail, plan.n_chunks, kv_lens);
    return hipGetLastError();
  }
  if (plan.tiled && s.top_k <= kRowKeep) {
    const hipError_t attr = allow_dynamic_lds<&select_rows_kernel<T, D>>(rows_lds_bytes<D>());
    if (attr != hipSuccess) return attr;
    dim3 grid((unsigned)((q_len + kRowsPerWg - 1) / kRowsPerWg), (unsigned)s.hkv, (unsigned)s.batch);
    hipLaunchKernelGGL((select_rows_kernel<T, D>), grid, dim3(512), rows_lds_bytes<D>(), st, q, k_comp, sel,
                       sel_scores, q_len, q_pos0, nb_cap, s.hq, s.hkv, s.group, s.bs, s.top_k, s.scale, s.keep_tail);
    return hipGetLastError();
  }
  if (plan.tiled) {
    dim3 grid((unsigned)((q_len + kTileRows - 1) / kTileRows), (unsigned)s.hkv, (unsigned)s.batch);
    hipLaunchKernelGGL((select_tile_kernel<T, D>), grid, dim3(256), 0, st, q, k_comp, sel, sel_scores, q_len, q_pos0,
                       nb_cap, s.hq, s.hkv, s.group, s.bs, s.top_k, s.scale, s.keep_tail);
    return hipGetLastError();
  }
  uint32_t* counters = static_cast<uint32_t*>(ws);
  uint64_t* wsk = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + (plan.n_chunks > 1 ? counter_bytes(rows) : 0));
  hipLaunchKernelGGL((select_split_kernel<T, D>), dim3((unsigned)(rows * plan.n_chunks)), dim3(256), 0, st, q,
                     k_comp, kc, kcw, kv_cap, sel, sel_scores, counters, wsk, q_len, q_pos0, nb_cap, s.hq, s.hkv, s.group, s.bs,
                     s.top_k, s.scale, s.keep_tail, plan.chunk, plan.n_chunks, close_block);
  return hipGetLastError();
}

}  // namespace

int64_t max_candidates(const Dims& s, int64_t kv_len) {
  return s.keep_tail ? kv_len / s.bs : (kv_len - 1) / s.bs;
}

SelectPlan plan_select_large(const Dims& s, int64_t q_len, int64_t q_pos0) {
  SelectPlan p{};
  const int64_t max_cand = max_candidates(s, q_pos0 + q_len);  // candidates of the last row
  const int64_t rows = (int64_t)s.batch * q_len * s.hkv;
  p.chunk = kLargeChunk;
  p.large = true;
  p.n_chunks = (max_cand + kLargeChunk - 1) / kLargeChunk;
  p.ws_bytes = (size_t)rows * p.n_chunks * (kLargeChunk * sizeof(uint32_t) + kLargeList * sizeof(uint64_t));
  // many query rows: the score pass over tiles of rows sharing a chunk
  p.tiled = q_len >= kTileRows;
  const int64_t score_grid = p.tiled ? large_tile_grid((int64_t)s.batch * s.hkv, p.n_chunks,
                                                       (q_len + kLargeTileRows - 1) / kLargeTileRows)
                                     : rows * p.n_chunks;
  p.grid = score_grid > rows ? score_grid : rows;
  return p;
}

SelectPlan plan_select(const Dims& s, int64_t q_len, int64_t q_pos0) {
  if (s.top_k > 64) return plan_select_large(s, q_len, q_pos0);
  SelectPlan p{};
  const int64_t kv_len = q_pos0 + q_len;
  const int64_t max_cand = max_candidates(s, kv_len);  // candidates of the last row
  const int64_t rows = (int64_t)s.batch * q_len * s.hkv;
  p.chunk = 256;
  p.n_chunks = 1;
  p.ws_bytes = 0;
  p.tiled = q_len >= kTileRows;
  p.grid = p.tiled ? (q_len + kTileRows - 1) / kTileRows : rows;
  if (p.tiled || max_cand <= 0) return p;
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
  p.grid = rows * p.n_chunks;
  // arrival counters (kept at zero between calls), then the chunk lists
  if (p.n_chunks > 1) p.ws_bytes = counter_bytes(rows) + (size_t)rows * p.n_chunks * (s.top_k - 1) * sizeof(uint64_t);
  return p;
}

hipError_t launch_large_pick(const Dims& s, int64_t q_len, int64_t q_pos0, int64_t n_chunks, void* ws, bool lists,
                             int32_t* sel, float* sel_scores, hipStream_t st) {
  const int64_t rows = (int64_t)s.batch * q_len * s.hkv;
  uint32_t* wss = static_cast<uint32_t*>(ws);
  uint64_t* wsl = reinterpret_cast<uint64_t*>(wss + rows * n_chunks * kLargeChunk);
  if (lists && n_chunks * kLargeChunk > kPoolCap) {
    hipLaunchKernelGGL(select_large_lists_kernel, dim3((unsigned)(rows * n_chunks)), dim3(kWave), 0, st, wss, wsl,
                       q_len, q_pos0, s.hkv, s.bs, s.keep_tail, n_chunks);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(select_large_pick_kernel, dim3((unsigned)rows), dim3(kPickThreads), 0, st, sel, sel_scores, wss,
                     wsl, q_len, q_pos0, s.hkv, s.bs, s.top_k, s.keep_tail, n_chunks, nullptr);
  return hipGetLastError();
}

hipError_t launch_select(const Dims& s, const SelectPlan& plan, const void* q, int64_t q_len, int64_t q_pos0,
                         const float* k_comp, int64_t kv_cap, int32_t* sel, float* sel_scores, void* ws,
                         hipStream_t st, const void* k_cache, int64_t close_block, bool pick,
                         const int32_t* kv_lens) {
  if (s.dtype == 1)
    return s.d == 64 ? launch_typed<uint16_t, 64>(s, plan, q, q_len, q_pos0, k_comp, kv_cap, sel, sel_scores, ws, st, k_cache, close_block, pick, kv_lens)
                     : launch_typed<uint16_t, 128>(s, plan, q, q_len, q_pos0, k_comp, kv_cap, sel, sel_scores, ws, st, k_cache, close_block, pick, kv_lens);
  return s.d == 64 ? launch_typed<float, 64>(s, plan, q, q_len, q_pos0, k_comp, kv_cap, sel, sel_scores, ws, st, k_cache, close_block, pick, kv_lens)
                   : launch_typed<float, 128>(s, plan, q, q_len, q_pos0, k_comp, kv_cap, sel, sel_scores, ws, st, k_cache, close_block, pick, kv_lens);
}

}  // namespace qsa
