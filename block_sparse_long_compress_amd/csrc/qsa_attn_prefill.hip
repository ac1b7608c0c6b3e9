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
// A workgroup owns one tile of consecutive tokens of one (sequence, KV
// head): W - NP consumer waves with NCG CGs each and NP producer waves (at
// d = 128 and G = 8: 15 waves of one CG, a 30-token tile, and 1 producer).
// The tile's
// selections are merged into the ascending union of their blocks, each with
// the set of tile tokens that selected it. The producer copies the union,
// SK keys at a time (an "item": K rows and V^T operand fragments, 16 KiB at
// d = 128), into a ring of LDS stages with direct-to-LDS buffer loads; LDS
// counters (ready / done per stage) replace workgroup barriers, so each
// consumer visits only the blocks its own tokens selected, at its own pace.
// A consumer computes S^T for its CG from the staged K, runs the online
// softmax (exp2 domain, lazy rescale), and accumulates O^T from the staged
// V^T; accumulators stay in registers for the whole tile.
//
// V^T fragments come from vt_pack_kernel, which writes V in exactly the lane
// order the PV product consumes. K rows are copied as whole lines into a
// swizzled row-major layout (k_swz()).
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

// K rows of a stage sit in LDS row-major, as 256-byte lines of sixteen
// 16-byte chunks, chunk q of line L stored in slot q ^ (L % (D/8)). A copy
// instruction then moves four whole lines (full cache lines from global
// memory; a 16-rows-by-64-bytes operand pattern copies about 3x slower), and
// the 16 lanes that read one MFMA operand column (16 consecutive keys, same
// dims) hit 16 different slots: no LDS bank conflicts.
template <int D>
__device__ __forceinline__ int k_swz(int line, int q) {
  return line * 256 + 16 * (q ^ (line % (D / 8)));
}
// LDS byte offset of the 16 bytes that lane (lg, col) holds for K operand
// (su, s): key 16 su + col of the stage, dims 32 s + 8 lg .. + 7.
template <int D>
__device__ __forceinline__ int k_operand_offset(int su, int s, int lg, int col) {
  const int off = (16 * su + col) * (2 * D) + 64 * s + 16 * lg;
  return k_swz<D>(off >> 8, (off >> 4) & 15);
}

// Keys per LDS stage, which is also the softmax step: 64 when registers
// allow, else 32 (the K operands of a step stay in VGPRs).
template <int D, int BS, int W, int NCG>
constexpr int stage_keys() {
  return (W == 16) ? 32 : (W == 8) ? ((BS == 64 && D * NCG <= 128) ? 64 : 32) : ((D * NCG >= 256 || BS < 64) ? 32 : 64);
}

// One ring stage: the K and V^T operand fragments of SK consecutive keys.
template <int D, int SK, int W>
struct Stage {
  static constexpr int kKFrags = (SK / 16) * (D / 32);  // 1 KiB each: 16 keys x 32 dims
  static constexpr int kVFrags = (SK / 32) * (D / 16);  // 1 KiB each: 16 dims x 32 keys
  static constexpr int kFrags = kKFrags + kVFrags;
  static constexpr int kBytes = kFrags * 1024;
  // up to 8 stages in 128 KiB (16 KiB stages), 4 for 32 KiB stages; the
  // host drops stages while the block lists do not fit beside them (a 9th
  // 16 KiB stage measured no faster)
  static constexpr int kMaxStages = (128 * 1024 / kBytes) < 8 ? (128 * 1024 / kBytes) : 8;
  static_assert(kKFrags == kVFrags, "K and V^T copies per stage");
};

// s_waitcnt vmcnt(n) for a runtime n <= 63 (larger n waits for everything).
template <int N>
__device__ __forceinline__ void wait_vmcnt_le_impl(int n) {
  if constexpr (N == 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= N) wait_vmcnt<N>();
    else wait_vmcnt_le_impl<N - 1>(n);
  }
}
__device__ __forceinline__ void wait_vmcnt_le(int n) { wait_vmcnt_le_impl<63>(n > 63 ? 0 : n); }

// LDS counters of the ring (one pair per stage), accessed with explicit
// ds instructions: the compiler makes every atomic or volatile LDS access
// wait for all direct-to-LDS copies in flight (vmcnt(0)), which would
// serialise the ring. Each asm block waits for its own LDS operation, and
// the hardware runs one wave's LDS operations in order, after the explicit
// vmcnt waits that publish a wave's copies.
__device__ __forceinline__ unsigned lds_addr(const void* p) { return (unsigned)(uintptr_t)p; }
// Word 3 of a raw buffer descriptor (byte offsets, no swizzle).
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ lds_void_t* lds_ptr(void* p) { return (lds_void_t*)(uintptr_t)lds_addr(p); }
// 16 bytes per lane from buffer `rs` at byte offset voff into LDS at dst + 16 * lane.
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t rs, unsigned voff, void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_ptr(dst), 16, voff, 0, 0, 0);
}
// Every wait of the ring ends (the wave furthest behind never waits on
// another wave); the spin is still bounded (about 2^20 polls), so that a
// broken invariant shows up as wrong output instead of a hung GPU.
__device__ __forceinline__ void lds_wait_ge(const unsigned* c, unsigned target) {
  for (int spin = 0; spin < (1 << 20); ++spin) {
    unsigned v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(c)) : "memory");
    if (__builtin_amdgcn_readfirstlane(v) >= target) break;
    __builtin_amdgcn_s_sleep(1);
  }
}
// Adds 1 (one lane of the wave). Nothing waits for the add: a wave's LDS
// operations complete in issue order, so it lands after the wave's earlier
// LDS reads, and a later compiler-counted wait only waits longer.
__device__ __forceinline__ void lds_signal(unsigned* c) {
  if (lane_id() == 0) asm volatile("ds_add_u32 %0, %1" ::"v"(lds_addr(c)), "v"(1u) : "memory");
}
// Stores v (one lane of the wave); nothing waits on a store.
__device__ __forceinline__ void lds_store(unsigned* c, unsigned v) {
  if (lane_id() == 0) asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(c)), "v"(v) : "memory");
}
// LDS layout after the ring of `stages` x Stage::kBytes:
//   ready[stages] done[stages] (u32)  mask[n_words] (u32)  wprefix[n_words] (u32)
//   tokmask[u_cap] (u64)  ulist[u_cap] (i32)  needers[u_cap] (i32)  cum_done[u_cap * ipb] (i32)
struct PrefillLds {
  int ready, done, mask, wprefix, tokmask, ulist, needers, cum_done, total;
};
__host__ __device__ inline PrefillLds prefill_lds(int stage_bytes, int stages, int n_words, int u_cap, int ipb) {
  PrefillLds L;
  L.ready = stage_bytes * stages;
  L.done = L.ready + stages * 4;
  L.mask = L.done + stages * 4;
  L.wprefix = L.mask + n_words * 4;
  L.tokmask = (L.wprefix + n_words * 4 + 7) / 8 * 8;
  L.ulist = L.tokmask + u_cap * 8;
  L.needers = L.ulist + u_cap * 4;
  L.cum_done = L.needers + u_cap * 4;
  L.total = L.cum_done + u_cap * ipb * 4;
  return L;
}

constexpr int producers_for(int) { return 1; }

template <int D, int BS, int W, int NCG>
__global__ __launch_bounds__(W * 64, 1) void prefill_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ vt,
    const int32_t* __restrict__ sel, uint16_t* __restrict__ out, int64_t q_len, int64_t q_pos0, int64_t kv_cap,
    int64_t n_units, int hq, int hkv, int G, int top_k, float scale_log2, int n_tiles, int xcd_groups, int stages,
    int n_words_max, int u_cap) {
  constexpr int SK = stage_keys<D, BS, W, NCG>();
  using ST = Stage<D, SK, W>;
  constexpr int NT = W * 64;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int UPB = BS / kUnit;
  constexpr int IPB = BS / SK;           // ring items (stages' worth of keys) per block
  constexpr int SUB = SK / 16;           // 16-key S^T tiles per item
  constexpr int UPC = SK / kUnit;        // 32-key PV steps per item
  // one CG per wave and at most 8 V^T fragments per item: the stage is
  // released as soon as its V^T fragments are read (see run below)
  constexpr bool kEarlyDone = NCG == 1 && UPC * DT <= 8;
  extern __shared__ __align__(16) unsigned char smem[];

  // Work item: (sequence, KV head, tile). Workgroups go to the 8 XCDs
  // round-robin (XCD = workgroup id mod 8), each XCD with its own L2. With
  // xcd_groups = n pairs (n divides 8), each group of 8/n XCDs serves one
  // (sequence, KV head) pair, so an XCD's L2 holds one pair's K and V^T;
  // with xcd_groups = -m (m pairs per XCD) each XCD walks its own m pairs.
  // Slots past the last tile exit at once.
  int bg, tile;
  if (xcd_groups > 0) {
    const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const int per = 8 / xcd_groups;  // XCDs per pair
    bg = xcd / per;
    tile = slot * per + xcd % per;
  } else if (xcd_groups < 0) {
    const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    bg = xcd + 8 * (slot / n_tiles);
    tile = slot % n_tiles;
  } else {
    bg = blockIdx.x / n_tiles;
    tile = blockIdx.x % n_tiles;
  }
  if (tile >= n_tiles) return;
  tile = n_tiles - 1 - tile;  // latest tokens (most blocks) first
  const int64_t b = bg / hkv;
  const int g = bg % hkv;
  const int tpc = 16 / G;
  // Producer waves (items split between them). One: a second producer at 16
  // waves measured slower (235 against 210 us at the 8K prompt), since it
  // takes a consumer's place and the ring, not the copy rate, sets the pace.
  constexpr int NP = producers_for(W);
  constexpr int FPP = Stage<D, stage_keys<D, BS, W, NCG>(), W>::kFrags;  // copies per item
  // Items a producer keeps in flight after each wait: issuing the next item
  // must keep its outstanding copies within what vmcnt tracks (63), else the
  // issue itself stalls.
  constexpr int kLagP = (63 - FPP) / FPP < 1 ? 1 : ((63 - FPP) / FPP < 6 ? (63 - FPP) / FPP : 6);
  constexpr int WC = W - NP;           // consumer waves
  const int qt = WC * NCG * tpc;
  const int64_t t0 = (int64_t)tile * qt;
  const int tid = threadIdx.x, lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lg = lane / 16, col = lane % 16;
  const int rows = (int)(q_len - t0 < qt ? q_len - t0 : qt);
  const int64_t kv_total = q_pos0 + q_len;
  const int64_t pos_first = q_pos0 + t0;
  const int64_t own_last = (pos_first + rows - 1) / BS;
  const int n_words = (int)(own_last / 32) + 1;
  const PrefillLds L = prefill_lds(ST::kBytes, stages, n_words_max, u_cap, IPB);
  unsigned* ready = reinterpret_cast<unsigned*>(smem + L.ready);
  unsigned* done = reinterpret_cast<unsigned*>(smem + L.done);
  uint32_t* mask = reinterpret_cast<uint32_t*>(smem + L.mask);
  uint32_t* wprefix = reinterpret_cast<uint32_t*>(smem + L.wprefix);
  unsigned long long* tokmask = reinterpret_cast<unsigned long long*>(smem + L.tokmask);
  int32_t* ulist = reinterpret_cast<int32_t*>(smem + L.ulist);
  int32_t* needers = reinterpret_cast<int32_t*>(smem + L.needers);
  int32_t* cum_done = reinterpret_cast<int32_t*>(smem + L.cum_done);

  // ---- union of the tile's selections, ascending, with the token set of each block
  for (int i = tid; i < n_words; i += NT) mask[i] = 0u;
  for (int i = tid; i < stages; i += NT) ready[i] = done[i] = 0u;
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
  // consumer waves whose tokens selected each union block
  const int wtok = NCG * tpc;  // tokens per consumer wave
  const unsigned long long wmask = wtok >= 64 ? ~0ull : (1ull << wtok) - 1ull;
  for (int i = tid; i < n_union; i += NT) {
    const unsigned long long tm = tokmask[i];
    int n = 0;
    for (int cw = 0; cw < WC; ++cw) n += ((tm >> (cw * wtok)) & wmask) != 0ull ? 1 : 0;
    needers[i] = n;
  }
  __syncthreads();
  // cum_done[it]: done signals that stage it % ring has received once
  // every needer of item it (and of the stage's earlier items) is done
  const int n_items = n_union * IPB;
  const int ring = stages;
  for (int s0 = tid; s0 < ring; s0 += NT) {
    int acc = 0;
    for (int it = s0; it < n_items; it += ring) {
      acc += needers[it / IPB];
      cum_done[it] = acc;
    }
  }
  __syncthreads();

  const uint16_t* kg = k + ((b * hkv + g) * kv_cap) * D;
  const uint16_t* vtg = vt + ((b * hkv + g) * n_units) * DT * kWave * 8;

  // Producer / consumer ring, no workgroup barrier. Producer wave w copies
  // items w, w + NP, ... (SK keys of one union block: K lines and V^T
  // fragments) into stage it % ring with direct-to-LDS loads, keeps up to
  // `lag` of its items in flight, and adds 1 to ready[stage] once an item
  // has landed. A consumer wave visits only the items its tokens selected:
  // it waits until ready shows the item, computes, and adds 1 to
  // done[stage]. An item goes into a stage only after every consumer that
  // needs one of the stage's earlier items is done with it (cum_done), so
  // consumers drift up to `ring` items apart and a wave that needs a block
  // holds up none of the waves that do not. Every wait ends: an item waited
  // for was issued `ring` items before, and lag * NP < ring keeps it out of
  // every producer's not-yet-signalled tail.
  if (w < NP) {
    const int lag = kLagP < (ring - 1) / NP ? kLagP : (ring - 1) / NP;
    // K: lines 4f .. 4f+3 of the item's rows, this lane fills slot col of
    // line 4f + lg (k_swz()); V^T: fragments are contiguous.
    unsigned k_voff[ST::kKFrags], v_voff[ST::kVFrags];
#pragma unroll
    for (int f = 0; f < ST::kKFrags; ++f) {
      const int line = 4 * f + lg;
      k_voff[f] = (unsigned)(line * 256 + 16 * (col ^ (line % (D / 8))));
    }
#pragma unroll
    for (int f = 0; f < ST::kVFrags; ++f) v_voff[f] = (unsigned)((f * kWave + lane) * 16);
    int ul = -1, ul_base = -1;  // 64 union block ids, one per lane
    int k_own = 0;              // items this producer has issued
    for (int it = w; it < n_items; it += NP, ++k_own) {
      const int slot = it % ring;
      // every consumer that needs one of the stage's earlier items is done with it
      if (it >= ring) lds_wait_ge(&done[slot], (unsigned)cum_done[it - ring]);
      const int ui = it / IPB;
      if ((ui >> 6) != ul_base) {
        ul_base = ui >> 6;
        ul = (ul_base << 6) + lane < n_union ? ulist[(ul_base << 6) + lane] : 0;
      }
      const int64_t c = __builtin_amdgcn_readlane(ul, ui & 63);
      const int part = it % IPB;
      const int64_t key_first = c * BS + (int64_t)part * SK;
      unsigned char* dst = smem + slot * ST::kBytes;
      // Buffer descriptors of the item's K rows and V^T fragments: the base
      // and range live in scalar registers, each lane's offset is fixed, so
      // issuing a copy needs no vector ALU work (the consumers keep the
      // vector ALUs busy). Rows past the prefix fall outside the K range and
      // read as zero (masked out below).
      {
        const int64_t k_left = key_first < kv_total ? (kv_total - key_first) * (D * 2) : 0;
        const int k_bytes = k_left < ST::kKFrags * 1024 ? (int)k_left : ST::kKFrags * 1024;
        const __amdgpu_buffer_rsrc_t krs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(kg + key_first * D), (short)0, k_bytes, kBufferFlags);
#pragma unroll
        for (int f = 0; f < ST::kKFrags; ++f) copy_to_lds(krs, k_voff[f], dst + f * 1024);
      }
      {
        const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(vtg + (c * UPB + part * UPC) * (DT * kWave * 8)), (short)0, ST::kVFrags * 1024, kBufferFlags);
#pragma unroll
        for (int f = 0; f < ST::kVFrags; ++f) copy_to_lds(vrs, v_voff[f], dst + (ST::kKFrags + f) * 1024);
      }
      if (k_own >= lag) {
        // this producer's item it - lag * NP has landed
        if (lag == kLagP) wait_vmcnt<kLagP * FPP>();
        else wait_vmcnt_le(lag * FPP);
        lds_signal(&ready[(it - lag * NP) % ring]);
      }
    }
    wait_vmcnt<0>();
    for (int j = k_own - lag > 0 ? k_own - lag : 0; j < k_own; ++j) lds_signal(&ready[(w + j * NP) % ring]);
    return;
  }
  const int cw = w - NP;

  // ---- per CG: this lane's column token, its position, softmax state, Q operands
  u32x4_t qf[NCG][KS];
  f32x4_t o[NCG][DT];
  // Softmax sums: one more PV product per 32 keys with an all-ones V^T
  // operand sums each column's bf16 P, the same P the outputs accumulate
  // (every row of the 16 x 16 result holds the column's sum).
  f32x4_t ol[NCG];
  const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  float m_run[NCG];
  int pos_q[NCG];  // absolute positions fit in int32 (checked on the host)
  bool row_ok[NCG];
  const int tau = col / G;
#pragma unroll
  for (int n = 0; n < NCG; ++n) {
    const int r = (cw * NCG + n) * tpc + tau;
    row_ok[n] = r < rows;
    pos_q[n] = (int)(pos_first + r);
    m_run[n] = -__builtin_inff();
    ol[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const uint16_t* qs = q + ((b * q_len + t0 + r) * hq + (int64_t)g * G + col % G) * D + 8 * lg;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[n][s] = row_ok[n] ? *reinterpret_cast<const u32x4_t*>(qs + 32 * s) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[n][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int wave_shift = cw * NCG * tpc;
  const unsigned long long cg_mask = (1ull << tpc) - 1ull;

  // Only the blocks this wave's tokens selected: a ballot over 64 union
  // entries at a time, then their items in order.
  for (int base = 0; base < n_union; base += kWave) {
    const bool mine = base + lane < n_union && ((tokmask[base + lane] >> wave_shift) & wmask) != 0ull;
    unsigned long long todo = __ballot(mine);
    while (todo != 0ull) {
    const int ui = base + __builtin_ctzll(todo);
    todo &= todo - 1ull;
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
#pragma unroll 1
    for (int part = 0; part < IPB; ++part) {
    const int it = ui * IPB + part;
    const int slot = it % ring;
    lds_wait_ge(&ready[slot], (unsigned)(it / ring + 1));
    {
    const int key0 = (int)(c * BS) + part * SK;  // positions fit in int32 (checked on the host)
    const bool diag = key0 + SK > pos_first;           // holds the own block of some token: causal mask
    const unsigned char* kb = smem + slot * ST::kBytes;
    const unsigned char* vb = kb + ST::kKFrags * 1024;

    // The work of one item for the CGs in the compile-time set MASK: all S
    // products first, then the softmax updates, then the PV products, with
    // no branch between the MFMAs of one phase so that LDS reads are batched
    // ahead of their MFMAs.
    auto run = [&]<unsigned MASK>() {
      u32x4_t kf[SUB][KS];
#pragma unroll
      for (int su = 0; su < SUB; ++su)
#pragma unroll
        for (int s = 0; s < KS; ++s)
          kf[su][s] = *reinterpret_cast<const u32x4_t*>(kb + k_operand_offset<D>(su, s, lg, col));
      f32x4_t acc[NCG][SUB];
#pragma unroll
      for (int n = 0; n < NCG; ++n) {
        if (((MASK >> n) & 1u) != 0u) {
#pragma unroll
          for (int su = 0; su < SUB; ++su) {
            acc[n][su] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) acc[n][su] = mfma_bf16(kf[su][s], qf[n][s], acc[n][su]);
          }
        }
      }
      // With one CG per wave the V^T fragments are read right after the S
      // products are issued (in flight during the softmax) and the stage is
      // released before the PV products: it is held only until its data has
      // been read, not for the whole visit.
      constexpr bool kEarly = kEarlyDone;
      u32x4_t vfe[kEarly ? UPC : 1][kEarly ? DT : 1];
      if constexpr (kEarly) {
#pragma unroll
        for (int u = 0; u < UPC; ++u)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            vfe[u][dt] = *reinterpret_cast<const u32x4_t*>(vb + ((u * DT + dt) * kWave + lane) * 16);
        // a wave's LDS operations complete in order: the add lands after the reads
        lds_signal(&done[slot]);
      }
      u32x4_t pf[NCG][UPC];
#pragma unroll
      for (int n = 0; n < NCG; ++n) {
        if (((MASK >> n) & 1u) != 0u) {
          float x[SUB * 4];
#pragma unroll
          for (int su = 0; su < SUB; ++su)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[su * 4 + i] = acc[n][su][i];
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
          // The exponent offset m_run is raised only when a score exceeds it
          // by more than 2^8: p stays <= 256 (exact in fp32, representable in
          // bf16) and the accumulators are rescaled rarely.
          const float m_old = m_run[n];
          const float cand = mx * scale_log2;
          const bool grow = mem[n] && cand > m_old + kRescaleSlack;
          const float m_new = grow ? cand : m_old;
          if (__ballot(grow && m_old != -__builtin_inff()) != 0) {
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_old - m_new) : 1.0f;
            ol[n] *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[n][dt] *= alpha;
          }
          m_run[n] = m_new;
          const float negm = (mem[n] && m_new != -__builtin_inff()) ? -m_new : -__builtin_inff();
          float pv[SUB * 4];
#pragma unroll
          for (int i = 0; i < SUB * 4; ++i) {
            pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], scale_log2, negm));
          }
          // P^T operand of 32-key step u: tiles 2u, 2u+1 (see kkey())
#pragma unroll
          for (int u = 0; u < UPC; ++u) {
            const float* pa = pv + 8 * u;
            pf[n][u] = u32x4_t{cvt_pk_bf16(pa[0], pa[1]), cvt_pk_bf16(pa[2], pa[3]), cvt_pk_bf16(pa[4], pa[5]),
                               cvt_pk_bf16(pa[6], pa[7])};
          }
        }
      }
#pragma unroll
      for (int u = 0; u < UPC; ++u) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          u32x4_t vf;
          if constexpr (kEarly) vf = vfe[u][dt];
          else vf = *reinterpret_cast<const u32x4_t*>(vb + ((u * DT + dt) * kWave + lane) * 16);
#pragma unroll
          for (int n = 0; n < NCG; ++n)
            if (((MASK >> n) & 1u) != 0u) o[n][dt] = mfma_bf16(vf, pf[n][u], o[n][dt]);
        }
#pragma unroll
        for (int n = 0; n < NCG; ++n)
          if (((MASK >> n) & 1u) != 0u) ol[n] = mfma_bf16(ones, pf[n][u], ol[n]);
      }
    };
    if constexpr (NCG == 2) {
      if (need == 3u) run.template operator()<3u>();
      else if (need == 1u) run.template operator()<1u>();
      else run.template operator()<2u>();
    } else {
      // one CG at a time (every subset would multiply the code)
      if (need & 1u) run.template operator()<1u>();
      if constexpr (NCG > 1) if (need & 2u) run.template operator()<2u>();
      if constexpr (NCG > 2) if (need & 4u) run.template operator()<4u>();
      if constexpr (NCG > 3) if (need & 8u) run.template operator()<8u>();
    }
    }
    if constexpr (!kEarlyDone) lds_signal(&done[slot]);
    }
    }
  }

#pragma unroll
  for (int n = 0; n < NCG; ++n) {
    const float l = ol[n][0];
    if (!row_ok[n]) continue;
    const float inv = 1.0f / l;
    const int r = (cw * NCG + n) * tpc + tau;
    uint16_t* dst = out + ((b * q_len + t0 + r) * hq + (int64_t)g * G + col % G) * D + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const u32x2_t pk = {cvt_pk_bf16(o[n][dt][0] * inv, o[n][dt][1] * inv),
                          cvt_pk_bf16(o[n][dt][2] * inv, o[n][dt][3] * inv)};
      *reinterpret_cast<u32x2_t*>(dst + 16 * dt) = pk;
    }
  }
}

// CGs per workgroup tile: tiles of at most 64 tokens, and for d = 128 at
// most 16 CGs.
inline int ncg_for(int G, int D) {
  const int cap = D == 128 ? 4 : 8;
  return G >= cap ? cap : G;
}
// Waves per workgroup and CGs per wave. d = 128 with G >= 4: 16 waves of one
// CG each (four per SIMD: one wave's MFMA work overlaps another's softmax,
// and a block needed by few tokens stalls few waves). Otherwise 8 waves of
// 2 or 4 CGs, or 4 waves.
inline int waves_for(int G, int D) {
  if (D == 128 && ncg_for(G, D) >= 4) return 16;
  return ncg_for(G, D) >= 4 ? 8 : 4;
}
inline int ncg_per_wave(int G, int D) {
  const int w = waves_for(G, D);
  return w == 16 ? 1 : (w == 8 ? ncg_for(G, D) / 2 : ncg_for(G, D));
}

struct PrefillGeom {
  int qt, n_tiles, n_words, u_cap, stages, lds;
};

template <int D, int BS, int W, int NCG>
PrefillGeom prefill_geom(const Dims& s, int64_t q_len, int64_t q_pos0) {
  using ST = Stage<D, stage_keys<D, BS, W, NCG>(), W>;
  PrefillGeom gm;
  const int64_t kv_total = q_pos0 + q_len;
  gm.qt = (W - producers_for(W)) * NCG * (16 / s.group);  // producer waves only copy
  gm.n_tiles = (int)((q_len + gm.qt - 1) / gm.qt);
  gm.n_words = (int)(((kv_total - 1) / BS) / 32) + 1;
  const int64_t n_blocks = (kv_total + BS - 1) / BS;
  const int64_t cap = (int64_t)gm.qt * s.top_k;
  gm.u_cap = (int)(cap < n_blocks ? cap : n_blocks);
  gm.stages = ST::kMaxStages;
  gm.lds = prefill_lds(ST::kBytes, gm.stages, gm.n_words, gm.u_cap, BS / stage_keys<D, BS, W, NCG>()).total;
  while (gm.stages > 2 && gm.lds > 160 * 1024) {
    --gm.stages;
    gm.lds = prefill_lds(ST::kBytes, gm.stages, gm.n_words, gm.u_cap, BS / stage_keys<D, BS, W, NCG>()).total;
  }
  return gm;
}

template <int D, int BS, int W, int NCG>
hipError_t launch_kernel(const Dims& s, const PrefillGeom& gm, int64_t q_len, int64_t q_pos0, int64_t kv_cap,
                         int64_t n_units, const void* q, const void* k, const uint16_t* vt, const int32_t* sel,
                         void* out, hipStream_t st) {
  const hipError_t attr = allow_dynamic_lds<&prefill_attn_kernel<D, BS, W, NCG>>(160 * 1024);
  if (attr != hipSuccess) return attr;
  const int n_bg = s.batch * s.hkv;
  // one (sequence, KV head) pair per group of XCDs when pairs and tiles split evenly over the 8 XCDs
  int xcd_groups = 0;
  unsigned n_wg = (unsigned)(gm.n_tiles * n_bg);
  if (n_bg <= 8 && 8 % n_bg == 0) {
    xcd_groups = n_bg;
    const int per = 8 / n_bg;
    n_wg = 8u * (unsigned)((gm.n_tiles + per - 1) / per);
  } else if (n_bg % 8 == 0) {
    xcd_groups = -(n_bg / 8);
  }
  const float scale_log2 = s.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((prefill_attn_kernel<D, BS, W, NCG>), dim3(n_wg), dim3(W * 64), gm.lds, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), vt, sel,
                     static_cast<uint16_t*>(out), q_len, q_pos0, kv_cap, n_units, s.hq, s.hkv, s.group, s.top_k,
                     scale_log2, gm.n_tiles, xcd_groups, gm.stages, gm.n_words, gm.u_cap);
  return hipGetLastError();
}

// Kernel variant (waves, CGs per wave) used at group size G: 1 -> <4,1>,
// 2 -> <4,2>, and for larger groups <16,1> at d = 128, <8,2> (G = 4) or
// <8,4> (G >= 8) at d = 64.
template <int D, int BS>
hipError_t launch_bs(const Dims& s, int64_t q_len, int64_t q_pos0, int64_t kv_cap, int64_t n_units, const void* q,
                     const void* k, const uint16_t* vt, const int32_t* sel, void* out, hipStream_t st) {
#define QSA_LAUNCH(W, NCG) \
  launch_kernel<D, BS, W, NCG>(s, prefill_geom<D, BS, W, NCG>(s, q_len, q_pos0), q_len, q_pos0, kv_cap, n_units, q, k, vt, sel, out, st)
  const int ncg = ncg_for(s.group, D);
  if (ncg == 1) return QSA_LAUNCH(4, 1);
  if (ncg == 2) return QSA_LAUNCH(4, 2);
  if constexpr (D == 64) {
    if (ncg == 4) return QSA_LAUNCH(8, 2);
    return QSA_LAUNCH(8, 4);
  } else {
    return QSA_LAUNCH(16, 1);
  }
#undef QSA_LAUNCH
}

template <int D, int BS>
int smem_bytes(const Dims& s, int64_t q_len, int64_t q_pos0) {
  const int ncg = ncg_for(s.group, D);
  if (ncg == 1) return prefill_geom<D, BS, 4, 1>(s, q_len, q_pos0).lds;
  if (ncg == 2) return prefill_geom<D, BS, 4, 2>(s, q_len, q_pos0).lds;
  if constexpr (D == 64) {
    if (ncg == 4) return prefill_geom<D, BS, 8, 2>(s, q_len, q_pos0).lds;
    return prefill_geom<D, BS, 8, 4>(s, q_len, q_pos0).lds;
  } else {
    return prefill_geom<D, BS, 16, 1>(s, q_len, q_pos0).lds;
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

int prefill_smem_bytes(const Dims& s, int64_t q_len, int64_t q_pos0);

PrefillPlan plan_prefill(const Dims& s, int64_t q_len, int64_t q_pos0) {
  PrefillPlan p{};
  const int w = waves_for(s.group, s.d);
  p.rows_per_wg = (w - producers_for(w)) * ncg_per_wave(s.group, s.d) * (16 / s.group);
  // The tiled kernel stages whole 32-key units of one block, holds a tile
  // row's selection in 64-bit token masks and keeps its block lists in LDS;
  // other bf16 shapes run one query row per workgroup.
  p.rows = s.dtype == 1 && (s.bs < 32 || s.top_k > 64 || prefill_smem_bytes(s, q_len, q_pos0) > 160 * 1024);
  if (s.dtype != 1 || p.rows) {
    p.rows_per_wg = 1;
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
    return s.bs == 32 ? smem_bytes<64, 32>(s, q_len, q_pos0)
                      : (s.bs == 64 ? smem_bytes<64, 64>(s, q_len, q_pos0) : smem_bytes<64, 128>(s, q_len, q_pos0));
  }
  return s.bs == 32 ? smem_bytes<128, 32>(s, q_len, q_pos0)
                    : (s.bs == 64 ? smem_bytes<128, 64>(s, q_len, q_pos0) : smem_bytes<128, 128>(s, q_len, q_pos0));
}

hipError_t launch_prefill(const Dims& s, const PrefillPlan& plan, const void* q, const void* k, const void* v,
                          int64_t q_len, int64_t q_pos0, int64_t kv_cap, const int32_t* sel, void* out, void* ws,
                          hipStream_t st) {
  if (plan.rows) return launch_prefill_rows(s, q, k, v, q_len, q_pos0, kv_cap, sel, out, st);
  return s.d == 64 ? launch_d<64>(s, plan, q, k, v, q_len, q_pos0, kv_cap, sel, out, ws, st)
                   : launch_d<128>(s, plan, q, k, v, q_len, q_pos0, kv_cap, sel, out, ws, st);
}

}  // namespace qsa
