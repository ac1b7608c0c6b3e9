// Block compression: one compressed key per complete block of Bs keys,
// the mean of the block's keys ("Qwen4 architecture: QSA, GatedResidual,
// PLE", section 1: keys are compressed into small blocks before scoring;
// the mean is this library's reading of the unspecified compression).
//
// HBM-streaming kernel. One wave owns one (b, g, block): every load
// instruction of the wave reads 1 KiB of consecutive keys (16 bytes per lane),
// each lane accumulates its 16-byte column slice over the rows it visits, and
// a butterfly over the lanes that share a column slice finishes the sum. All
// loads of a block are issued before the first add (Bs*d*elem bytes in flight
// per wave). Summation order is fixed, so results are deterministic.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {
namespace {

template <typename T, int D, int BS>
__global__ __launch_bounds__(256) void compress_kernel(const T* __restrict__ k, float* __restrict__ k_comp,
                                                       int64_t kv_cap, int64_t nb_cap, int64_t blk_begin,
                                                       int64_t n_blk, int64_t n_items) {
  constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte load
  constexpr int LPR = D / VEC;         // lanes covering one key row
  constexpr int RPL = kWave / LPR;     // rows per wave-wide load
  // loads per lane; a block shorter than one wave-wide load leaves the lanes
  // of its missing rows idle (they add zeros)
  constexpr int NLOAD = BS >= RPL ? BS / RPL : 1;
  static_assert(RPL >= 1, "shape");

  const int64_t item = (int64_t)blockIdx.x * 4 + wave_id();
  if (item >= n_items) return;
  const int64_t bg = item / n_blk;
  const int64_t c = blk_begin + item % n_blk;
  const int lane = lane_id();
  const int row0 = lane / LPR;
  const int col = (lane % LPR) * VEC;

  const T* src = k + (bg * kv_cap + c * BS + (row0 < BS ? row0 : 0)) * D + col;
  constexpr int BATCH = NLOAD < 16 ? NLOAD : 16;  // loads kept in flight together
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
  for (int j0 = 0; j0 < NLOAD; j0 += BATCH) {
    u32x4_t raw[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j)
      raw[j] = row0 < BS ? *reinterpret_cast<const u32x4_t*>(src + (int64_t)(j0 + j) * RPL * D)
                         : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          acc[2 * w] += bf16_lo(raw[j][w]);
          acc[2 * w + 1] += bf16_hi(raw[j][w]);
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[w] += __uint_as_float(raw[j][w]);
      }
    }
  }
#pragma unroll
  for (int m = LPR; m < kWave; m <<= 1) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += shfl_xor_f32(acc[e], m);
  }
  if (row0 == 0) {
    constexpr float inv = 1.0f / BS;  // exact: BS is a power of two
    float* dst = k_comp + (bg * nb_cap + c) * D + col;
#pragma unroll
    for (int e = 0; e < VEC; e += 4) {
      f32x4_t v = {acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
      *reinterpret_cast<f32x4_t*>(dst + e) = v;
    }
  }
}

template <typename T, int D>
hipError_t launch_d(int bs, const void* k, float* k_comp, int64_t kv_cap, int64_t nb_cap, int64_t blk_begin,
                    int64_t n_blk, int64_t n_items, hipStream_t st) {
  const int64_t grid = (n_items + 3) / 4;
  const T* kp = static_cast<const T*>(k);
  switch (bs) {
    case 4:
      hipLaunchKernelGGL((compress_kernel<T, D, 4>), dim3(grid), dim3(256), 0, st, kp, k_comp, kv_cap, nb_cap,
                         blk_begin, n_blk, n_items);
      break;
    case 8:
      hipLaunchKernelGGL((compress_kernel<T, D, 8>), dim3(grid), dim3(256), 0, st, kp, k_comp, kv_cap, nb_cap,
                         blk_begin, n_blk, n_items);
      break;
    case 16:
      hipLaunchKernelGGL((compress_kernel<T, D, 16>), dim3(grid), dim3(256), 0, st, kp, k_comp, kv_cap, nb_cap,
                         blk_begin, n_blk, n_items);
      break;
    case 32:
      hipLaunchKernelGGL((compress_kernel<T, D, 32>), dim3(grid), dim3(256), 0, st, kp, k_comp, kv_cap, nb_cap,
                         blk_begin, n_blk, n_items);
      break;
    case 64:
      hipLaunchKernelGGL((compress_kernel<T, D, 64>), dim3(grid), dim3(256), 0, st, kp, k_comp, kv_cap, nb_cap,
                         blk_begin, n_blk, n_items);
      break;
    case 128:
      hipLaunchKernelGGL((compress_kernel<T, D, 128>), dim3(grid), dim3(256), 0, st, kp, k_comp, kv_cap, nb_cap,
                         blk_begin, n_blk, n_items);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_compress(const Dims& s, const void* k, int64_t kv_cap, int64_t blk_begin, int64_t blk_end,
                           float* k_comp, hipStream_t st) {
  const int64_t n_blk = blk_end - blk_begin;
  if (n_blk <= 0) return hipSuccess;
  const int64_t nb_cap = kv_cap / s.bs;
  const int64_t n_items = (int64_t)s.batch * s.hkv * n_blk;
  if (s.dtype == 1) {
    return s.d == 64 ? launch_d<uint16_t, 64>(s.bs, k, k_comp, kv_cap, nb_cap, blk_begin, n_blk, n_items, st)
                     : launch_d<uint16_t, 128>(s.bs, k, k_comp, kv_cap, nb_cap, blk_begin, n_blk, n_items, st);
  }
  return s.d == 64 ? launch_d<float, 64>(s.bs, k, k_comp, kv_cap, nb_cap, blk_begin, n_blk, n_items, st)
                   : launch_d<float, 128>(s.bs, k, k_comp, kv_cap, nb_cap, blk_begin, n_blk, n_items, st);
}

}  // namespace qsa
