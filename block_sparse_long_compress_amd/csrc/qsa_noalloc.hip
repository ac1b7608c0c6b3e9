// qsa_decode_step_noalloc: the decode step with its workspace in library-owned
// device memory, for callers that cannot allocate (code under graph capture,
// tight serving loops, harnesses that forbid allocation). The workspace is a
// file-scope device array; each GPU the library runs on holds its own copy of
// it, at its own address, until the process ends.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/qsa.h"

namespace qsa {
qsa_status decode_step_validate(const qsa_shape* shape, const void* q, const void* k, const void* v,
                                const float* k_comp, int64_t kv_len, int64_t kv_cap, const int32_t* sel,
                                const float* sel_scores, const void* out);
}

namespace {

// The largest decode-step workspace this entry point serves
// (QSA_NOALLOC_SCRATCH_BYTES, 8 MiB): a step over 512 sequences of 128K tokens
// with 2 KV heads (4 MiB at 256), or the released budget (top-513 of 65,536
// blocks) for 8 sequences (5.3 MiB).
constexpr size_t kScratchBytes = QSA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// Host code must never use this name as a device address: in host code it
// names a host-side stand-in. Its device address, per device, comes from
// hipGetSymbolAddress below and is the only handle kernels are given.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// Zero the first `n` bytes of the scratch (n a multiple of 16) with vector
// stores: the arrival counters a step expects at zero.
__global__ void zero_counters_kernel(uint4* __restrict__ p, int64_t n16) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Device address of this device's scratch array (set-up once per device, with
// that device current).
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" qsa_status qsa_decode_step_noalloc(const qsa_shape* shape, const void* q, const void* k, const void* v,
                                              float* k_comp, int64_t kv_len, int64_t kv_cap, int32_t* sel,
                                              float* sel_scores, void* out, void* stream) {
  // every check of qsa_decode_step first: on an error nothing is enqueued
  const qsa_status st = qsa::decode_step_validate(shape, q, k, v, k_comp, kv_len, kv_cap, sel, sel_scores, out);
  if (st != QSA_OK) return st;
  const size_t need = qsa_workspace_bytes(shape, QSA_OP_DECODE_STEP, 1, kv_len);
  if (need == (size_t)-1) return QSA_ERR_INVALID;
  if (need > kScratchBytes) return QSA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    if (scratch_ptr(&ws) != hipSuccess) return QSA_ERR_HIP;
    // the decode-step workspace starts with two arrival-counter areas (one
    // counter per (sequence, KV head), each area rounded up to 256 bytes);
    // zero both, so a step never depends on what an earlier call left there
    const int64_t rows = (int64_t)shape->batch * shape->n_kv_heads;
    const size_t cnt = ((size_t)rows * 4 + 255) / 256 * 256;
    const size_t clear = 2 * cnt < need ? 2 * cnt : need;
    const int64_t n16 = (int64_t)(clear / 16);
    const unsigned grid = (unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
    hipLaunchKernelGGL(zero_counters_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint4*>(ws), n16);
    if (hipGetLastError() != hipSuccess) return QSA_ERR_HIP;
  }
  return qsa_decode_step(shape, q, k, v, k_comp, kv_len, kv_cap, sel, sel_scores, out, ws, need, stream);
}
