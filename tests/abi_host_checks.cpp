// Host-side checks of the C ABI (include/qsa.h), built with the host
// compiler's address and undefined-behaviour sanitizers by
// test_abi_sanitized.py and run on the CPU. Every call here either queries a
// workspace size (the planners of every path run) or carries an argument the
// host validation rejects, so nothing is ever launched and no GPU is needed.
// Exit status 0 when every status code is the documented one.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "qsa.h"

namespace {

int failures = 0;

void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

qsa_shape shape(int batch, int hq, int hkv, int d, int bs, int k, int dtype, int keep_tail = 0) {
  qsa_shape s;
  s.batch = batch;
  s.n_q_heads = hq;
  s.n_kv_heads = hkv;
  s.head_dim = d;
  s.block_size = bs;
  s.top_k = k;
  s.dtype = dtype;
  s.scale = 0.f;
  s.keep_tail = keep_tail;
  return s;
}

}  // namespace

int main() {
  // fake device addresses: never dereferenced (every call below is rejected before a launch)
  void* P = reinterpret_cast<void*>(uintptr_t(4096));
  void* MIS = reinterpret_cast<void*>(uintptr_t(4100));
  float* PF = static_cast<float*>(P);
  int32_t* PI = static_cast<int32_t*>(P);
  const size_t BAD = (size_t)-1;

  expect(qsa_abi_version(), QSA_ABI_VERSION, "abi version");
  for (int st = 0; st < 6; ++st)
    if (!qsa_status_str((qsa_status)st)) ++failures;

  // workspace sizes of every op over a spread of shapes (the planners of the
  // tiled, split, large-k, fused, sliced, scan-split, ragged and per-row paths)
  const int ds[] = {64, 128};
  const int bss[] = {4, 8, 16, 32, 64, 128};
  const int ks[] = {1, 2, 16, 33, 64, 65, 200, 513};
  const int64_t lens[] = {1, 3, 63, 64, 65, 4096, 131072, 262144, 1048576};
  const int batches[] = {1, 3, 64, 200};
  size_t checked = 0;
  for (int d : ds)
    for (int bs : bss)
      for (int k : ks)
        for (int b : batches)
          for (int dt = 0; dt < 2; ++dt)
            for (int kt = 0; kt < 2; ++kt) {
              if (kt && k < 2) continue;
              qsa_shape s = shape(b, 16, 2, d, bs, k, dt, kt);
              for (int64_t n : lens) {
                for (int op = 0; op <= QSA_OP_SELECT_RAGGED; ++op) {
                  // prefill and selection over the last 4096 query rows of n positions
                  const bool rows = op == QSA_OP_PREFILL || op == QSA_OP_SELECT || op == QSA_OP_INDEXER_SELECT ||
                                    op == QSA_OP_PREFILL_Q8;
                  const int64_t q_len = rows ? (n < 4096 ? n : 4096) : 1;
                  const size_t w = qsa_workspace_bytes(&s, op, q_len, n);
                  if (w != BAD && w > (size_t(1) << 40)) {  // at most 1 TiB for these sizes
                    std::fprintf(stderr, "FAIL workspace %zu for op %d d %d bs %d k %d b %d n %lld\n", w, op, d, bs,
                                 k, b, (long long)n);
                    ++failures;
                  }
                  ++checked;
                }
                (void)qsa_decode_step_fused(&s, n);
              }
            }
  if (checked < 1000) ++failures;

  // invalid shapes and arguments: rejected on the host, nothing enqueued
  qsa_shape good = shape(2, 16, 2, 128, 64, 16, QSA_BF16);
  qsa_shape bad_heads = shape(2, 15, 2, 128, 64, 16, QSA_BF16);
  qsa_shape bad_d = shape(2, 16, 2, 96, 64, 16, QSA_BF16);
  qsa_shape bad_tail = shape(2, 16, 2, 128, 64, 1, QSA_BF16, 1);
  qsa_shape bad_dtype = shape(2, 16, 2, 128, 64, 16, 7);
  expect(qsa_workspace_bytes(nullptr, QSA_OP_SELECT, 1, 64) == BAD, 1, "null shape size");
  expect(qsa_workspace_bytes(&good, 99, 1, 64) == BAD, 1, "unknown op size");
  expect(qsa_compress_keys(&bad_heads, P, 64, 64, 0, PF, nullptr), QSA_ERR_INVALID, "heads not a multiple");
  expect(qsa_compress_keys(&bad_d, P, 64, 64, 0, PF, nullptr), QSA_ERR_UNSUPPORTED, "head dim 96");
  expect(qsa_compress_keys(&bad_dtype, P, 64, 64, 0, PF, nullptr), QSA_ERR_INVALID, "dtype");
  expect(qsa_compress_keys(&good, P, 65, 64, 0, PF, nullptr), QSA_ERR_INVALID, "kv_len > kv_cap");
  expect(qsa_compress_keys(&good, MIS, 64, 64, 0, PF, nullptr), QSA_ERR_INVALID, "misaligned keys");
  expect(qsa_score_select(&bad_tail, P, 1, 63, PF, 64, 64, PI, nullptr, P, 1 << 20, nullptr), QSA_ERR_INVALID,
         "keep_tail with k = 1");
  expect(qsa_score_select(&good, P, 1, 62, PF, 64, 64, PI, nullptr, P, 1 << 20, nullptr), QSA_ERR_INVALID,
         "positions inconsistent");
  expect(qsa_score_select(&good, P, 1, 4095, PF, 4096, 4096, nullptr, nullptr, P, 1 << 20, nullptr),
         QSA_ERR_INVALID, "null selection");
  expect(qsa_sparse_attn_decode(&good, P, P, P, 0, 64, PI, P, P, 1 << 20, nullptr), QSA_ERR_INVALID, "kv_len 0");
  expect(qsa_sparse_attn_decode(&good, P, P, P, 70000, 70000, PI, P, nullptr, 0, nullptr), QSA_ERR_WORKSPACE,
         "decode without workspace");
  expect(qsa_sparse_attn_prefill(&good, P, P, P, 64, 1, 64, PI, P, P, 1 << 30, nullptr), QSA_ERR_INVALID,
         "prefill beyond capacity");
  expect(qsa_sparse_attn_prefill(&good, P, P, P, 64, 0, 64, PI, P, nullptr, 0, nullptr), QSA_ERR_WORKSPACE,
         "prefill without workspace");
  expect(qsa_decode_step(&good, P, P, P, PF, 4097, 4096, PI, nullptr, P, P, 1 << 20, nullptr), QSA_ERR_INVALID,
         "step beyond capacity");
  qsa_shape b64 = shape(64, 16, 2, 128, 64, 16, QSA_BF16);
  expect(qsa_decode_step(&b64, P, P, P, PF, 131072, 131072, PI, nullptr, P, P, 16, nullptr), QSA_ERR_WORKSPACE,
         "step workspace too small");
  void* MIS4 = reinterpret_cast<void*>(uintptr_t(4098));  // not 4-byte aligned
  expect(qsa_decode_step_ragged(&good, P, P, P, PF, reinterpret_cast<const int32_t*>(MIS4), 64, 64, PI, nullptr, P,
                                P, 1 << 20, nullptr),
         QSA_ERR_INVALID, "ragged lengths misaligned");
  expect(qsa_score_select_ragged(&good, P, PF, reinterpret_cast<const int32_t*>(MIS4), 64, 64, PI, nullptr, P,
                                 1 << 20, nullptr),
         QSA_ERR_INVALID, "ragged selection lengths misaligned");
  expect(qsa_score_select_ragged(&b64, P, PF, reinterpret_cast<const int32_t*>(P), 131072, 131072, PI, nullptr,
                                 nullptr, 0, nullptr),
         QSA_ERR_WORKSPACE, "ragged selection without workspace");
  expect(qsa_sparse_attn_decode_ragged(&good, P, P, P, nullptr, 64, 64, PI, P, P, 1 << 20, nullptr), QSA_ERR_INVALID,
         "ragged attention without lengths");
  expect(qsa_sparse_attn_decode_ragged(&good, P, P, P, reinterpret_cast<const int32_t*>(P), 70000, 70000, PI, P,
                                       nullptr, 0, nullptr),
         QSA_ERR_WORKSPACE, "ragged attention without workspace");
  qsa_shape big = shape(64, 16, 2, 128, 4, 513, QSA_BF16, 1);
  expect(qsa_decode_step_noalloc(&big, P, P, P, PF, 262144, 262144, PI, nullptr, P, nullptr), QSA_ERR_WORKSPACE,
         "no-alloc step beyond its scratch");
  expect(qsa_decode_step_noalloc(&good, nullptr, P, P, PF, 64, 64, PI, nullptr, P, nullptr), QSA_ERR_INVALID,
         "no-alloc step without query");
  qsa_indexer bad_ix{96, QSA_AGG_SUM, 0.f};
  expect(qsa_indexer_keys(&good, &bad_ix, PF, PF, 64, 64, 0, PF, nullptr), QSA_ERR_INVALID, "indexer dim 96");
  qsa_indexer ix{64, QSA_AGG_MAX, 0.f};
  qsa_shape k65 = shape(2, 16, 2, 128, 64, 65, QSA_BF16);
  expect(qsa_indexer_select(&k65, &ix, PF, P, 1, 127, PF, 128, 256, PI, nullptr, nullptr, 0, nullptr),
         QSA_ERR_WORKSPACE, "indexer k > 64 without workspace");
  qsa_shape k65b4 = shape(2, 16, 2, 128, 4, 65, QSA_BF16);
  expect(qsa_indexer_select(&k65b4, &ix, PF, P, 1, 4 * 70000 - 1, PF, 4 * 70000, 4 * 70000, PI, nullptr, P,
                            size_t(1) << 40, nullptr),
         QSA_ERR_UNSUPPORTED, "indexer k > 64 over more than 65536 candidates");
  float* PFW = static_cast<float*>(P);
  expect(qsa_indexer_decode_step(&good, &ix, PF, PF, P, P, P, PFW, PFW, 257, 256, PI, nullptr, P, nullptr),
         QSA_ERR_INVALID, "indexer step beyond capacity");
  expect(qsa_indexer_decode_step(&good, &ix, PF, nullptr, P, P, P, PFW, PFW, 64, 256, PI, nullptr, P, nullptr),
         QSA_ERR_INVALID, "indexer step without W_k");
  expect(qsa_indexer_decode_step(&k65, &ix, PF, PF, P, P, P, PFW, PFW, 128, 256, PI, nullptr, P, nullptr),
         QSA_ERR_UNSUPPORTED, "indexer step with k > 64");
  const int8_t* PC = static_cast<const int8_t*>(P);
  const uint16_t* PS = static_cast<const uint16_t*>(P);
  expect(qsa_sparse_attn_prefill_q8(&good, P, PC, PC, static_cast<const uint16_t*>(MIS), PS, 64, 0, 4096, PI, P,
                                    nullptr, 0, nullptr),
         QSA_ERR_INVALID, "8-bit prefill scales misaligned");
  expect(qsa_sparse_attn_prefill_q8(&good, P, PC, PC, PS, PS, 64, 4040, 4096, PI, P, nullptr, 0, nullptr), QSA_ERR_INVALID,
         "8-bit prefill beyond capacity");
  qsa_shape f32_16 = shape(2, 16, 2, 128, 16, 16, QSA_F32);
  expect(qsa_sparse_attn_prefill_q8(&f32_16, P, PC, PC, PS, PS, 64, 0, 4096, PI, P, nullptr, 0, nullptr), QSA_ERR_UNSUPPORTED,
         "8-bit prefill with a float32 shape");
  qsa_shape f32 = shape(2, 16, 2, 128, 64, 16, QSA_F32);
  expect(qsa_kv_quantize(&f32, P, P, 64, 64, 0, static_cast<int8_t*>(P), static_cast<int8_t*>(P),
                         static_cast<uint16_t*>(P), static_cast<uint16_t*>(P), nullptr),
         QSA_ERR_UNSUPPORTED, "8-bit cache from float32");

  if (failures) {
    std::fprintf(stderr, "%d failure(s)\n", failures);
    return 1;
  }
  std::printf("ok: %zu workspace queries, every invalid call rejected\n", checked);
  return 0;
}
