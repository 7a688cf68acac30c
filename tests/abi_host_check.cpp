// Host-only driver for the sanitizer build of the C ABI (AddressSanitizer + UndefinedBehaviorSanitizer on
// the host code of abi.hip; device code is not instrumented and nothing here launches a kernel).  It calls
// every entry point along its argument-checking paths, including the size arithmetic near its overflow
// limits, and exits nonzero if any call returns an unexpected status.  Run by tests/test_abi.py.
#include <stdint.h>
#include <stdio.h>

#include <cmath>
#include <cstring>

#include "../include/paged_attention_attn.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "%s: got %d, want %d\n", what, got, want);
    ++failures;
  }
}

int main() {
  void* P = reinterpret_cast<void*>(uintptr_t{0x10000});  // never dereferenced
  void* M = reinterpret_cast<void*>(uintptr_t{0x10008});  // misaligned for 16-byte tensors
  int* I = static_cast<int*>(P);
  float* F = static_cast<float*>(P);
  const float nan = std::nanf("");
  const float inf = INFINITY;
  hipStream_t S = reinterpret_cast<hipStream_t>(uintptr_t{0x20000});  // never used: every call fails first

  // prefill family
  for (int f = 0; f < 4; ++f) {
    auto call = [&](void* q, int B, int H, int Hkv, int N, int d, float scale) {
      switch (f) {
        case 0: return attn_fwd(q, P, P, P, nullptr, B, H, Hkv, N, d, 1, scale, nullptr);
        case 1: return attn_fwd_f32((float*)q, F, F, F, nullptr, B, H, Hkv, N, d, 1, scale, nullptr);
        case 2: return attn_fwd_window(q, P, P, P, nullptr, B, H, Hkv, N, d, 4, 0, scale, nullptr);
        default: return attn_fwd_fp8(q, P, P, P, nullptr, B, H, Hkv, N, d, 1, scale, 1.f, 1.f, 1.f, nullptr);
      }
    };
    expect(call(nullptr, 1, 2, 2, 16, 64, 0.1f), ATTN_ERR_NULL_POINTER, "prefill null q");
    expect(call(P, 1, 4, 3, 16, 64, 0.1f), ATTN_ERR_INVALID_SHAPE, "prefill H % Hkv");
    expect(call(P, -1, 2, 2, 16, 64, 0.1f), ATTN_ERR_INVALID_SHAPE, "prefill negative B");
    expect(call(P, 1, 2, 2, 16, 96, 0.1f), ATTN_ERR_UNSUPPORTED_HEAD_DIM, "prefill d");
    expect(call(M, 1, 2, 2, 16, 64, 0.1f), ATTN_ERR_MISALIGNED, "prefill alignment");
    expect(call(P, 0x7fffffff, 0x7fffffff, 1, 0x7ffffff0, 128, 0.1f), ATTN_ERR_TOO_LARGE, "prefill overflow");
    expect(call(P, 1, 1, 1, 1 << 23, 128, 0.1f), ATTN_ERR_TOO_LARGE, "prefill 2 GiB head");
    expect(call(P, 1, 1, 1, 0x7ffffff0, 128, 0.1f), ATTN_ERR_TOO_LARGE, "prefill N near INT_MAX");
    expect(call(nullptr, 0, 2, 2, 16, 64, 0.1f), ATTN_OK, "prefill empty batch");
    for (float bad : {0.f, -1.f, nan, inf}) expect(call(P, 1, 2, 2, 16, 64, bad), ATTN_ERR_INVALID_SCALE, "scale");
  }
  expect(attn_fwd_fp8(P, P, P, P, nullptr, 1, 2, 2, 40, 64, 1, 0.1f, 1.f, 1.f, 1.f, nullptr), ATTN_ERR_INVALID_SHAPE,
         "fp8 N % 16");
  expect(attn_fwd_window(P, P, P, P, nullptr, 1, 2, 2, 16, 64, 0, 0, 0.1f, nullptr), ATTN_ERR_INVALID_SHAPE,
         "window 0");

  // decode workspace arithmetic at its limits
  expect(paged_attn_decode_workspace_size(-1, 8, 128, 16, 10) == 0, 1, "workspace negative seqs");
  expect(paged_attn_decode_workspace_size(4, 8, 96, 16, 10) == 0, 1, "workspace d");
  expect(paged_attn_decode_workspace_size(0x7fffffff, 0x7fffffff, 128, 16, 0x7fffffff) == 0, 1, "workspace overflow");
  expect(paged_attn_decode_workspace_size(64, 32, 128, 16, 512) > 0, 1, "workspace normal");
  const size_t ws = paged_attn_decode_workspace_size(4, 8, 128, 16, 10);

  // decode: eager, fp8, no-alloc
  auto dec = [&](int which, void* q, void* bt, int S_, int H, int Hkv, int d, int ps, int mp, int np_, float scale,
                 void* w, size_t wb) {
    if (which == 0)
      return paged_attn_decode(q, P, P, (int*)bt, I, P, nullptr, S_, H, Hkv, d, ps, mp, np_, scale, w, wb, nullptr);
    if (which == 1)
      return paged_attn_decode_fp8(q, P, P, 0.5f, 0.5f, (int*)bt, I, P, nullptr, S_, H, Hkv, d, ps, mp, np_, scale, w,
                                   wb, nullptr);
    return paged_attn_decode_no_alloc(q, P, P, (int*)bt, I, P, nullptr, S_, H, Hkv, d, ps, mp, np_, scale, nullptr);
  };
  for (int which = 0; which < 3; ++which) {
    expect(dec(which, P, nullptr, 4, 8, 2, 128, 16, 10, 100, 0.1f, P, ws), ATTN_ERR_NULL_POINTER, "decode null table");
    expect(dec(which, P, P, 4, 8, 3, 128, 16, 10, 100, 0.1f, P, ws), ATTN_ERR_INVALID_SHAPE, "decode H % Hkv");
    expect(dec(which, P, P, 4, 8, 2, 80, 16, 10, 100, 0.1f, P, ws), ATTN_ERR_UNSUPPORTED_HEAD_DIM, "decode d");
    expect(dec(which, P, P, 4, 8, 2, 128, 32, 10, 100, 0.1f, P, ws), ATTN_ERR_UNSUPPORTED_PAGE_SIZE, "decode page");
    expect(dec(which, P, P, 4, 64, 2, 128, 16, 10, 100, 0.1f, P, 1u << 30), ATTN_ERR_UNSUPPORTED_GROUP, "decode grp");
    expect(dec(which, M, P, 4, 8, 2, 128, 16, 10, 100, 0.1f, P, ws), ATTN_ERR_MISALIGNED, "decode alignment");
    expect(dec(which, P, P, 4, 8, 2, 128, 16, 1 << 28, 100, 0.1f, P, ws), ATTN_ERR_TOO_LARGE, "decode positions");
    expect(dec(which, P, P, 4, 8, 2, 128, 16, 10, 100, nan, P, ws), ATTN_ERR_INVALID_SCALE, "decode scale");
    expect(dec(which, nullptr, nullptr, 0, 8, 2, 128, 16, 10, 100, 0.1f, nullptr, 0), ATTN_OK, "decode empty");
  }
  expect(dec(0, P, P, 4, 8, 2, 128, 16, 10, 100, 0.1f, P, ws - 1), ATTN_ERR_WORKSPACE_TOO_SMALL, "decode ws");
  expect(dec(2, P, P, 100000, 32, 8, 128, 16, 1024, 40000, 0.1f, nullptr, 0), ATTN_ERR_SCRATCH_TOO_SMALL,
         "no-alloc scratch limit");

  // chunked prefill
  auto pp = [&](void* q, int S_, int H, int Hkv, int d, int ps, int mp, int np_, int mq, float scale) {
    return paged_prefill(q, P, P, P, P, I, I, I, P, nullptr, S_, H, Hkv, d, ps, mp, np_, mq, scale, nullptr);
  };
  expect(pp(nullptr, 2, 8, 2, 128, 16, 4, 10, 33, 0.1f), ATTN_ERR_NULL_POINTER, "chunked null");
  expect(pp(P, 2, 6, 4, 128, 16, 4, 10, 33, 0.1f), ATTN_ERR_INVALID_SHAPE, "chunked H % Hkv");
  expect(pp(P, 2, 8, 2, 128, 16, 1 << 28, 10, 33, 0.1f), ATTN_ERR_TOO_LARGE, "chunked positions");
  expect(pp(P, 2, 8, 8, 128, 16, 4, 10, 1 << 20, 0.1f), ATTN_ERR_TOO_LARGE, "chunked chunk rows");
  expect(pp(P, 0x7fffffff, 0x7fffffff, 1, 128, 16, 4, 10, 0x7fffffff, 0.1f), ATTN_ERR_TOO_LARGE, "chunked grid");
  expect(pp(nullptr, 0, 8, 2, 128, 16, 4, 10, 33, 0.1f), ATTN_OK, "chunked empty");

  // decode graph: argument errors come back before any capture
  attn_decode_call c;
  std::memset(&c, 0, sizeof(c));
  c.q = P; c.k_cache = P; c.v_cache = P; c.block_table = I; c.seq_lens = I; c.o = P; c.num_seqs = 4; c.H = 8;
  c.Hkv = 2; c.d = 128; c.page_size = 16; c.max_pages_per_seq = 10; c.num_pages = 100; c.scale = 0.1f;
  c.workspace = P; c.workspace_bytes = ws;
  void* handle = P;
  attn_decode_call bad = c;
  bad.page_size = 32;
  attn_decode_call calls[2] = {c, bad};
  expect(paged_attn_decode_graph_create(calls, 2, S, &handle), ATTN_ERR_UNSUPPORTED_PAGE_SIZE, "graph page");
  expect(handle == nullptr, 1, "graph handle cleared");
  bad = c;
  bad.q = M;
  calls[1] = bad;
  expect(paged_attn_decode_graph_create(calls, 2, S, &handle), ATTN_ERR_MISALIGNED, "graph alignment");
  expect(paged_attn_decode_graph_create(calls, 0, S, &handle), ATTN_ERR_INVALID_SHAPE, "graph empty");
  expect(paged_attn_decode_graph_create(calls, 1, nullptr, &handle), ATTN_ERR_NULL_POINTER, "graph null stream");
  expect(paged_attn_decode_graph_launch(nullptr, nullptr), ATTN_ERR_NULL_POINTER, "graph launch null");
  expect(paged_attn_decode_graph_destroy(nullptr), ATTN_OK, "graph destroy null");

  for (int code = -3; code < 20; ++code)
    if (attn_status_string(code) == nullptr || std::strlen(attn_status_string(code)) == 0) ++failures;

  if (failures == 0) printf("abi host checks passed\n");
  return failures == 0 ? 0 : 1;
}
