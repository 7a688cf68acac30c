// The C ABI: host-side argument checks, then the launchers in launch.hpp.
// Nothing here touches device memory or synchronises; every check uses only
// the host-visible sizes and pointer values.

#include <stdint.h>

#include <mutex>

#include "../../include/paged_attention_attn.h"
#include "launch.hpp"

namespace {

// Decode workspace for callers that cannot allocate (paged_attn_decode_no_alloc).  Each GPU the library
// runs on holds its own copy until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: only the address hipGetSymbolAddress returns for a device is ever passed to a kernel.
constexpr size_t kScratchBytes = ATTN_DECODE_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The device address of `scratch` on the device that runs `stream`, looked up once per device with that
// device current (the caller's current device is restored).
int scratch_for(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return ATTN_ERR_LAUNCH;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return ATTN_ERR_LAUNCH;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return ATTN_ERR_LAUNCH;
    if (e != hipSuccess || ptr == nullptr) return ATTN_ERR_LAUNCH;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Elements of a [a0, a1, a2, a3] tensor, or -1 when it overflows 2^62.
long long elems(long long a0, long long a1, long long a2, long long a3) {
  const long long lim = 1LL << 62;
  long long r = 1;
  for (long long x : {a0, a1, a2, a3}) {
    if (x != 0 && r > lim / x) return -1;
    r *= x;
  }
  return r;
}

// Shape checks first: an empty call (B == 0 or N == 0) is valid whatever the
// pointers are, because nothing is read or written.
// The kernels track the running maximum of raw (unscaled) scores, which is the
// maximum of the scaled ones only for a positive scale.
bool scale_ok(float scale) { return scale > 0.f && scale <= 3.4e38f; }

int check_prefill(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H,
                  int Hkv, int N, int d, float scale) {
  if (B < 0 || N < 0 || H < 1 || Hkv < 1 || H % Hkv != 0) return ATTN_ERR_INVALID_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
  if (!scale_ok(scale)) return ATTN_ERR_INVALID_SCALE;
  if (B == 0 || N == 0) return ATTN_OK;
  if (!q || !k || !v || !o) return ATTN_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return ATTN_ERR_MISALIGNED;
  if (elems(B, H, N, d) < 0) return ATTN_ERR_TOO_LARGE;
  // query tiles x heads x batch must fit one 1-D grid
  const long long units = elems(B, H, ((long long)N + 31) / 32, 1);
  if (units < 0 || units > 0x7fffffffLL) return ATTN_ERR_TOO_LARGE;
  // the kernels read one (batch entry, KV head) of K or V through a buffer resource, whose size
  // (and the lanes' offsets into it) are below 2^31 bytes
  if ((long long)N * d * 2 > 0x7fffffffLL) return ATTN_ERR_TOO_LARGE;
  return ATTN_OK;
}

int launch_status(hipError_t e) {
  if (e == hipSuccess) return ATTN_OK;
  if (e == hipErrorInvalidValue) return ATTN_ERR_TOO_LARGE;
  return ATTN_ERR_LAUNCH;
}

constexpr size_t kWsAlign = 256;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace layout: partial outputs [slots, H, d] fp32, partial LSE [slots, H]
// fp32, then the [num_seqs, 2] int32 slot range of each sequence and one int32
// holding the total page count; each region
// starts on a kWsAlign boundary.  slots = partitions + num_seqs.
struct DecodeWs {
  long long slots;
  size_t o_bytes, lse_bytes, range_bytes;
  size_t total() const { return o_bytes + lse_bytes + range_bytes; }
};

bool decode_ws(int num_seqs, int H, int d, int max_pages_per_seq, DecodeWs* w) {
  long long parts = paa::decode_max_parts(H);
  const long long pages = (long long)num_seqs * max_pages_per_seq;
  if (parts > pages) parts = pages;
  if (parts < 1) parts = 1;
  w->slots = parts + num_seqs;
  const long long rows = elems(w->slots, H, 1, 1);
  if (rows < 0 || elems(rows, d + 1, 4, 1) < 0) return false;
  w->o_bytes = round_up((size_t)rows * d * sizeof(float), kWsAlign);
  w->lse_bytes = round_up((size_t)rows * sizeof(float), kWsAlign);
  w->range_bytes = round_up(((size_t)num_seqs * 2 + 1) * sizeof(int32_t), kWsAlign);
  return true;
}

// Argument checks shared by both decode entry points and the graph builder: the bf16 cache, or (fp8)
// an E4M3 cache with per-tensor scales.  Host-visible sizes and pointer values only.
int check_decode(const void* q, const void* k_cache, const void* v_cache, bool fp8, float k_scale, float v_scale,
                 const int32_t* block_table, const int32_t* seq_lens, const void* o, const float* lse, int num_seqs,
                 int H, int Hkv, int d, int page_size, int max_pages_per_seq, int num_pages, float scale,
                 const void* workspace, size_t workspace_bytes) {
  if (num_seqs < 0 || H < 1 || Hkv < 1 || H % Hkv != 0 || max_pages_per_seq < 0 || num_pages < 0)
    return ATTN_ERR_INVALID_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
  if (page_size != 16) return ATTN_ERR_UNSUPPORTED_PAGE_SIZE;
  if (H / Hkv > 16) return ATTN_ERR_UNSUPPORTED_GROUP;
  if (!scale_ok(scale) || (fp8 && (!scale_ok(k_scale) || !scale_ok(v_scale)))) return ATTN_ERR_INVALID_SCALE;
  if (num_seqs == 0) return ATTN_OK;  // empty call: nothing is read or written
  // block_table may be NULL only when it has no columns (then it is never read)
  if (!q || !k_cache || !v_cache || (!block_table && max_pages_per_seq > 0) || !seq_lens || !o || !workspace)
    return ATTN_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 4) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(lse, 4) || !aligned(workspace, 16))
    return ATTN_ERR_MISALIGNED;
  if (elems(num_pages, page_size, Hkv, d) < 0) return ATTN_ERR_TOO_LARGE;
  // page positions and (sequence, head) rows are 32-bit inside the kernels
  if ((long long)num_seqs * max_pages_per_seq > 0x7fffffffLL / page_size ||
      (long long)num_seqs * H > 0x7fffffffLL)
    return ATTN_ERR_TOO_LARGE;
  DecodeWs w;
  if (!decode_ws(num_seqs, H, d, max_pages_per_seq, &w)) return ATTN_ERR_TOO_LARGE;
  if (workspace_bytes < w.total()) return ATTN_ERR_WORKSPACE_TOO_SMALL;
  return ATTN_OK;
}

// Enqueues one decode (partial and reduce kernels) after check_decode has passed.
int launch_decode(const void* q, const void* k_cache, const void* v_cache, bool fp8, float k_scale, float v_scale,
                  const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse, int num_seqs, int H,
                  int Hkv, int d, int max_pages_per_seq, int num_pages, float scale, void* workspace,
                  hipStream_t stream) {
  if (num_seqs == 0) return ATTN_OK;
  DecodeWs w;
  decode_ws(num_seqs, H, d, max_pages_per_seq, &w);
  const int parts = paa::decode_parts(num_seqs, H, Hkv, max_pages_per_seq);
  char* base = static_cast<char*>(workspace);
  float* ws_o = reinterpret_cast<float*>(base);
  float* ws_lse = reinterpret_cast<float*>(base + w.o_bytes);
  int* ws_range = reinterpret_cast<int*>(base + w.o_bytes + w.lse_bytes);
  return launch_status(paa::paged_decode(q, k_cache, v_cache, fp8, k_scale, v_scale, block_table, seq_lens, o, lse,
                                         num_seqs, H, Hkv, d, max_pages_per_seq, num_pages, scale, ws_o, ws_lse,
                                         ws_range, parts, (int)w.slots, stream));
}

int decode_call(const void* q, const void* k_cache, const void* v_cache, bool fp8, float k_scale, float v_scale,
                const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse, int num_seqs, int H, int Hkv,
                int d, int page_size, int max_pages_per_seq, int num_pages, float scale, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  const int rc = check_decode(q, k_cache, v_cache, fp8, k_scale, v_scale, block_table, seq_lens, o, lse, num_seqs, H,
                              Hkv, d, page_size, max_pages_per_seq, num_pages, scale, workspace, workspace_bytes);
  if (rc != ATTN_OK) return rc;
  return launch_decode(q, k_cache, v_cache, fp8, k_scale, v_scale, block_table, seq_lens, o, lse, num_seqs, H, Hkv, d,
                       max_pages_per_seq, num_pages, scale, workspace, stream);
}

struct DecodeGraph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

// The same checks as paged_attn_decode, for one call of a graph (nothing is launched).
int check_decode_call(const attn_decode_call& c) {
  if (c.kv_fp8 != 0 && c.kv_fp8 != 1) return ATTN_ERR_INVALID_SHAPE;
  return check_decode(c.q, c.k_cache, c.v_cache, c.kv_fp8 != 0, c.k_scale, c.v_scale, c.block_table, c.seq_lens, c.o,
                      c.lse, c.num_seqs, c.H, c.Hkv, c.d, c.page_size, c.max_pages_per_seq, c.num_pages, c.scale,
                      c.workspace, c.workspace_bytes);
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N, int d,
             int causal, float scale, hipStream_t stream) {
  const int rc = check_prefill(q, k, v, o, lse, B, H, Hkv, N, d, scale);
  if (rc != ATTN_OK) return rc;
  if (B == 0 || N == 0) return ATTN_OK;
  return launch_status(paa::prefill_bf16(q, k, v, o, lse, B, H, Hkv, N, d, causal != 0, 0, 0, scale, stream));
}

int attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N,
                    int d, int window, int n_global, float scale, hipStream_t stream) {
  const int rc = check_prefill(q, k, v, o, lse, B, H, Hkv, N, d, scale);
  if (rc != ATTN_OK) return rc;
  if (window < 1 || n_global < 0) return ATTN_ERR_INVALID_SHAPE;
  if (B == 0 || N == 0) return ATTN_OK;
  return launch_status(paa::prefill_bf16(q, k, v, o, lse, B, H, Hkv, N, d, true, window, n_global, scale, stream));
}

int attn_fwd_fp8(const void* q, const void* k, const void* v_t, void* o, float* lse, int B, int H, int Hkv, int N,
                 int d, int causal, float scale, float q_scale, float k_scale, float v_scale, hipStream_t stream) {
  const int rc = check_prefill(q, k, v_t, o, lse, B, H, Hkv, N, d, scale);
  if (rc != ATTN_OK) return rc;
  if (!scale_ok(q_scale) || !scale_ok(k_scale) || !scale_ok(v_scale)) return ATTN_ERR_INVALID_SCALE;
  if (N % 16 != 0) return ATTN_ERR_INVALID_SHAPE;  // rows of the transposed V start 16-byte aligned
  if (B == 0 || N == 0) return ATTN_OK;
  return launch_status(
      paa::prefill_fp8(q, k, v_t, o, lse, B, H, Hkv, N, d, causal != 0, scale, q_scale, k_scale, v_scale, stream));
}

int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int Hkv, int N,
                 int d, int causal, float scale, hipStream_t stream) {
  const int rc = check_prefill(q, k, v, o, lse, B, H, Hkv, N, d, scale);
  if (rc != ATTN_OK) return rc;
  if (B == 0 || N == 0) return ATTN_OK;
  return launch_status(paa::prefill_f32(q, k, v, o, lse, B, H, Hkv, N, d, causal != 0, scale, stream));
}

size_t paged_attn_decode_workspace_size(int num_seqs, int H, int d, int page_size, int max_pages_per_seq) {
  if (num_seqs < 0 || H < 1 || (d != 64 && d != 128) || page_size != 16 || max_pages_per_seq < 0) return 0;
  if (num_seqs == 0) return kWsAlign;
  DecodeWs w;
  if (!decode_ws(num_seqs, H, d, max_pages_per_seq, &w)) return 0;
  return w.total();
}

int paged_attn_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                      const int32_t* seq_lens, void* o, float* lse, int num_seqs, int H, int Hkv, int d, int page_size,
                      int max_pages_per_seq, int num_pages, float scale, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  return decode_call(q, k_cache, v_cache, false, 1.f, 1.f, block_table, seq_lens, o, lse, num_seqs, H, Hkv, d,
                     page_size, max_pages_per_seq, num_pages, scale, workspace, workspace_bytes, stream);
}

int paged_attn_decode_fp8(const void* q, const void* k_cache, const void* v_cache, float k_scale, float v_scale,
                          const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse, int num_seqs,
                          int H, int Hkv, int d, int page_size, int max_pages_per_seq, int num_pages, float scale,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_call(q, k_cache, v_cache, true, k_scale, v_scale, block_table, seq_lens, o, lse, num_seqs, H, Hkv, d,
                     page_size, max_pages_per_seq, num_pages, scale, workspace, workspace_bytes, stream);
}

int paged_prefill(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                  const int32_t* block_table, const int32_t* ctx_lens, const int32_t* q_start, void* o, float* lse,
                  int num_seqs, int H, int Hkv, int d, int page_size, int max_pages_per_seq, int num_pages,
                  int max_q_len, float scale, hipStream_t stream) {
  if (num_seqs < 0 || max_q_len < 0 || H < 1 || Hkv < 1 || H % Hkv != 0 || max_pages_per_seq < 1 || num_pages < 1)
    return ATTN_ERR_INVALID_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
  if (page_size != 16) return ATTN_ERR_UNSUPPORTED_PAGE_SIZE;
  if (!scale_ok(scale)) return ATTN_ERR_INVALID_SCALE;
  if (num_seqs == 0 || max_q_len == 0) return ATTN_OK;
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !block_table || !ctx_lens || !q_start || !o)
    return ATTN_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(o, 16) || !aligned(lse, 4) || !aligned(block_table, 4) ||
      !aligned(ctx_lens, 4) || !aligned(q_start, 4))
    return ATTN_ERR_MISALIGNED;
  // positions (context + chunk) are ints on the device; the grid is one dimension
  if ((long long)max_pages_per_seq * page_size > 0x7fffffffLL) return ATTN_ERR_TOO_LARGE;
  if (elems(num_pages, page_size, Hkv, d) < 0 || elems(num_seqs, max_pages_per_seq, 1, 1) < 0)
    return ATTN_ERR_TOO_LARGE;
  const long long units = elems(num_seqs, H, ((long long)max_q_len + 31) / 32, 1);
  if (units < 0 || units > 0x7fffffffLL) return ATTN_ERR_TOO_LARGE;
  // one sequence's chunk rows of k_new / v_new are read through a buffer resource below 2^31 bytes
  if ((long long)max_q_len * Hkv * d * 2 > 0x7fffffffLL) return ATTN_ERR_TOO_LARGE;
  return launch_status(paa::paged_prefill_bf16(q, k_new, v_new, k_cache, v_cache, block_table, ctx_lens, q_start, o,
                                               lse, num_seqs, H, Hkv, d, max_pages_per_seq, num_pages, max_q_len,
                                               scale, stream));
}

int paged_attn_decode_no_alloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                               const int32_t* seq_lens, void* o, float* lse, int num_seqs, int H, int Hkv, int d,
                               int page_size, int max_pages_per_seq, int num_pages, float scale, hipStream_t stream) {
  // the workspace checks run against a stand-in pointer; the real address is looked up only after every
  // host-side check has passed
  const void* stand_in = reinterpret_cast<const void*>(uintptr_t{256});
  int rc = check_decode(q, k_cache, v_cache, false, 1.f, 1.f, block_table, seq_lens, o, lse, num_seqs, H, Hkv, d,
                        page_size, max_pages_per_seq, num_pages, scale, stand_in, kScratchBytes);
  if (rc == ATTN_ERR_WORKSPACE_TOO_SMALL) return ATTN_ERR_SCRATCH_TOO_SMALL;
  if (rc != ATTN_OK || num_seqs == 0) return rc;
  void* ws = nullptr;
  rc = scratch_for(stream, &ws);
  if (rc != ATTN_OK) return rc;
  return launch_decode(q, k_cache, v_cache, false, 1.f, 1.f, block_table, seq_lens, o, lse, num_seqs, H, Hkv, d,
                       max_pages_per_seq, num_pages, scale, ws, stream);
}

// ---- the decode step as a replayable hipGraph ----

int paged_attn_decode_graph_create(const attn_decode_call* calls, int num_calls, hipStream_t capture_stream,
                                   void** graph_out) {
  if (graph_out == nullptr) return ATTN_ERR_NULL_POINTER;
  *graph_out = nullptr;
  if (calls == nullptr || capture_stream == nullptr) return ATTN_ERR_NULL_POINTER;  // the null stream cannot be captured
  if (num_calls < 1) return ATTN_ERR_INVALID_SHAPE;
  // every argument check happens before capture begins
  for (int i = 0; i < num_calls; ++i) {
    const int rc = check_decode_call(calls[i]);
    if (rc != ATTN_OK) return rc;
  }
  // one-time kernel attributes are set outside the capture
  for (int i = 0; i < num_calls; ++i)
    if (paa::decode_setup(calls[i].d, calls[i].kv_fp8 != 0) != hipSuccess) return ATTN_ERR_LAUNCH;
  if (hipStreamBeginCapture(capture_stream, hipStreamCaptureModeThreadLocal) != hipSuccess) return ATTN_ERR_LAUNCH;
  int rc = ATTN_OK;
  for (int i = 0; i < num_calls && rc == ATTN_OK; ++i) {
    const attn_decode_call& c = calls[i];
    rc = launch_decode(c.q, c.k_cache, c.v_cache, c.kv_fp8 != 0, c.k_scale, c.v_scale, c.block_table, c.seq_lens,
                       c.o, c.lse, c.num_seqs, c.H, c.Hkv, c.d, c.max_pages_per_seq, c.num_pages, c.scale, c.workspace,
                       capture_stream);
  }
  hipGraph_t graph = nullptr;
  const hipError_t end = hipStreamEndCapture(capture_stream, &graph);  // always end the capture
  // Every argument was checked before the capture began, so any failure from here on is the runtime's
  // (ATTN_ERR_LAUNCH); a graph that cannot be released is reported the same way.
  if (rc != ATTN_OK || end != hipSuccess || graph == nullptr) {
    const bool released = graph == nullptr || hipGraphDestroy(graph) == hipSuccess;
    return released && rc != ATTN_OK ? rc : ATTN_ERR_LAUNCH;
  }
  hipGraphExec_t exec = nullptr;
  if (hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess) {
    const hipError_t released = hipGraphDestroy(graph);
    (void)released;  // the call has failed (ATTN_ERR_LAUNCH) whether or not the graph could be released
    return ATTN_ERR_LAUNCH;
  }
  *graph_out = new DecodeGraph{graph, exec};
  return ATTN_OK;
}

int paged_attn_decode_graph_launch(void* graph, hipStream_t stream) {
  if (graph == nullptr) return ATTN_ERR_NULL_POINTER;
  return hipGraphLaunch(static_cast<DecodeGraph*>(graph)->exec, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int paged_attn_decode_graph_destroy(void* graph) {
  if (graph == nullptr) return ATTN_OK;
  DecodeGraph* g = static_cast<DecodeGraph*>(graph);
  const hipError_t e1 = hipGraphExecDestroy(g->exec);
  const hipError_t e2 = hipGraphDestroy(g->graph);
  delete g;
  return e1 == hipSuccess && e2 == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULL_POINTER: return "a required pointer argument is NULL";
    case ATTN_ERR_INVALID_SHAPE: return "invalid shape: sizes must be non-negative, H and Hkv >= 1, H % Hkv == 0";
    case ATTN_ERR_UNSUPPORTED_HEAD_DIM: return "unsupported head dimension: d must be 64 or 128";
    case ATTN_ERR_UNSUPPORTED_PAGE_SIZE: return "unsupported page size: page_size must be 16";
    case ATTN_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than paged_attn_decode_workspace_size()";
    case ATTN_ERR_MISALIGNED: return "misaligned pointer: tensors need 16-byte, lse/tables 4-byte alignment";
    case ATTN_ERR_TOO_LARGE: return "sizes too large for the launch grid or 64-bit offsets";
    case ATTN_ERR_UNSUPPORTED_GROUP: return "unsupported grouping: at most 16 query heads per KV head in decode";
    case ATTN_ERR_LAUNCH: return "kernel launch or graph operation failed (HIP runtime error)";
    case ATTN_ERR_INVALID_SCALE: return "invalid scale: it must be a finite positive number";
    case ATTN_ERR_SCRATCH_TOO_SMALL:
      return "the call needs more than the library's fixed decode scratch (ATTN_DECODE_SCRATCH_BYTES); "
             "use paged_attn_decode with a caller-supplied workspace";
    default: return "unknown status code";
  }
}

}  // extern "C"
