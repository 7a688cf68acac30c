/*
 * paged_attention_attn — exact attention forward and paged-KV decode for one
 * AMD Instinct MI355X (gfx950), as a C ABI.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *    library allocates nothing, frees nothing, keeps no per-call state,
 *    never synchronises the stream and never reads device data on the host
 *    (the decode-graph entry points below create and release driver graph
 *    objects, and only when asked to).
 *    Every call only enqueues kernels on `stream` (0 = the null stream) and
 *    returns; results are ready when that stream reaches them.
 *  - Tensors are dense, row-major (C order) with the shapes given below.
 *    q, k, v, o, k_cache, v_cache must be 16-byte aligned; lse, block_table,
 *    seq_lens and workspace 4-byte aligned (workspace: 16-byte).
 *  - "bf16" buffers hold IEEE bfloat16 values (2 bytes each).
 *  - A nonzero return value is an ATTN_ERR_* code describing an argument error
 *    found on the host before anything was launched, or ATTN_ERR_LAUNCH when
 *    the HIP runtime rejected a launch.  Unsupported inputs are always an
 *    error: the library has no slower fallback path.
 *  - Calls are graph-capturable: no allocation, stable argument addresses.
 *  - Outputs are deterministic: fixed reduction order, no atomics.
 */
#ifndef PAGED_ATTENTION_ATTN_H_
#define PAGED_ATTENTION_ATTN_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

/* Only the functions below are exported from the shared library (it is built with hidden
 * visibility by default). */
#define ATTN_API __attribute__((visibility("default")))

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL_POINTER = 1,          /* a required pointer is NULL */
  ATTN_ERR_INVALID_SHAPE = 2,         /* negative size, H or Hkv < 1, H % Hkv != 0 */
  ATTN_ERR_UNSUPPORTED_HEAD_DIM = 3,  /* d not in {64, 128} */
  ATTN_ERR_UNSUPPORTED_PAGE_SIZE = 4, /* page_size != 16 */
  ATTN_ERR_WORKSPACE_TOO_SMALL = 5,   /* workspace_bytes below the required size */
  ATTN_ERR_MISALIGNED = 6,            /* a pointer breaks the alignment rule above */
  ATTN_ERR_TOO_LARGE = 7,             /* sizes overflow the launch grid, 64-bit offsets, or the
                                         2 GiB a kernel reads through one buffer resource */
  ATTN_ERR_UNSUPPORTED_GROUP = 8,     /* decode: more than 16 query heads per KV head */
  ATTN_ERR_LAUNCH = 9,                /* hipGetLastError reported a failed launch */
  ATTN_ERR_INVALID_SCALE = 10,        /* scale is not a finite positive number */
  ATTN_ERR_SCRATCH_TOO_SMALL = 11     /* paged_attn_decode_no_alloc: the call needs more workspace
                                         than ATTN_DECODE_SCRATCH_BYTES */
};

/*
 * attn_fwd — exact scaled dot-product attention forward, bf16 in/out.
 *
 * Computes O = softmax(scale * Q K^T + M) V with M = 0 (causal == 0) or the
 * causal mask (causal != 0: key j is visible to query i iff j <= i), and the
 * per-row log-sum-exp LSE_i = ln sum_j exp(scale * q_i . k_j + M_ij).
 * ("Fast Attention Kernels and Operator Fusion", section "FlashAttention-Style
 * Kernels", for the formula; the score matrix is never written to memory.)
 *
 *   q   [B, H,   N, d] bf16      k, v [B, Hkv, N, d] bf16
 *   o   [B, H,   N, d] bf16 (written, rounded to nearest even)
 *   lse [B, H,   N]    fp32 (written; may be NULL to skip)
 * Query head h reads KV head h / (H / Hkv) (grouped-query attention; H must
 * be a multiple of Hkv).  d must be 64 or 128; scale must be finite and
 * positive (1/sqrt(d) in the pages' formula).  One batch entry's K or V head,
 * N * d * 2 bytes, must stay below 2 GiB (ATTN_ERR_TOO_LARGE).  B == 0 or N == 0
 * is a valid empty call (pointers are then not checked and may be NULL).
 * Arithmetic: bf16 products, fp32 accumulation and softmax; the
 * probabilities are rounded to bf16 before the product with V.
 */
ATTN_API int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N, int d,
             int causal, float scale, hipStream_t stream);

/*
 * attn_fwd_window — causal attention with a sliding window and global tokens,
 * bf16 in/out: the block-sparse pattern of "Kernel Fusion and Custom
 * Kernels", section "4. FlashInfer" (a Longformer-style sliding window plus
 * global tokens), under the causal mask.  Key j is visible to query i iff
 * j <= i and (i - j < window or j < n_global).  Key tiles that hold no visible
 * key (between the global tokens and the left edge of a query tile's window)
 * are never read.  Shapes, layouts, scale rules, GQA mapping, LSE and the
 * arithmetic are those of attn_fwd; window must be >= 1 and n_global >= 0
 * (ATTN_ERR_INVALID_SHAPE otherwise).  window >= N is the plain causal mask.
 */
ATTN_API int attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N,
                    int d, int window, int n_global, float scale, hipStream_t stream);

/*
 * attn_fwd_f32 — the same operation with fp32 inputs, outputs and arithmetic
 * throughout (no reduced-precision matrix instructions): the attention of
 * "Fast Attention Kernels and Operator Fusion", section "FlashAttention-Style
 * Kernels", tiled with the online softmax of "Kernel Fusion and Custom
 * Kernels", section "3. FlashAttention: The Milestone of Fusion" (v1), so the
 * score matrix is never written to memory.  Shapes, masking, head grouping and
 * LSE as for attn_fwd; d must be 64 or 128.  One work item per query row: this
 * is the exactness reference of the family, not a throughput path.
 */
ATTN_API int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int Hkv, int N,
                 int d, int causal, float scale, hipStream_t stream);

/*
 * attn_fwd_fp8 — attn_fwd with FP8 operands: Q, K and V in OCP E4M3 (1 byte
 * each; bias 7, no infinities, largest 448) with per-tensor scales, the FP8
 * path of FlashAttention v3 ("Kernel Fusion and Custom Kernels", section "3.
 * FlashAttention: The Milestone of Fusion").  The inputs are q_scale * Q,
 * k_scale * K and v_scale * V; both products use the 8-bit matrix
 * instructions, with fp32 accumulation and softmax.  The probabilities are
 * scaled by 2^4 (so those down to 2^-10 of the row's running maximum stay in
 * E4M3's normal range) and rounded to E4M3 before the product with V
 * (relative error up to 2^-4 each); O is divided by the sum of the same
 * rounded probabilities, so it is a weighted mean of V rows (identical rows
 * come back unchanged) and differs from exact attention of the scaled
 * inputs by at most about 2^-4 * sum_j p_ij |v_j - O_i| per element.  LSE
 * uses the unrounded probabilities and is as precise as attn_fwd's, up to
 * the 8-bit matrix instruction's accumulation error in the scores.
 *
 *   q    [B, H, N, d] E4M3
 *   k    [B, Hkv, N, d] E4M3
 *   v_t  [B, Hkv, d, N] E4M3 — V transposed (keys contiguous)
 *   o    [B, H, N, d] bf16 (written)
 *   lse  [B, H, N] fp32 (written; may be NULL)
 * N must be a multiple of 16; scale and the three tensor scales finite and
 * positive; other rules as attn_fwd.
 */
ATTN_API int attn_fwd_fp8(const void* q, const void* k, const void* v_t, void* o, float* lse, int B, int H, int Hkv, int N,
                 int d, int causal, float scale, float q_scale, float k_scale, float v_scale, hipStream_t stream);

/*
 * paged_prefill — chunked prefill over a paged KV cache, appending the chunk.
 * A batch of sequences each brings a chunk of new tokens; sequence s already
 * holds ctx_lens[s] tokens in the paged cache ("Fast Attention Kernels and
 * Operator Fusion", section "Paged Attention Kernels").  In one launch the
 * chunk's keys and values are appended to the cache at positions ctx_lens[s],
 * ctx_lens[s] + 1, ... (the append operation listed in "Kernel Fusion and
 * Custom Kernels", section "4. FlashInfer"; the KV-cache update fused into the
 * attention pass, as in the fusion list of "Fast Attention Kernels and
 * Operator Fusion") and chunk query i, at position ctx_lens[s] + i, attends
 * over positions 0 .. ctx_lens[s] + i of its sequence (the causal mask aligned
 * at the end: a one-token chunk is a decode step, a chunk without context is
 * causal prefill).
 *
 *   q           [T, H, d] bf16 — the chunks' queries, back to back: sequence s
 *               owns rows q_start[s] .. q_start[s+1]-1
 *   k_new       [T, Hkv, d] bf16 — the same tokens' keys
 *   v_new       [T, Hkv, d] bf16 — the same tokens' values
 *   k_cache     [num_pages, page_size, Hkv, d] bf16 — read (context) and written (append)
 *   v_cache     [num_pages, page_size, Hkv, d] bf16 — read (context) and written (append)
 *   block_table [num_seqs, max_pages_per_seq] int32 — physical page ids; must
 *               already cover positions up to ctx_lens[s] + chunk length - 1
 *   ctx_lens    [num_seqs] int32 — tokens already cached per sequence
 *   q_start     [num_seqs + 1] int32 — chunk row offsets (nondecreasing, q_start[0] = 0)
 *   o           [T, H, d] bf16 (written)
 *   lse         [T, H] fp32 (written; may be NULL)
 *   max_q_len   host upper bound on every chunk length (sizes the grid)
 * page_size must be 16, d 64 or 128, scale finite and positive,
 * max_pages_per_seq and num_pages at least 1; max_q_len * Hkv * d * 2 bytes (the
 * most chunk rows of k_new one sequence may own) must stay below 2 GiB
 * (ATTN_ERR_TOO_LARGE).  num_seqs == 0 or max_q_len == 0 is a valid empty call
 * (pointers may be NULL).  The caller keeps its own
 * lengths: after the call sequence s holds ctx_lens[s] + chunk length tokens.
 * Device-side rules (the length arrays and the table are never read on the
 * host): chunk lengths are at most max_q_len (rows beyond are neither computed
 * nor appended) and ctx_lens[s] + chunk length <= max_pages_per_seq *
 * page_size; a page id outside [0, num_pages) is clamped for reading (the
 * result is then unspecified) and is never written; pages one sequence
 * appends to must not be read by another in the same call.  No workspace, no
 * atomics: the result is deterministic.  Arithmetic as attn_fwd.
 */
ATTN_API int paged_prefill(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                  const int32_t* block_table, const int32_t* ctx_lens, const int32_t* q_start, void* o, float* lse,
                  int num_seqs, int H, int Hkv, int d, int page_size, int max_pages_per_seq, int num_pages,
                  int max_q_len, float scale, hipStream_t stream);

/*
 * paged_attn_decode_workspace_size — bytes of device workspace that
 * paged_attn_decode needs for these shapes (0 on invalid shapes).  The
 * workspace holds one partial (normalised O, LSE) per (page range, sequence)
 * pair, which the reduce kernel merges with the rescaling identity of the
 * online softmax ("Kernel Fusion and Custom Kernels", section "3.
 * FlashAttention: The Milestone of Fusion", v1: partial results combine by
 * rescaling with the running maxima and sums).  It is about
 * (P + num_seqs) * H * (d + 1) * 4 bytes, where P <= 32768 / H is the number
 * of equal page ranges the decode cuts the cache into: linear in num_seqs, H
 * and d, and never larger for longer sequences, so the N^2 score matrix whose
 * memory "Finding the Next One: Fusion Beyond Attention" describes as the
 * materialised path's cost is never allocated.
 */
ATTN_API size_t paged_attn_decode_workspace_size(int num_seqs, int H, int d, int page_size, int max_pages_per_seq);

/*
 * paged_attn_decode — single-query attention per sequence over a paged KV
 * cache ("Fast Attention Kernels and Operator Fusion", section "Paged
 * Attention Kernels": logical block b of sequence s lives in physical page
 * block_table[s][b]; the kernel translates every token position through it).
 *
 *   q           [num_seqs, H, d] bf16 — the query of each sequence, at its last position
 *   k_cache     [num_pages, page_size, Hkv, d] bf16
 *   v_cache     [num_pages, page_size, Hkv, d] bf16
 *   block_table [num_seqs, max_pages_per_seq] int32 — physical page ids
 *   seq_lens    [num_seqs] int32 — L_s, tokens cached for sequence s
 *   o           [num_seqs, H, d] bf16 (written)
 *   lse         [num_seqs, H] fp32 (written; may be NULL)
 *   workspace   >= paged_attn_decode_workspace_size(...) bytes, device memory
 *               the call may overwrite (split partial results); reuse is fine
 *               once the stream has passed the call.
 * Token t of sequence s is slot t % page_size of page block_table[s][t / page_size];
 * the query sees all L_s tokens (no mask).  page_size must be 16, d 64 or 128,
 * H / Hkv at most 16, scale finite and positive.  num_seqs == 0 is a valid empty call (pointers may be NULL).
 * Device-side rules (seq_lens and block_table are never read on the host):
 * entries at index >= ceil(L_s / page_size) of a table row are never read;
 * slots at or past L_s are never used (their contents, even NaN, do not
 * matter); L_s is clamped to [0, max_pages_per_seq * page_size]; a page id
 * outside [0, num_pages) is not dereferenced and its tokens are treated as
 * absent.  L_s == 0 gives O = 0 and LSE = -inf.
 * Internally: a split-KV kernel cuts the pages of all sequences, laid end to
 * end, into equal ranges (one workgroup each, independent of the length mix)
 * and writes one partial result per (range, sequence) pair to the workspace;
 * a separate reduce kernel merges them on the same stream.  Its cost per
 * workgroup includes one pass over seq_lens (num_seqs reads).
 */
ATTN_API int paged_attn_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                      const int32_t* seq_lens, void* o, float* lse, int num_seqs, int H, int Hkv, int d, int page_size,
                      int max_pages_per_seq, int num_pages, float scale, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * paged_attn_decode_no_alloc — paged_attn_decode for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments, layouts, rules and
 * results, without the workspace arguments.  Its split-KV partials go to a
 * fixed device array of ATTN_DECODE_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends; the call allocates nothing.
 * A call whose workspace (paged_attn_decode_workspace_size) would exceed that
 * size returns ATTN_ERR_SCRATCH_TOO_SMALL before anything is launched (at
 * d = 128, num_seqs * H up to about 31000 fits).  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (on different
 * streams, or from different threads) race and must be ordered by the
 * caller.  Nothing in the array needs clearing between calls.  The device
 * address of the array is looked up on the first call on each device, with
 * that device made current for the lookup (the caller's current device is
 * restored).
 */
#define ATTN_DECODE_SCRATCH_BYTES (32u << 20)
ATTN_API int paged_attn_decode_no_alloc(const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                                        int num_seqs, int H, int Hkv, int d, int page_size, int max_pages_per_seq,
                                        int num_pages, float scale, hipStream_t stream);

/*
 * paged_attn_decode_fp8 — paged_attn_decode over an FP8 KV cache: k_cache and
 * v_cache hold OCP E4M3 bytes (sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, no infinities, S.1111.111 = NaN), [num_pages, page_size, Hkv, d], and
 * the cached keys and values are those values times k_scale and v_scale (per
 * tensor).  This is the FP8 variant of "Kernel Fusion and Custom Kernels",
 * section "3. FlashAttention: The Milestone of Fusion" (v3, FP8 inputs) applied
 * to the paged cache of "Fast Attention Kernels and Operator Fusion", section
 * "Paged Attention Kernels"; it halves the bytes the decode streams.
 *   q, block_table, seq_lens, o, lse, workspace and every rule on them are those
 *   of paged_attn_decode (q bf16, o bf16, the same workspace size).
 *   k_scale, v_scale  finite and positive, else ATTN_ERR_INVALID_SCALE.
 * Each byte is turned into bf16 exactly (every finite E4M3 value is a bf16);
 * the scores use scale * k_scale, each partial output is multiplied by
 * v_scale.  Slots at or past L_s may hold anything, NaN codes included.
 */
ATTN_API int paged_attn_decode_fp8(const void* q, const void* k_cache, const void* v_cache, float k_scale, float v_scale,
                          const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse, int num_seqs,
                          int H, int Hkv, int d, int page_size, int max_pages_per_seq, int num_pages, float scale,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The decode step as a replayable graph ("Fast Attention Kernels and
 * Operator Fusion", section "Fusion and CUDA Graphs with torch.compile": a
 * graph records a fixed sequence of GPU operations and replays it with one
 * submission, which needs stable addresses and shapes; it helps most where
 * launch overhead matters, as in small-batch decode).
 *
 * attn_decode_call holds the arguments of one paged_attn_decode call (same
 * meaning, layout and rules; the stream is the graph's).  A model's decode
 * step makes one such call per layer.  kv_fp8 = 1 makes it a
 * paged_attn_decode_fp8 call instead (E4M3 caches, k_scale and v_scale under
 * that function's rules); with kv_fp8 = 0 the scales are ignored; any other
 * value is ATTN_ERR_INVALID_SHAPE.
 *
 * paged_attn_decode_graph_create — checks every call exactly as
 * paged_attn_decode does, then captures the num_calls calls in order (each a
 * split-KV kernel and a reduce kernel) on capture_stream, which must not be
 * the null stream and must not be capturing already, and instantiates the
 * graph.  Calls run one after another, so they may share a workspace.  On
 * success *graph_out receives an opaque handle owned by the caller (release
 * it with paged_attn_decode_graph_destroy); on any error *graph_out is NULL
 * and nothing stays captured.  The graph holds the pointers and sizes given
 * here: each replay reads the CURRENT contents of every q, cache, block_table
 * and seq_lens and overwrites o, lse and the workspaces, so callers update
 * those buffers in place between replays.  Creating a graph allocates host
 * and driver resources; replaying it allocates nothing.
 */
typedef struct attn_decode_call {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* o;
  float* lse;
  int num_seqs, H, Hkv, d, page_size, max_pages_per_seq, num_pages;
  float scale;
  void* workspace;
  size_t workspace_bytes;
  int kv_fp8;
  float k_scale, v_scale;
} attn_decode_call;

ATTN_API int paged_attn_decode_graph_create(const attn_decode_call* calls, int num_calls, hipStream_t capture_stream,
                                   void** graph_out);

/* paged_attn_decode_graph_launch — one replay of the captured decode calls on
 * `stream` (asynchronous, stream-ordered).  ATTN_ERR_NULL_POINTER for a NULL
 * handle, ATTN_ERR_LAUNCH if the runtime rejects the launch. */
ATTN_API int paged_attn_decode_graph_launch(void* graph, hipStream_t stream);

/* paged_attn_decode_graph_destroy — releases a handle from
 * paged_attn_decode_graph_create (NULL is accepted).  Replays already
 * enqueued are not waited for: synchronise the stream first. */
ATTN_API int paged_attn_decode_graph_destroy(void* graph);

/* attn_status_string — a static, human-readable description of a status code.
 * Unsupported inputs are reported as errors rather than served by a slower
 * path: "Finding the Next One: Fusion Beyond Attention" warns that a fused
 * kernel which silently falls back to the materialised computation loses its
 * benefit without any sign; here every such case is a nonzero status that
 * this string explains. */
ATTN_API const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTENTION_ATTN_H_ */
