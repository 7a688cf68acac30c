// Internal launchers behind the C ABI (argument checking happens in abi.hip;
// these assume validated shapes and only translate them into launches).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace paa {

// window <= 0 (or >= N) means the plain causal mask when causal is set
// Chunked prefill over a paged KV cache, appending the chunk (see paged_prefill in the C header).
hipError_t paged_prefill_bf16(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              const int* block_table, const int* ctx_lens, const int* q_start, void* o, float* lse,
                              int num_seqs, int H, int Hkv, int d, int max_pages, int num_pages, int max_q_len,
                              float scale, hipStream_t stream);
// FP8 (e4m3) Q, K and transposed V with per-tensor scales, bf16 O (see attn_fwd_fp8 in the C header).
hipError_t prefill_fp8(const void* q, const void* k, const void* vt, void* o, float* lse, int B, int H, int Hkv,
                       int N, int d, bool causal, float scale, float q_scale, float k_scale, float v_scale,
                       hipStream_t stream);
hipError_t prefill_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                        int N, int d, bool causal, int window, int n_global, float scale, hipStream_t stream);

hipError_t prefill_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int Hkv,
                       int N, int d, bool causal, float scale, hipStream_t stream);

// Decode partitions: the concatenated page list is cut into `parts` equal
// ranges, one workgroup each.  Both are functions of host-known shapes only
// (never of seq_lens).  decode_max_parts(H) bounds decode_parts(...) for every
// Hkv that divides H with at most 16 query heads per KV head.
int decode_max_parts(int H);
// One-time per-process setup of the decode kernels (no launch); done before any graph capture.
hipError_t decode_setup(int d, bool fp8);
int decode_parts(int num_seqs, int H, int Hkv, int max_pages_per_seq);

// Decode over a bf16 cache, or (fp8) over an E4M3 cache holding its values divided by k_scale, v_scale.
hipError_t paged_decode(const void* q, const void* k_cache, const void* v_cache, bool fp8, float k_scale,
                        float v_scale, const int* block_table, const int* seq_lens, void* o, float* lse, int num_seqs,
                        int H, int Hkv, int d, int max_pages_per_seq, int num_pages, float scale, float* ws_o,
                        float* ws_lse, int* ws_range, int parts, int slots, hipStream_t stream);

}  // namespace paa
