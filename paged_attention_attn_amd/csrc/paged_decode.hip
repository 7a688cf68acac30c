// Single-query attention over a paged KV cache (decode), bf16 cache and
// query, fp32 math, for gfx950.
//
// What is computed: for each sequence s, its one query per head attends over
// the seq_lens[s] cached keys/values, which live in fixed-size pages of a
// shared pool; logical block b of the sequence is physical page
// block_table[s][b] ("Fast Attention Kernels and Operator Fusion", section
// "Paged Attention Kernels": the kernel translates every logical position
// through the table, since neighbouring tokens need not be adjacent in memory).
// Decode reads the whole cache for one query row, so the work is bound by HBM
// reads of K and V (same page, section "FlashAttention-Style Kernels", on why
// decode differs from prefill).
//
// Two kernels, stream-ordered, no host synchronisation:
//  1. decode_partial: one workgroup per (sequence, split of C tokens, block of
//     KV heads); one wave per KV head handles all query heads of its group.
//     Per chunk of 2 pages (32 tokens) it reads K straight into the MFMA A
//     layout, stages V through wave-private LDS for transposed reads, and
//     keeps a running max / sum / rescaled output (the online softmax of
//     "Kernel Fusion and Custom Kernels", section 3).  It writes the split's
//     normalised output and its log-sum-exp to a workspace.
//  2. decode_reduce: merges the splits of each (sequence, head) with the same
//     rescaling identity: weights exp(LSE_c - max LSE).
//
// Bounds: pages past ceil(L / page_size) are never read; slots at or past L
// (the unused tail of the last page) are masked by index and their V rows are
// replaced by zeros before the MFMA, so whatever the pool holds there (NaN in
// the tests) never reaches the result.  A page id outside [0, num_pages) is
// never dereferenced: its tokens count as masked.

#include "device_common.hpp"
#include "launch.hpp"

namespace paa {

namespace {

constexpr int kPage = 16;         // tokens per page (the ABI accepts only 16)
constexpr int kChunkTokens = 32;  // 2 pages per MFMA k-step over tokens

template <int D>
struct DecodeLds {
  static constexpr int kStrideV = D + 16;  // bf16 elements; rows 8 dwords apart in bank space
  static constexpr int kPerWave = kChunkTokens * kStrideV;
};

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int* bt;
  const int* lens;
  float* ws_o;
  float* ws_lse;
  int H, Hkv, group, max_pages, num_pages, split_tokens, max_splits, waves;
  float scale, scale_log2;
};

__device__ __forceinline__ int seq_len_clamped(const DecodeArgs& a, int s) {
  int L = a.lens[s];
  L = L < 0 ? 0 : L;
  const int cap = a.max_pages * kPage;
  return L > cap ? cap : L;
}

template <int D>
__global__ __launch_bounds__(512) void decode_partial_kernel(DecodeArgs a) {
  constexpr int kKSteps = D / 32;          // 16x16x32 k-steps over d for the scores
  constexpr int kDBlocks = D / 16;         // 16-wide d blocks of the output
  constexpr int kChunksPerRow = D / 8;     // 16-byte chunks per V row
  constexpr int kVChunks = kPage * kChunksPerRow / 64;  // per lane per page
  using Lds = DecodeLds<D>;

  extern __shared__ __attribute__((aligned(16))) uint16_t lds_raw[];
  const int wave = threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  const int c16 = lane / 16;  // 16-lane group
  const int r16 = lane % 16;  // token row (K loads) / head column (scores)
  PAA_LDS uint16_t* vl = (PAA_LDS uint16_t*)lds_raw + wave * Lds::kPerWave;

  const int split = blockIdx.x;
  const int s = blockIdx.y;
  const int g = blockIdx.z * a.waves + wave;
  const int L = seq_len_clamped(a, s);
  const int t_begin = split * a.split_tokens;
  if (t_begin >= L) return;  // uniform across the workgroup
  const int t_end = min(L, t_begin + a.split_tokens);

  const size_t tok_stride = (size_t)a.Hkv * D;  // elements between consecutive slots
  const int* bt_row = a.bt + (size_t)s * a.max_pages;

  // Q^T fragment (B operand): head g*group + r16 (zero beyond the group), d = 32t + 8*c16 + 0..7
  const int head = g * a.group + r16;
  const bool head_ok = r16 < a.group;
  u32x4_t qf[kKSteps];
#pragma unroll
  for (int t = 0; t < kKSteps; ++t)
    qf[t] = head_ok ? *(const u32x4_t*)(a.q + ((size_t)s * a.H + head) * D + 32 * t + 8 * c16) : u32x4_t{0, 0, 0, 0};

  float m_run = -INFINITY;
  float l_run = 0.f;  // this lane's share of the sum for head r16
  f32x4_t acc[kDBlocks];
#pragma unroll
  for (int nb = 0; nb < kDBlocks; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int t0 = t_begin; t0 < t_end; t0 += kChunkTokens) {
    u32x4_t kf[2][kKSteps];
    u32x4_t vr[2][kVChunks];
    bool page_ok[2];
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const int tp = t0 + kPage * pp;  // first token of this page
      int pid = -1;
      if (tp < t_end) pid = bt_row[tp / kPage];
      page_ok[pp] = pid >= 0 && pid < a.num_pages;
      const uint16_t* kpage = a.kc + (size_t)(page_ok[pp] ? pid : 0) * kPage * tok_stride + (size_t)g * D;
      const uint16_t* vpage = a.vc + (size_t)(page_ok[pp] ? pid : 0) * kPage * tok_stride + (size_t)g * D;
#pragma unroll
      for (int t = 0; t < kKSteps; ++t)
        kf[pp][t] = page_ok[pp] ? *(const u32x4_t*)(kpage + r16 * tok_stride + 32 * t + 8 * c16)
                                : u32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < kVChunks; ++i) {
        const int c = lane + 64 * i;
        const int row = c / kChunksPerRow;
        const int col = (c % kChunksPerRow) * 8;
        const bool ok = page_ok[pp] && (tp + row < t_end);
        vr[pp][i] = ok ? *(const u32x4_t*)(vpage + row * tok_stride + col) : u32x4_t{0, 0, 0, 0};
      }
    }
    // stage V rows [page][slot][d] into this wave's LDS slice
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
      for (int i = 0; i < kVChunks; ++i) {
        const int c = lane + 64 * i;
        const int row = c / kChunksPerRow;
        const int col = (c % kChunksPerRow) * 8;
        *(PAA_LDS u32x4_t*)(vl + (kPage * pp + row) * Lds::kStrideV + col) = vr[pp][i];
      }

    // scores S[token][head]: lane holds tokens 4*c16 + i of each page, head r16
    f32x4_t sc[2];
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      sc[pp] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < kKSteps; ++t) sc[pp] = mfma16x16x32(kf[pp][t], qf[t], sc[pp]);
    }
    // mask slots at or past the end and every slot of a page that was not read
    float tmax = -INFINITY;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t0 + kPage * pp + 4 * c16 + i;
        if (!page_ok[pp] || tok >= t_end) sc[pp][i] = -INFINITY;
        tmax = fmaxf(tmax, sc[pp][i]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2((m_run - m_use) * a.scale_log2);
    const float neg_ms = -m_use * a.scale_log2;
    m_run = m_new;
    float p[8];
    float psum = 0.f;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[4 * pp + i] = fast_exp2(fmaf(sc[pp][i], a.scale_log2, neg_ms));
        psum += p[4 * pp + i];
      }
    l_run = l_run * alpha + psum;
    const u32x4_t pf = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                        pack_bf16x2(p[6], p[7])};

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // O^T[d][head] += V^T P^T: logical token k = 8*c16 + j is slot 4*c16 + j%4 of page j/4
#pragma unroll
    for (int nb = 0; nb < kDBlocks; ++nb) {
      const int row = 4 * c16 + r16 / 4;
      const int col = 16 * nb + 4 * (r16 % 4);
      const u32x2_t lo = lds_read_tr16(vl + row * Lds::kStrideV + col);
      const u32x2_t hi = lds_read_tr16(vl + (kPage + row) * Lds::kStrideV + col);
      const u32x4_t vf = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[nb][i] *= alpha;
      acc[nb] = mfma16x16x32(vf, pf, acc[nb]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // split result for head r16: normalised output and log-sum-exp
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (head_ok) {
    // a split whose pages were all rejected has no visible key: zero output, LSE = -inf
    const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const size_t base = ((size_t)s * a.H + head) * a.max_splits + split;
    float* wo = a.ws_o + base * D;
#pragma unroll
    for (int nb = 0; nb < kDBlocks; ++nb) {
      f32x4_t w = acc[nb] * inv_l;
      *(f32x4_t*)(wo + 16 * nb + 4 * c16) = w;
    }
    if (c16 == 0) a.ws_lse[base] = l_tot > 0.f ? a.scale * m_run + __logf(l_tot) : -INFINITY;
  }
}

// One wave per (sequence, head): merge the splits of that row.
template <int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a, uint16_t* o, float* lse, int rows) {
  constexpr int kPerLane = D / 64;
  const int row = blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (row >= rows) return;
  const int s = row / a.H;
  const int L = seq_len_clamped(a, s);
  const int n = (L + a.split_tokens - 1) / a.split_tokens;
  const size_t base = (size_t)row * a.max_splits;
  float mx = -INFINITY;
  for (int c = 0; c < n; ++c) mx = fmaxf(mx, a.ws_lse[base + c]);
  float wsum = 0.f;
  float out[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) out[i] = 0.f;
  for (int c = 0; c < n && mx != -INFINITY; ++c) {
    const float lc = a.ws_lse[base + c];
    if (lc == -INFINITY) continue;  // split without a visible key
    const float w = __expf(lc - mx);
    wsum += w;
    const float* src = a.ws_o + (base + c) * D;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) out[i] = fmaf(w, src[lane + 64 * i], out[i]);
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  uint16_t* orow = o + (size_t)row * D;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const uint32_t w = pack_bf16x2(out[i] * inv, 0.f);
    orow[lane + 64 * i] = (uint16_t)(w & 0xffffu);
  }
  if (lse != nullptr && lane == 0) lse[row] = wsum > 0.f ? mx + __logf(wsum) : -INFINITY;
}

template <int D>
hipError_t launch_decode(DecodeArgs a, uint16_t* o, float* lse, int num_seqs, hipStream_t stream) {
  int waves = 1;
  for (int w = 8; w >= 1; --w)
    if (a.Hkv % w == 0) { waves = w; break; }
  a.waves = waves;
  const int lds_bytes = waves * DecodeLds<D>::kPerWave * 2;
  // allow the largest slice (8 waves) once; thread-safe static initialisation
  static const hipError_t attr = hipFuncSetAttribute((const void*)decode_partial_kernel<D>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     8 * DecodeLds<D>::kPerWave * 2);
  if (attr != hipSuccess) return attr;
  dim3 grid1((unsigned)a.max_splits, (unsigned)num_seqs, (unsigned)(a.Hkv / waves));
  hipLaunchKernelGGL(decode_partial_kernel<D>, grid1, dim3(64 * waves), lds_bytes, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = num_seqs * a.H;
  hipLaunchKernelGGL(decode_reduce_kernel<D>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, a, o, lse, rows);
  return hipGetLastError();
}

}  // namespace

int decode_split_tokens(int num_seqs, int page_size, int max_pages_per_seq) {
  const long long max_len = (long long)page_size * max_pages_per_seq;
  int c = 256;
  // shorter splits when there would be too few workgroups to fill 256 CUs
  while (c > kChunkTokens && (long long)num_seqs * ((max_len + c - 1) / c) < 1024) c /= 2;
  return c;
}

int decode_max_splits(int num_seqs, int page_size, int max_pages_per_seq) {
  const long long max_len = (long long)page_size * max_pages_per_seq;
  const int c = decode_split_tokens(num_seqs, page_size, max_pages_per_seq);
  return (int)((max_len + c - 1) / c);
}

hipError_t paged_decode_bf16(const void* q, const void* k_cache, const void* v_cache, const int* block_table,
                             const int* seq_lens, void* o, float* lse, int num_seqs, int H, int Hkv, int d,
                             int page_size, int max_pages_per_seq, int num_pages, float scale, float* ws_o,
                             float* ws_lse, int split_tokens, int max_splits, hipStream_t stream) {
  (void)page_size;
  DecodeArgs a{};
  a.q = (const uint16_t*)q;
  a.kc = (const uint16_t*)k_cache;
  a.vc = (const uint16_t*)v_cache;
  a.bt = block_table;
  a.lens = seq_lens;
  a.ws_o = ws_o;
  a.ws_lse = ws_lse;
  a.H = H;
  a.Hkv = Hkv;
  a.group = H / Hkv;
  a.max_pages = max_pages_per_seq;
  a.num_pages = num_pages;
  a.split_tokens = split_tokens;
  a.max_splits = max_splits;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  if (d == 64) return launch_decode<64>(a, (uint16_t*)o, lse, num_seqs, stream);
  return launch_decode<128>(a, (uint16_t*)o, lse, num_seqs, stream);
}

}  // namespace paa
