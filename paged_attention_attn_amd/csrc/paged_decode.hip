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
//  1. decode_partial: the pages of all sequences, laid end to end, are cut
//     into `parts` equal ranges (one per workgroup, whatever the length mix,
//     so every workgroup streams the same number of bytes).  A workgroup has
//     one wave per KV head; each wave walks its range two pages (32 tokens)
//     at a time, keeps a running max / sum / rescaled output for the query
//     heads of its group (the online softmax of "Kernel Fusion and Custom
//     Kernels", section 3) and, where its range leaves a sequence, writes that
//     sequence's partial output and log-sum-exp to the workspace.  The output
//     is divided by the sum of the probabilities as rounded to bf16 for P.V
//     (the weights its numerator used), the LSE uses their fp32 sum.
//     The next two pages are loaded while the current two are computed; K is
//     loaded straight into the MFMA A layout and V is staged through
//     wave-private LDS for transposed reads.  Every K and V line of the cache
//     is read exactly once per call, so the loads carry the non-temporal hint
//     (streamed, not kept in the caches): measured, the partial kernel went
//     from 206 to 184 us on the 64-sequence workload.
//  2. decode_reduce: merges the partials of each (sequence, head) with the
//     same rescaling identity, weights exp(LSE_c - max LSE).
//
// A partial of sequence s written by workgroup (range) r goes to workspace
// slot s + r: the ranges of one sequence are consecutive and the next
// sequence starts in the range where this one ends, so slots never collide
// and there are at most parts + num_seqs of them.  The workgroups holding a
// sequence's first and last page also record those two slots for the reduce.
//
// Bounds: pages past ceil(L / page_size) are never read; slots at or past L
// (the unused tail of the last page) are masked by index and their V rows are
// replaced by zeros before the MFMA, so whatever the pool holds there (NaN in
// the tests) never reaches the result.  A page id outside [0, num_pages) is
// never dereferenced: its tokens count as masked.

#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace paa {

namespace {

constexpr int kPage = 16;         // tokens per page (the ABI accepts only 16)
constexpr int kStepTokens = 32;   // 2 pages per MFMA k-step over tokens
constexpr int kMaxWaves = 8;      // KV heads (waves) per workgroup
constexpr int kTargetWaves = 2048;  // waves per launch: 8 per CU on 256 CUs
constexpr int kReduceSplitSlots = 16;  // partials per row from which the reduce gives a row 4 waves

template <int D>
struct DecodeLds {
  static constexpr int kStrideV = D + 16;  // bf16 elements; rows 8 dwords apart in bank space
  static constexpr int kPerWave = kStepTokens * kStrideV;
};

struct DecodeArgs {
  const uint16_t* q;
  const void* kc;  // bf16, or E4M3 bytes for the FP8 cache
  const void* vc;
  const int* bt;
  const int* lens;
  float* ws_o;     // [slots, H, D] partial outputs (normalised)
  float* ws_lse;   // [slots, H] partial log-sum-exp
  int* ws_range;   // [S, 2] first and last slot of each sequence, then the total page count
  uint16_t* o;
  float* lse;
  int S, H, Hkv, group, max_pages, num_pages, parts, slots, waves;
  float scale, scale_log2;  // the softmax scale (times k_scale for the FP8 cache)
  float vscale;             // factor on the output: v_scale for the FP8 cache, 1 otherwise
};

__device__ __forceinline__ int seq_len_clamped(const DecodeArgs& a, int s) {
  int L = a.lens[s];
  L = L < 0 ? 0 : L;
  const int cap = a.max_pages * kPage;
  return L > cap ? cap : L;
}

__device__ __forceinline__ int pages_of(int L) { return (L + kPage - 1) / kPage; }

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

// Inclusive prefix sum across the workgroup (nthreads <= 512); `red` holds kMaxWaves ints.
__device__ __forceinline__ int block_inclusive_scan(int v, int* red) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int u = __shfl_up(v, m);
    if (lane >= m) v += u;
  }
  if (lane == 63) red[wave] = v;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += red[w];
  __syncthreads();
  return v + before;
}

// First global page of range r when `total` pages are cut into `parts` ranges.
__device__ __forceinline__ int range_begin(int r, long long total, int parts) {
  return (int)(((long long)r * total + parts - 1) / parts);
}

// A step: up to two pages of one sequence.  Every field is wave-uniform.
struct Step {
  int s;      // sequence
  int p;      // local index of the first page
  int np;     // pages in the step: 1 or 2 (0 = the range is exhausted)
  int L;      // tokens of sequence s
  int n;      // pages of sequence s
  bool first; // first step of this range's segment of sequence s
  bool last;  // last step of that segment
  int pid[2]; // physical pages of the step (filled when its loads are issued; -1 = none)
};

// Walks the global page range [x, end) of one workgroup, sequence by sequence.
struct Walker {
  int s, c, n, L;  // current sequence, its first global page, its page count and length
  int x, end;      // next global page, end of the range

  __device__ Step next(const DecodeArgs& a) {
    Step st;
    st.np = 0;
    if (x >= end) return st;
    bool fresh = false;
    while (x >= c + n) {  // leave finished (or empty) sequences; x < end <= total keeps s < S
      c += n;
      if (++s >= a.S) {  // unreachable while the page counts agree with the scan; stop rather than read past
        x = end;
        return st;
      }
      L = seq_len_clamped(a, s);
      n = pages_of(L);
      fresh = true;
    }
    st.s = s;
    st.p = x - c;
    const int seg_hi = min(end, c + n) - c;
    st.np = min(2, seg_hi - st.p);
    st.L = L;
    st.n = n;
    st.first = fresh;
    st.last = st.p + st.np == seg_hi;
    x += st.np;
    return st;
  }
};

// Two E4M3 bytes (the low or high half of w, lower byte first) -> two bf16, exactly (every finite
// E4M3 value is a bf16).
template <bool HIGH>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH));
}

// Eight E4M3 bytes -> eight bf16 (an MFMA operand), in byte order.
__device__ __forceinline__ u32x4_t e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  return u32x4_t{e4m3x2_to_bf16x2<false>(lo), e4m3x2_to_bf16x2<true>(lo), e4m3x2_to_bf16x2<false>(hi),
                 e4m3x2_to_bf16x2<true>(hi)};
}

template <int D, bool FP8>
__global__ __launch_bounds__(64 * kMaxWaves) void decode_partial_kernel(DecodeArgs a) {
  constexpr int kKSteps = D / 32;          // 16x16x32 k-steps over d for the scores
  constexpr int kDBlocks = D / 16;         // 16-wide d blocks of the output
  constexpr int kChunksPerRow = D / 8;     // 16-byte bf16 chunks per V row in LDS
  // the cache as loaded: bf16, or E4M3 bytes (8 bytes of a K row per k-step, V rows in 16-byte
  // chunks of 16 values), turned into bf16 only when the step is computed
  using CacheT = std::conditional_t<FP8, uint8_t, uint16_t>;
  // K loads: bf16, 16 bytes (8 values) per lane per k-step; E4M3, 16 bytes (16 values) per lane per
  // two k-steps.  For the E4M3 cache the contraction over d is taken in a permuted order, the same
  // for K and q: k-step 2u + v, lane group c16 covers d = 16*c16 + 64*u + 8*v .. +7, so one load
  // fills two k-steps and each instruction reads 64 contiguous bytes of each of 16 rows.
  using KRaw = u32x4_t;
  constexpr int kKLoads = FP8 ? kKSteps / 2 : kKSteps;
  constexpr int kRawPerRow = FP8 ? D / 16 : kChunksPerRow;  // 16-byte loads per V row
  constexpr int kVRaw = kPage * kRawPerRow / 64;            // per lane per page
  static_assert(kPage * kRawPerRow % 64 == 0, "V loads split evenly over the lanes");
  const CacheT* kc = (const CacheT*)a.kc;
  const CacheT* vc = (const CacheT*)a.vc;
  using Lds = DecodeLds<D>;

  extern __shared__ __attribute__((aligned(16))) uint16_t lds_raw[];
  __shared__ int red[kMaxWaves];
  __shared__ int found[2];
  const int wave = threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  const int nthreads = 64 * a.waves;
  const int c16 = lane / 16;  // 16-lane group
  const int r16 = lane % 16;  // token row (K loads) / head column (scores)
  PAA_LDS uint16_t* vl = (PAA_LDS uint16_t*)lds_raw + wave * Lds::kPerWave;

  // ---- this workgroup's range of the concatenated page list ----
  __shared__ int total_sh;
  if (threadIdx.x == 0) found[0] = -1;
  long long total;
  int start, end;
  const int r = blockIdx.x;
  if (a.S <= nthreads) {
    // one scan gives both the total and the sequence holding the range's first page
    const int s = threadIdx.x;
    const int v = s < a.S ? pages_of(seq_len_clamped(a, s)) : 0;
    const int incl = block_inclusive_scan(v, red);
    if (threadIdx.x == nthreads - 1) total_sh = incl;
    __syncthreads();
    total = total_sh;
    start = range_begin(r, total, a.parts);
    end = range_begin(r + 1, total, a.parts);
    if (v > 0 && incl - v <= start && start < incl) {
      found[0] = s;
      found[1] = incl - v;
    }
    __syncthreads();
  } else {
    int part_pages = 0;
    for (int s = threadIdx.x; s < a.S; s += nthreads) part_pages += pages_of(seq_len_clamped(a, s));
    part_pages = wave_sum(part_pages);
    if (lane == 0) red[wave] = part_pages;
    __syncthreads();
    total = 0;
    for (int w = 0; w < a.waves; ++w) total += red[w];
    __syncthreads();
    start = range_begin(r, total, a.parts);
    end = range_begin(r + 1, total, a.parts);
    // the sequence holding global page `start`, and that sequence's first global page
    int carry = 0;
    for (int base = 0; base < a.S && start < end; base += nthreads) {
      const int s = base + threadIdx.x;
      const int v = s < a.S ? pages_of(seq_len_clamped(a, s)) : 0;
      const int incl = block_inclusive_scan(v, red);
      if (v > 0 && carry + incl - v <= start && start < carry + incl) {
        found[0] = s;
        found[1] = carry + incl - v;
      }
      if (threadIdx.x == nthreads - 1) red[0] = incl;
      __syncthreads();
      carry += red[0];
      const bool done = found[0] >= 0;
      __syncthreads();
      if (done) break;
    }
  }
  if (r == 0 && blockIdx.y == 0 && threadIdx.x == 0) a.ws_range[2 * a.S] = (int)total;  // for the reduce
  if (start >= end) return;  // an empty range (more ranges than pages); uniform across the workgroup
  const int s0 = found[0];
  const int c0 = found[1];

  const int g = blockIdx.y * a.waves + wave;  // KV head of this wave
  const int head = g * a.group + r16;         // query head of this lane's score column
  const bool head_ok = r16 < a.group;
  const size_t tok_stride = (size_t)a.Hkv * D;  // elements between consecutive slots of a page

  Walker wk;
  wk.s = s0;
  wk.c = c0;
  wk.L = seq_len_clamped(a, s0);
  wk.n = pages_of(wk.L);
  wk.x = start;
  wk.end = end;

  // block-table window: lane j holds bt[bt_s][bt_base + j]
  int bt_vec = -1, bt_s = -1, bt_base = 0;
  auto page_id = [&](const Step& st, int k) -> int {  // physical page of local page st.p + k
    const int lp = st.p + k;
    if (st.s != bt_s || lp < bt_base || lp >= bt_base + 64) {
      bt_s = st.s;
      bt_base = lp;
      const int j = lp + lane;
      bt_vec = j < st.n ? a.bt[(size_t)st.s * a.max_pages + j] : -1;
    }
    return __builtin_amdgcn_readlane(bt_vec, lp - bt_base);
  };

  KRaw kf[2][kKLoads], kn[2][kKLoads];
  u32x4_t vr[2][kVRaw], vn[2][kVRaw], qf[kKSteps], qn[kKSteps];

  // loads of one step into (k, v, q): K in the MFMA A layout, V rows as 16-byte chunks
  auto issue = [&](Step& st, KRaw (&k)[2][kKLoads], u32x4_t (&v)[2][kVRaw], u32x4_t (&qq)[kKSteps]) {
    if (st.first) {
#pragma unroll
      for (int t = 0; t < kKSteps; ++t)
        qq[t] = head_ok ? *(const u32x4_t*)(a.q + ((size_t)st.s * a.H + head) * D +
                                            (FP8 ? 16 * c16 + 64 * (t / 2) + 8 * (t % 2) : 32 * t + 8 * c16))
                        : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const int tp = (st.p + pp) * kPage;  // first token of this page
      const int pid = pp < st.np ? page_id(st, pp) : -1;
      st.pid[pp] = pid;
      const bool ok = pid >= 0 && pid < a.num_pages;
      const CacheT* kpage = kc + (size_t)(ok ? pid : 0) * kPage * tok_stride + (size_t)g * D;
      const CacheT* vpage = vc + (size_t)(ok ? pid : 0) * kPage * tok_stride + (size_t)g * D;
#pragma unroll
      for (int t = 0; t < kKLoads; ++t)
        k[pp][t] = ok ? __builtin_nontemporal_load(
                            (const KRaw*)(kpage + r16 * tok_stride + (FP8 ? 16 * c16 + 64 * t : 32 * t + 8 * c16)))
                      : KRaw{};
#pragma unroll
      for (int i = 0; i < kVRaw; ++i) {
        const int c = lane + 64 * i;
        const int row = c / kRawPerRow;
        const int col = (c % kRawPerRow) * (FP8 ? 16 : 8);
        v[pp][i] = (ok && tp + row < st.L)
                       ? __builtin_nontemporal_load((const u32x4_t*)(vpage + row * tok_stride + col))
                       : u32x4_t{0, 0, 0, 0};
      }
    }
  };

  float m_run = -INFINITY;
  float l_run = 0.f;   // this lane's share of the sum for head r16
  float lr_run = 0.f;  // ... and of the same probabilities as rounded to bf16 for P.V (O is divided by it)
  f32x4_t acc[kDBlocks];

  Step cur = wk.next(a);
  cur.first = true;
  issue(cur, kf, vr, qf);
  int seg_lo = 0;  // local page where the current segment began

  while (cur.np > 0) {
    Step nxt = wk.next(a);
    if (cur.first) {
      seg_lo = cur.p;
      m_run = -INFINITY;
      l_run = 0.f;
      lr_run = 0.f;
#pragma unroll
      for (int nb = 0; nb < kDBlocks; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // next step's loads are in flight while this one is computed
    if (nxt.np > 0) issue(nxt, kn, vn, qn);
    // stage V rows [page][slot][d] of the current step into this wave's LDS slice
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
      for (int i = 0; i < kVRaw; ++i) {
        const int c = lane + 64 * i;
        const int row = c / kRawPerRow;
        PAA_LDS uint16_t* dst = vl + (kPage * pp + row) * Lds::kStrideV;
        if constexpr (FP8) {  // 16 values -> two 16-byte bf16 chunks
          const u32x4_t w = vr[pp][i];
          const int col = (c % kRawPerRow) * 16;
          *(PAA_LDS u32x4_t*)(dst + col) = e4m3x8_to_bf16x8(w[0], w[1]);
          *(PAA_LDS u32x4_t*)(dst + col + 8) = e4m3x8_to_bf16x8(w[2], w[3]);
        } else {
          *(PAA_LDS u32x4_t*)(dst + (c % kRawPerRow) * 8) = vr[pp][i];
        }
      }

    // scores S[token][head]: lane holds tokens 4*c16 + i of each page, head r16
    f32x4_t sc[2];
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      sc[pp] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < kKSteps; ++t) {
        u32x4_t kb;
        if constexpr (FP8)
          kb = e4m3x8_to_bf16x8(kf[pp][t / 2][2 * (t % 2)], kf[pp][t / 2][2 * (t % 2) + 1]);
        else
          kb = kf[pp][t];
        sc[pp] = mfma16x16x32(kb, qf[t], sc[pp]);
      }
    }
    // mask slots at or past the end, pages outside the step and pages that were not read
    float tmax = -INFINITY;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const bool ok = cur.pid[pp] >= 0 && cur.pid[pp] < a.num_pages;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = (cur.p + pp) * kPage + 4 * c16 + i;
        if (!ok || tok >= cur.L) sc[pp][i] = -INFINITY;
        tmax = fmaxf(tmax, sc[pp][i]);
      }
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
    lr_run = lr_run * alpha + (add_bf16_pair(pf[0], add_bf16_pair(pf[1], 0.f)) +
                               add_bf16_pair(pf[2], add_bf16_pair(pf[3], 0.f)));

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

    if (cur.last) {
      // this range's partial of sequence cur.s for head r16: normalised output and log-sum-exp
      float l_tot = l_run + __shfl_xor(l_run, 16);
      l_tot += __shfl_xor(l_tot, 32);
      float lr_tot = lr_run + __shfl_xor(lr_run, 16);
      lr_tot += __shfl_xor(lr_tot, 32);
      const int slot = cur.s + blockIdx.x;
      if (head_ok) {
        // a segment whose pages were all rejected has no visible key: zero output, LSE = -inf
        const float inv_l = lr_tot > 0.f ? a.vscale / lr_tot : 0.f;
        const size_t base = (size_t)slot * a.H + head;
        float* wo = a.ws_o + base * D;
#pragma unroll
        for (int nb = 0; nb < kDBlocks; ++nb) {
          f32x4_t w = acc[nb] * inv_l;
          *(f32x4_t*)(wo + 16 * nb + 4 * c16) = w;
        }
        if (c16 == 0) a.ws_lse[base] = l_tot > 0.f ? a.scale * m_run + __logf(l_tot) : -INFINITY;
      }
      if (g == 0 && lane == 0) {
        if (seg_lo == 0) a.ws_range[2 * cur.s] = slot;  // this range holds page 0
        if (cur.p + cur.np == cur.n) a.ws_range[2 * cur.s + 1] = slot;  // ... and/or the last page
      }
    }
    // the step that begins a segment resets the state, whatever the previous one was
    cur = nxt;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
#pragma unroll
      for (int t = 0; t < kKLoads; ++t) kf[pp][t] = kn[pp][t];
#pragma unroll
      for (int i = 0; i < kVRaw; ++i) vr[pp][i] = vn[pp][i];
    }
    if (cur.first) {
#pragma unroll
      for (int t = 0; t < kKSteps; ++t) qf[t] = qn[t];
    }
  }
}

// WPR waves per (sequence, head) merge the partials of that row.  The
// sequence's partials sit in slots first..last; slot j came from range j - s,
// and a range with no pages (possible when there are more ranges than pages)
// wrote nothing, so it is skipped.  Every wave takes the max LSE over all the
// row's slots; with WPR > 1 the slots are then cut into WPR consecutive
// pieces, one per wave, and the waves' weighted sums are added in LDS in wave
// order (a fixed order: the result does not depend on timing).  Several waves
// per row pay off when there are few rows and many slots per row (a small
// batch of long sequences), where one wave would walk its slots one round
// trip at a time.
template <int D, int WPR>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a) {
  static_assert(WPR == 1 || WPR == 4, "one row per wave, or one row per workgroup");
  constexpr int kPerLane = D / 64;
  constexpr int kBatch = 8;  // partial rows loaded together
  const int wave = threadIdx.x / 64;
  const int row = blockIdx.x * (4 / WPR) + wave / WPR;
  const int piece = wave % WPR;
  const int lane = threadIdx.x % 64;
  if (row >= a.S * a.H) return;  // with WPR == 4 the whole workgroup leaves together
  const int s = row / a.H;
  const int h = row % a.H;
  const int L = seq_len_clamped(a, s);
  float out[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) out[i] = 0.f;
  float wsum = 0.f, mx = -INFINITY;
  if (L > 0) {
    const long long total = a.ws_range[2 * a.S];
    // clamped so that a stale or damaged range can never address outside the workspace
    const int first = min(max(a.ws_range[2 * s], 0), a.slots - 1);
    const int last = min(max(a.ws_range[2 * s + 1], first), a.slots - 1);
    const int n = last - first + 1;
    const int per = (n + WPR - 1) / WPR;
    const int lo = min(piece * per, n);
    const int hi = min(lo + per, n);
    auto lse_of = [&](int j) -> float {  // LSE of slot first + j, -inf for an empty range
      const int r = first + j - s;
      if (r < 0 || r >= a.parts || range_begin(r, total, a.parts) >= range_begin(r + 1, total, a.parts))
        return -INFINITY;
      return a.ws_lse[(size_t)(first + j) * a.H + h];
    };
    // this wave's first 64 LSEs and first kBatch partial rows are loaded in the same round trip as the
    // LSEs of the max below
    const float lse_lo = lo + lane < hi ? lse_of(lo + lane) : -INFINITY;
    float ov[kBatch][kPerLane];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float* src = a.ws_o + ((size_t)(first + min(lo + u, n - 1)) * a.H + h) * D;
#pragma unroll
      for (int i = 0; i < kPerLane; ++i) ov[u][i] = src[lane + 64 * i];
    }
    for (int c0 = 0; c0 < n; c0 += 64) mx = fmaxf(mx, c0 + lane < n ? lse_of(c0 + lane) : -INFINITY);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
    for (int c0 = lo; c0 < hi && mx != -INFINITY; c0 += 64) {
      const int cnt = min(64, hi - c0);
      const float lc = c0 == lo ? lse_lo : (lane < cnt ? lse_of(c0 + lane) : -INFINITY);
      const float w = lc == -INFINITY ? 0.f : __expf(lc - mx);  // a partial without a visible key weighs 0
      float ws = w;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) ws += __shfl_xor(ws, m);
      wsum += ws;
      // a slot whose weight is 0 (empty range, or no visible key) may hold anything, so its values
      // are replaced by 0 rather than multiplied by 0
      int j0 = 0;
      if (c0 == lo) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const float wj = u < cnt ? __shfl(w, u) : 0.f;
#pragma unroll
          for (int i = 0; i < kPerLane; ++i) out[i] = fmaf(wj, wj == 0.f ? 0.f : ov[u][i], out[i]);
        }
        j0 = kBatch;
      }
      for (; j0 < cnt; j0 += kBatch) {
        float v[kBatch][kPerLane], wj[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int j = min(j0 + u, cnt - 1);
          wj[u] = j0 + u < cnt ? __shfl(w, j) : 0.f;
          const float* src = a.ws_o + ((size_t)(first + c0 + j) * a.H + h) * D;
#pragma unroll
          for (int i = 0; i < kPerLane; ++i) v[u][i] = src[lane + 64 * i];
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
#pragma unroll
          for (int i = 0; i < kPerLane; ++i) out[i] = fmaf(wj[u], wj[u] == 0.f ? 0.f : v[u][i], out[i]);
      }
    }
  }
  if constexpr (WPR > 1) {
    __shared__ float red_o[WPR][D];
    __shared__ float red_w[WPR];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) red_o[piece][lane + 64 * i] = out[i];
    if (lane == 0) red_w[piece] = wsum;
    __syncthreads();
    if (piece != 0) return;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      float acc = red_o[0][lane + 64 * i];
#pragma unroll
      for (int p = 1; p < WPR; ++p) acc += red_o[p][lane + 64 * i];
      out[i] = acc;
    }
    wsum = red_w[0];
#pragma unroll
    for (int p = 1; p < WPR; ++p) wsum += red_w[p];
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  uint16_t* orow = a.o + (size_t)row * D;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const uint32_t w = pack_bf16x2(out[i] * inv, 0.f);
    orow[lane + 64 * i] = (uint16_t)(w & 0xffffu);
  }
  if (a.lse != nullptr && lane == 0) a.lse[row] = wsum > 0.f ? mx + __logf(wsum) : -INFINITY;
}

int waves_for(int Hkv) {
  for (int w = kMaxWaves; w >= 1; --w)
    if (Hkv % w == 0) return w;
  return 1;
}

// Raise the partial kernel's dynamic LDS limit to the largest slice, once per process
// (thread-safe static initialisation).
template <int D, bool FP8>
hipError_t setup_decode() {
  static const hipError_t attr = hipFuncSetAttribute((const void*)decode_partial_kernel<D, FP8>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     kMaxWaves * DecodeLds<D>::kPerWave * 2);
  return attr;
}

template <int D, bool FP8>
hipError_t launch_decode(DecodeArgs a, hipStream_t stream) {
  a.waves = waves_for(a.Hkv);
  const int lds_bytes = a.waves * DecodeLds<D>::kPerWave * 2;
  const hipError_t attr = setup_decode<D, FP8>();
  if (attr != hipSuccess) return attr;
  dim3 grid1((unsigned)a.parts, (unsigned)(a.Hkv / a.waves));
  hipLaunchKernelGGL((decode_partial_kernel<D, FP8>), grid1, dim3(64 * a.waves), lds_bytes, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long rows = (long long)a.S * a.H;
  // slots per row average parts / S + 1: with many, a workgroup per row splits them over its 4 waves
  if (a.parts >= kReduceSplitSlots * a.S)
    hipLaunchKernelGGL((decode_reduce_kernel<D, 4>), dim3((unsigned)rows), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_reduce_kernel<D, 1>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t decode_setup(int d, bool fp8) {
  if (fp8) return d == 64 ? setup_decode<64, true>() : setup_decode<128, true>();
  return d == 64 ? setup_decode<64, false>() : setup_decode<128, false>();
}

int decode_max_parts(int H) {
  // Hkv >= H / 16 (at most 16 query heads per KV head), so kTargetWaves / Hkv <= 16 * kTargetWaves / H
  const int by_heads = (16 * kTargetWaves) / (H > 0 ? H : 1);
  return by_heads < 1 ? 1 : (by_heads > kTargetWaves ? kTargetWaves : by_heads);
}

int decode_parts(int num_seqs, int H, int Hkv, int max_pages_per_seq) {
  long long p = kTargetWaves / Hkv;
  const long long pages = (long long)num_seqs * max_pages_per_seq;
  if (p > pages) p = pages;
  if (p > decode_max_parts(H)) p = decode_max_parts(H);
  return p < 1 ? 1 : (int)p;
}

hipError_t paged_decode(const void* q, const void* k_cache, const void* v_cache, bool fp8, float k_scale,
                        float v_scale, const int* block_table, const int* seq_lens, void* o, float* lse, int num_seqs,
                        int H, int Hkv, int d, int max_pages_per_seq, int num_pages, float scale, float* ws_o,
                        float* ws_lse, int* ws_range, int parts, int slots, hipStream_t stream) {
  DecodeArgs a{};
  a.q = (const uint16_t*)q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.bt = block_table;
  a.lens = seq_lens;
  a.ws_o = ws_o;
  a.ws_lse = ws_lse;
  a.ws_range = ws_range;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.S = num_seqs;
  a.H = H;
  a.Hkv = Hkv;
  a.group = H / Hkv;
  a.max_pages = max_pages_per_seq;
  a.num_pages = num_pages;
  a.parts = parts;
  a.slots = slots;
  // the FP8 cache holds its values divided by k_scale and v_scale: k_scale joins the softmax scale,
  // v_scale multiplies each partial output (the LSE does not depend on it)
  a.scale = fp8 ? scale * k_scale : scale;
  a.scale_log2 = a.scale * kLog2e;
  a.vscale = fp8 ? v_scale : 1.f;
  if (fp8) return d == 64 ? launch_decode<64, true>(a, stream) : launch_decode<128, true>(a, stream);
  return d == 64 ? launch_decode<64, false>(a, stream) : launch_decode<128, false>(a, stream);
}

}  // namespace paa
