// Exact causal / non-causal attention forward, bf16 in/out, fp32 accumulation,
// for gfx950 (CDNA4).
//
// What is computed ("Fast Attention Kernels and Operator Fusion", section
// "FlashAttention-Style Kernels"): O = softmax(scale * Q K^T + M) V with M the
// causal mask or zero, processed tile by tile so the score matrix only ever
// lives in registers.  The running row maximum, running row sum and the
// rescale of the partial output when the maximum grows are the online softmax
// of "Kernel Fusion and Custom Kernels", section "3. FlashAttention: The
// Milestone of Fusion" (v1); one wave owning its own query rows follows the v2
// work partitioning described there.
//
// Mapping onto the chip:
//  * a workgroup is 4 waves; each wave owns 32 query rows of one query head.
//    The 4 waves cover HPW heads of one GQA group x (4 / HPW) row blocks, so
//    all of them read the same K/V head and share its LDS tiles.
//  * K/V tiles of 64 keys are staged global -> VGPR -> LDS, double buffered:
//    the loads of tile j+1 are in flight while tile j is computed.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q kept in
//    VGPRs for the whole kernel), so each lane ends up holding 16 scores of
//    ONE query row (row l%32; the two half-waves split the keys).  Row max is
//    a lane-local max plus one permlane32 swap; the row sum stays lane-local
//    until the epilogue.
//  * O^T = V^T P^T with the same MFMA: B = the lane's own probabilities
//    (bf16), A = V read with ds_read_b64_tr_b16, and the contraction order of
//    keys is permuted to match where the score MFMA left each probability.
//    The accumulator of lane l again belongs to query row l%32, so the
//    rescale by exp(m_old - m_new) is lane-local.
//  * causal: tiles entirely above the diagonal of the workgroup are never
//    loaded; a wave whose rows all precede a tile skips its math; only tiles
//    crossing the diagonal (or the ragged end of the sequence) are masked.
//    Work units are issued heaviest first.

#include "device_common.hpp"
#include "launch.hpp"

namespace paa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBc = 64;  // keys per tile

template <int D>
struct PrefillLds {
  // K rows padded by 16 bytes: 16 consecutive rows read at one column hit distinct banks.
  static constexpr int kStrideK = D + 8;    // in bf16 elements
  // V rows padded by 64 bytes: the 4-row blocks of the transposed reads hit distinct banks.
  static constexpr int kStrideV = D + 32;
  static constexpr int kTileK = kBc * kStrideK;
  static constexpr int kTileV = kBc * kStrideV;
  static constexpr int kBytes = 2 * (kTileK + kTileV) * 2;  // double buffered, 2 bytes each
};

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int B, H, Hkv, N;
  int n_qtiles;      // query row tiles per head group
  int units_per_qt;  // B * Hkv * (group / HPW)
  float scale;       // softmax scale applied to Q.K
  float scale_log2;  // scale * log2(e)
};

template <int D, bool CAUSAL, int HPW>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int kRowBlocks = kWaves / HPW;            // row blocks of 32 per head in a workgroup
  constexpr int kTileRows = kRowBlocks * kRowsPerWave; // query rows per head in a workgroup
  constexpr int kChunksPerRow = D / 8;                // 16-byte chunks in one K/V row
  constexpr int kChunksPerThread = kBc * kChunksPerRow / kThreads;
  constexpr int kKSteps = D / 16;                     // MFMA k-steps over the head dim
  constexpr int kDBlocks = D / 32;                    // 32-wide blocks of the head dim in O
  using L = PrefillLds<D>;

  extern __shared__ __attribute__((aligned(16))) uint16_t lds_raw[];
  PAA_LDS uint16_t* lds = (PAA_LDS uint16_t*)lds_raw;

  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int half = lane / 32;  // which half-wave
  const int l32 = lane % 32;

  // ---- work unit: heaviest query tiles first ----
  const int unit = blockIdx.x;
  const int qt = a.n_qtiles - 1 - unit / a.units_per_qt;
  int rest = unit % a.units_per_qt;
  const int group = a.H / a.Hkv;
  const int subgroups = group / HPW;
  const int hsub = rest % subgroups;
  rest /= subgroups;
  const int g = rest % a.Hkv;
  const int b = rest / a.Hkv;

  const int head = g * group + hsub * HPW + wave / kRowBlocks;
  const int q0_tile = qt * kTileRows;
  const int q0 = q0_tile + (wave % kRowBlocks) * kRowsPerWave;  // first row of this wave
  const int my_row = q0 + l32;

  const size_t N = a.N;
  const uint16_t* qh = a.q + ((size_t)b * a.H + head) * N * D;
  const uint16_t* kh = a.k + ((size_t)b * a.Hkv + g) * N * D;
  const uint16_t* vh = a.v + ((size_t)b * a.Hkv + g) * N * D;

  // ---- Q fragment (B operand of S^T = K Q^T): row my_row, d = 16t + 8*half + 0..7 ----
  u32x4_t qf[kKSteps];
#pragma unroll
  for (int t = 0; t < kKSteps; ++t) {
    if (my_row < a.N)
      qf[t] = *(const u32x4_t*)(qh + (size_t)my_row * D + 16 * t + 8 * half);
    else
      qf[t] = u32x4_t{0, 0, 0, 0};
  }

  // ---- key range of this workgroup ----
  const int kv_end = CAUSAL ? min(a.N, q0_tile + kTileRows) : a.N;
  const int n_tiles = (kv_end + kBc - 1) / kBc;

  // ---- staging: thread owns chunks tid + 256*i of the [64 x D] tile ----
  u32x4_t kreg[kChunksPerThread], vreg[kChunksPerThread];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      const int c = tid + kThreads * i;
      const int r = c / kChunksPerRow;
      const int col = (c % kChunksPerRow) * 8;
      const int key = j * kBc + r;
      if (key < a.N) {
        kreg[i] = *(const u32x4_t*)(kh + (size_t)key * D + col);
        vreg[i] = *(const u32x4_t*)(vh + (size_t)key * D + col);
      } else {
        kreg[i] = u32x4_t{0, 0, 0, 0};
        vreg[i] = u32x4_t{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
    PAA_LDS uint16_t* kt = lds + buf * (L::kTileK + L::kTileV);
    PAA_LDS uint16_t* vt = kt + L::kTileK;
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      const int c = tid + kThreads * i;
      const int r = c / kChunksPerRow;
      const int col = (c % kChunksPerRow) * 8;
      *(PAA_LDS u32x4_t*)(kt + r * L::kStrideK + col) = kreg[i];
      *(PAA_LDS u32x4_t*)(vt + r * L::kStrideV + col) = vreg[i];
    }
  };

  // ---- running state of row my_row ----
  float m_run = -INFINITY;  // running max of raw scores (before scale)
  float l_run = 0.f;        // this lane's share of the running sum
  f32x16_t acc[kDBlocks];
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  load_tile(0);
  store_tile(0);

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_tiles) load_tile(j + 1);
    __syncthreads();

    const int k0 = j * kBc;
    const bool wave_active = !CAUSAL || (k0 <= q0 + kRowsPerWave - 1);
    if (wave_active) {
      const PAA_LDS uint16_t* kt = lds + buf * (L::kTileK + L::kTileV);
      const PAA_LDS uint16_t* vt = kt + L::kTileK;

      // S^T block mb: keys k0 + 32mb + 8(i/4) + 4*half + i%4, query my_row
      f32x16_t s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        for (int i = 0; i < 16; ++i) s[mb][i] = 0.f;
#pragma unroll
        for (int t = 0; t < kKSteps; ++t) {
          const u32x4_t kf = *(const PAA_LDS u32x4_t*)(kt + (32 * mb + l32) * L::kStrideK + 16 * t + 8 * half);
          s[mb] = mfma32x32x16(kf, qf[t], s[mb]);
        }
      }

      // mask: causal keys after the row, and keys past the end of the sequence
      const bool need_mask = (CAUSAL && (k0 + kBc - 1 > q0)) || (k0 + kBc > a.N);
      if (need_mask) {
        const int lim = CAUSAL ? min(my_row, a.N - 1) : a.N - 1;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * mb + 8 * (i / 4) + 4 * half + (i % 4);
            if (key > lim) s[mb][i] = -INFINITY;
          }
      }

      // online softmax update for row my_row
      float tmax = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[mb][i]);
      tmax = fmaxf(tmax, swap_halves(tmax, half));
      const float m_new = fmaxf(m_run, tmax);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2((m_run - m_use) * a.scale_log2);
      const float neg_ms = -m_use * a.scale_log2;
      m_run = m_new;

      u32x4_t pf[4];  // B operands of the 4 PV k-steps (16 keys each)
      float psum = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        float p[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          p[i] = fast_exp2(fmaf(s[mb][i], a.scale_log2, neg_ms));
          psum += p[i];
        }
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          pf[2 * mb + sh] = u32x4_t{pack_bf16x2(p[8 * sh + 0], p[8 * sh + 1]), pack_bf16x2(p[8 * sh + 2], p[8 * sh + 3]),
                                    pack_bf16x2(p[8 * sh + 4], p[8 * sh + 5]), pack_bf16x2(p[8 * sh + 6], p[8 * sh + 7])};
        }
      }
      l_run = l_run * alpha + psum;

#pragma unroll
      for (int db = 0; db < kDBlocks; ++db) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
      }

      // O^T += V^T P^T.  PV k-step ks covers keys 16ks..16ks+15 of the tile; logical k = 8*half + jj
      // maps to key 16ks + 8(jj/4) + 4*half + jj%4.  A operand via two transposed reads.
      const int grp = lane / 16;       // 16-lane group
      const int gi = lane % 16;        // lane within the group
      const int colhalf = grp % 2;     // which 16 columns of the 32-wide d block
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int krow = 16 * ks + 4 * half + gi / 4;
          const int dcol = 32 * db + 16 * colhalf + 4 * (gi % 4);
          const u32x2_t lo = lds_read_tr16(vt + krow * L::kStrideV + dcol);
          const u32x2_t hi = lds_read_tr16(vt + (krow + 8) * L::kStrideV + dcol);
          const u32x4_t vf = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
          acc[db] = mfma32x32x16(vf, pf[ks], acc[db]);
        }
      }
    }

    if (j + 1 < n_tiles) store_tile(buf ^ 1);
  }

  // ---- epilogue: O = acc / l, LSE = scale * m + ln(l) ----
  const float l_tot = l_run + swap_halves(l_run, half);
  const float inv_l = 1.f / l_tot;
  if (my_row < a.N) {
    uint16_t* orow = a.o + (((size_t)b * a.H + head) * N + my_row) * D;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * db + 8 * gq + 4 * half;
        u32x2_t w = {pack_bf16x2(acc[db][4 * gq + 0] * inv_l, acc[db][4 * gq + 1] * inv_l),
                     pack_bf16x2(acc[db][4 * gq + 2] * inv_l, acc[db][4 * gq + 3] * inv_l)};
        *(u32x2_t*)(orow + d0) = w;
      }
    }
    if (a.lse != nullptr && half == 0)
      a.lse[((size_t)b * a.H + head) * N + my_row] = a.scale * m_run + __logf(l_tot);
  }
}

template <int D, bool CAUSAL, int HPW>
hipError_t launch_prefill(const PrefillArgs& base, hipStream_t stream) {
  PrefillArgs a = base;
  constexpr int kTileRows = (kWaves / HPW) * kRowsPerWave;
  a.n_qtiles = (a.N + kTileRows - 1) / kTileRows;
  a.units_per_qt = a.B * a.Hkv * ((a.H / a.Hkv) / HPW);
  const long long units = (long long)a.n_qtiles * a.units_per_qt;
  if (units > 0x7fffffffLL) return hipErrorInvalidValue;
  constexpr int lds_bytes = PrefillLds<D>::kBytes;
  // raise the dynamic LDS limit once per instantiation (thread-safe static initialisation)
  static const hipError_t attr = hipFuncSetAttribute((const void*)prefill_bf16_kernel<D, CAUSAL, HPW>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, HPW>), dim3((unsigned)units), dim3(kThreads), lds_bytes,
                     stream, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t dispatch_hpw(const PrefillArgs& a, hipStream_t stream) {
  const int group = a.H / a.Hkv;
  if (group % 4 == 0) return launch_prefill<D, CAUSAL, 4>(a, stream);
  if (group % 2 == 0) return launch_prefill<D, CAUSAL, 2>(a, stream);
  return launch_prefill<D, CAUSAL, 1>(a, stream);
}

}  // namespace

hipError_t prefill_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                        int N, int d, bool causal, float scale, hipStream_t stream) {
  PrefillArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.N = N;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  if (d == 64) return causal ? dispatch_hpw<64, true>(a, stream) : dispatch_hpw<64, false>(a, stream);
  return causal ? dispatch_hpw<128, true>(a, stream) : dispatch_hpw<128, false>(a, stream);
}

}  // namespace paa
