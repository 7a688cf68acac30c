// Exact attention forward with FP8 (OCP e4m3) Q, K and V and per-tensor scales, bf16 output,
// for gfx950.
//
// What is computed: the softmax attention of the dequantized inputs,
// O = softmax(scale * (qs Q8) (ks K8)^T + M) (vs V8), with M the causal mask or zero.  Using 8-bit
// operands for both products, with per-tensor scales, is the FP8 path of FlashAttention v3
// ("Kernel Fusion and Custom Kernels", section "3. FlashAttention: The Milestone of Fusion",
// v3: FP8 for Q.K and P.V, about twice the matrix throughput of 16-bit operands).  As there, the
// probabilities are rounded to e4m3 before the product with V.
//
// Probabilities in e4m3: each row's probabilities are taken relative to a reference maximum that
// only moves when a tile's maximum exceeds it by more than 2^kFp8RescaleLog2, and are scaled up by
// 2^kFp8ShiftLog2 (folded into the exponent, so it costs nothing): p' = 2^(s - m_ref + shift) lies
// in (0, 2^(4 + 4)] = (0, 256], inside e4m3's range (largest 448), and probabilities down to 2^-10
// of the reference stay normal (relative rounding error <= 2^-4).  O is normalised by the sum of
// the ROUNDED probabilities, computed by one more 8-bit MFMA against an all-ones operand, so O is
// a weighted mean of V rows whose weights are the rounded probabilities (identical V rows return
// that row).  The LSE uses the fp32 sum of the unrounded values (the shift taken back out).
//
// Mapping: the two-group ping-pong workgroup of the bf16 kernel (8 waves; waves w and w + 4 share
// a SIMD and run one phase apart, so one group's MFMA phase overlaps the other's softmax), with
// v_mfma_scale_f32_32x32x64_f8f6f4 (scales fixed at 1; the per-tensor scales are applied to the
// fp32 scores and output).  Each phase takes two 64-key tiles: with 8-bit operands a tile's MFMA
// work is half that of bf16, and one tile per phase left the barriers and waits of a period at
// about a sixth of its time.  The layouts below are per 64-key tile:
//  * operand pairing of that instruction (checked on gfx950): lane l supplies row l%32 of A and
//    column l%32 of B, and byte j of lane l meets byte j of lanes with the same l/32; any
//    assignment of contraction indices to (l/32, j) that A and B share is valid.
//  * S^T = K Q^T: for k-step t the contraction index (l/32, j) is head dim 64t + 32(l/32) + j, so a
//    lane reads 32 contiguous bytes of a K row (two 16-byte LDS reads) and of its Q row.
//  * O^T = V^T P^T: the score MFMA leaves lane l the probabilities of keys
//    8(i/4) + 4(l/32) + i%4 (+32 for the second 32-key block), i = 0..15, of row l%32.  The
//    contraction index (l/32, j) is taken to be key 32(l/32) + j, so a lane's A operand is 32
//    contiguous bytes of its V^T row (V is supplied transposed, [B, Hkv, d, N], keys
//    contiguous), read as two 16-byte LDS reads.  For the B operand the two halves of the wave
//    trade probabilities: after packing them to e4m3 in groups of four keys, one
//    v_permlane32_swap per group gives the lower half the keys 0..31 and the upper half the keys
//    32..63, already in order.
//  * LDS: K tiles are 64 rows of d bytes, V^T tiles d rows of 64 bytes; 16-byte chunk c of row r is
//    stored at chunk c ^ f(r), chosen so that every read above is free of bank conflicts
//    (64 banks of 4 bytes); the swizzle is applied by choosing which chunk each lane of the direct
//    global->LDS load fetches.
// Requirements: d in {64, 128}; N a multiple of 16 (each V^T row starts 16-byte aligned).

#include <atomic>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"
#include "tile_pipeline.hpp"

namespace paa {

namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr float kFp8RescaleLog2 = 4.0f;  // lazy rescale threshold of this kernel (log2 units)
constexpr float kFp8ShiftLog2 = 4.0f;    // probabilities are scaled by 2^4 before rounding to e4m3
static_assert(kFp8RescaleLog2 + kFp8ShiftLog2 <= 8.0f, "probabilities must stay <= 256 < 448");
constexpr int kE4m3Ones = 0x38383838;    // four e4m3 bytes of 1.0
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16_t mfma_fp8(i32x8_t a, i32x8_t b, f32x16_t c) {
  // formats 0/0: both operands e4m3; scale exponents 127: a factor of 1
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Four fp32 -> four e4m3 bytes (round to nearest even), first value in the lowest byte.
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

template <int D>
struct Fp8Layout {
  static constexpr int kKRowBytes = D;                 // K tile: 64 rows of D bytes
  static constexpr int kKCpr = D / 16;                 // 16-byte chunks per K row
  static constexpr int kKTileBytes = kBc * D;
  static constexpr int kKBlocks = kKTileBytes / 1024;  // wave-wide 1 KB loads per K tile
  static constexpr int kVRowBytes = kBc;               // V^T tile: D rows of 64 bytes
  static constexpr int kVTileBytes = D * kBc;
  static constexpr int kVBlocks = kVTileBytes / 1024;
  static constexpr int kLoadsPerWave = (kKBlocks + kVBlocks) / 8;
  static_assert((kKBlocks + kVBlocks) % 8 == 0, "loads must split evenly over eight waves");
};

// chunk position swizzles (functions of the row only)
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? (r >> 1) & 7 : (r >> 2) & 3;
}
__device__ __forceinline__ int swz_v(int d) { return (d >> 2) & 3; }

struct Fp8Args {
  const uint8_t* q;   // [B, H, N, D] e4m3
  const uint8_t* k;   // [B, Hkv, N, D] e4m3
  const uint8_t* vt;  // [B, Hkv, D, N] e4m3 (V transposed)
  uint16_t* o;        // [B, H, N, D] bf16
  float* lse;         // [B, H, N] or null
  int B, H, Hkv, N;
  int n_qtiles, units_per_qt, mirror;
  float scale_eff;    // scale * q_scale * k_scale
  float scale_log2;   // scale_eff * log2(e)
  float rescale_raw;  // kFp8RescaleLog2 / scale_log2
  float v_scale;
};

template <int D, bool CAUSAL, int HPW, int STAGES>
__global__ __launch_bounds__(512, 1) void prefill_fp8_kernel(Fp8Args a) {
  constexpr int WAVES = 8;
  using T = Fp8Layout<D>;
  constexpr int kRowBlocks = WAVES / HPW;
  constexpr int kTileRows = kRowBlocks * 32;
  constexpr int kKSteps = D / 64;
  constexpr int kDBlocks = D / 32;
  constexpr int kSub = 2;  // 64-key tiles per iteration (per ping-pong phase)
  constexpr int kLoadsPerStage = kSub * T::kLoadsPerWave;
  static_assert(STAGES >= 2 && STAGES <= 4, "2 to 4 stages");

  __shared__ __attribute__((aligned(1024))) char k_st0[kSub * T::kKTileBytes];
  __shared__ __attribute__((aligned(1024))) char k_st1[kSub * T::kKTileBytes];
  __shared__ __attribute__((aligned(1024))) char k_st2[kSub * T::kKTileBytes];
  __shared__ __attribute__((aligned(1024))) char k_st3[kSub * T::kKTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_st0[kSub * T::kVTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_st1[kSub * T::kVTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_st2[kSub * T::kVTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_st3[kSub * T::kVTileBytes];
  auto kst = [&](auto i_tag) __attribute__((always_inline)) -> PAA_LDS char* {
    constexpr int i = decltype(i_tag)::value % STAGES;
    if constexpr (i == 0) return (PAA_LDS char*)k_st0;
    else if constexpr (i == 1) return (PAA_LDS char*)k_st1;
    else if constexpr (i == 2) return (PAA_LDS char*)k_st2;
    else return (PAA_LDS char*)k_st3;
  };
  auto vst = [&](auto i_tag) __attribute__((always_inline)) -> PAA_LDS char* {
    constexpr int i = decltype(i_tag)::value % STAGES;
    if constexpr (i == 0) return (PAA_LDS char*)v_st0;
    else if constexpr (i == 1) return (PAA_LDS char*)v_st1;
    else if constexpr (i == 2) return (PAA_LDS char*)v_st2;
    else return (PAA_LDS char*)v_st3;
  };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int grp = wave / 4;
  const int lane = tid % 64;
  const int half = lane / 32;
  const int l32 = lane % 32;

  // ---- work unit: heaviest query tiles first (mirrored when the whole grid is resident) ----
  const int units = a.n_qtiles * a.units_per_qt;
  const int half_units = units / 2;
  const int unit = (a.mirror && (int)blockIdx.x >= half_units) ? units - 1 + half_units - (int)blockIdx.x
                                                                : (int)blockIdx.x;
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
  const int q0 = q0_tile + (wave % kRowBlocks) * 32;

  const size_t N = a.N;
  const uint8_t* qh = a.q + ((size_t)b * a.H + head) * N * D;
  const uint8_t* kh = a.k + ((size_t)b * a.Hkv + g) * N * D;
  const uint8_t* vh = a.vt + ((size_t)b * a.Hkv + g) * (size_t)D * N;

  // 64-key tiles [0, n_tiles); iteration i covers tiles kSub * i .. kSub * i + kSub - 1 (a tile past
  // n_tiles, or past this wave's last causal tile, is loaded as a repeat and fully masked)
  const int kv_end = CAUSAL ? min(a.N, q0_tile + kTileRows) : a.N;
  const int n_tiles = (kv_end + kBc - 1) / kBc;
  const int n_iter = (n_tiles + kSub - 1) / kSub;
  const int last_tile = CAUSAL ? min(n_tiles - 1, (q0 + 31) / kBc) : n_tiles - 1;
  const int n_act = last_tile / kSub + 1;

  // One stage: the K tiles of iteration s and the V^T tiles of iteration s - 1.  The waves' loads
  // of one tile are numbered u = wave * kLoadsPerWave + i over the K blocks, then the V^T blocks;
  // tiles past the end repeat the last one (never read, or fully masked), so every stage issues the
  // same count.
  // Loads go through buffer resources spanning this (batch, KV head)'s K and V^T, so each costs
  // one vector add on a lane offset fixed for the loop: K rows past the end read as zeros (they
  // are masked); V^T rows run on into the next row, so the last tile's chunks past the end are
  // pointed back at valid keys instead.
  const int kv_bytes = a.N * D;  // below 2^31 (checked on the host)
  const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)kh, (short)0, kv_bytes, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)vh, (short)0, kv_bytes, kRawBufferWord3);
  auto load_block = [&](int u, int jk, int jv, PAA_LDS char* kdst, PAA_LDS char* vdst) __attribute__((always_inline)) {
    if (u < T::kKBlocks) {
      constexpr int kRowsPerBlock = 1024 / D;
      const int r = u * kRowsPerBlock + lane / T::kKCpr;
      const int c = (lane % T::kKCpr) ^ swz_k<D>(r);
      const uint32_t off = (uint32_t)(r * D + c * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(k_rsrc, (PAA_LDS void*)(kdst + u * 1024), 16,
                                               (int)(off + (uint32_t)(jk * kBc * D)), 0, 0, 0);
    } else {
      const int vb = u - T::kKBlocks;
      const int d = vb * 16 + lane / 4;
      const int c = (lane % 4) ^ swz_v(d);
      const int key0 = jv * kBc + 16 * c;
      const int key = jv * kBc + kBc <= a.N ? key0 : min(key0, a.N - 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(v_rsrc, (PAA_LDS void*)(vdst + vb * 1024), 16, d * a.N + key, 0, 0, 0);
    }
  };
  auto issue_stage = [&](auto s_tag, int s) __attribute__((always_inline)) {
    using Prev = std::integral_constant<int, decltype(s_tag)::value + STAGES - 1>;
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub) {
      const int jk = min(kSub * s + sub, n_tiles - 1), jv = min(max(kSub * (s - 1) + sub, 0), n_tiles - 1);
#pragma unroll
      for (int i = 0; i < T::kLoadsPerWave; ++i)
        load_block(wave * T::kLoadsPerWave + i, jk, jv, kst(s_tag) + sub * T::kKTileBytes,
                   vst(Prev{}) + sub * T::kVTileBytes);
    }
  };

  // ---- Q fragments (B operand of S^T): row q0 + l32, bytes 64t + 32 half .. +31 ----
  i32x8_t qf[kKSteps];
  {
    const int row = q0 + l32;
#pragma unroll
    for (int t = 0; t < kKSteps; ++t) {
      if (row < a.N) {
        const u32x4_t lo = *(const u32x4_t*)(qh + (size_t)row * D + 64 * t + 32 * half);
        const u32x4_t hi = *(const u32x4_t*)(qh + (size_t)row * D + 64 * t + 32 * half + 16);
        qf[t] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      } else {
        qf[t] = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  }
  // prologue: stage 0 (K_0 only; the V^T half of each wave's loads repeats tile 0 into a free
  // buffer so that the count matches later stages), then stages 1 .. STAGES-1
  issue_stage(std::integral_constant<int, 0>{}, 0);
  auto prologue = [&](auto s_tag, int s) __attribute__((always_inline)) { issue_stage(s_tag, s); };
  for_stages<1, STAGES>(prologue, 0, STAGES);

  // ---- per-lane LDS byte offsets ----
  int koff[kKSteps][2];  // K row l32 (+32 per key block), chunks 4t + 2 half + e
#pragma unroll
  for (int t = 0; t < kKSteps; ++t)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      koff[t][e] = l32 * T::kKRowBytes + ((4 * t + 2 * half + e) ^ swz_k<D>(l32)) * 16;
  int voff[2];  // V^T row l32 (+32 per head-dim block), chunks 2 half and 2 half + 1: keys 32 half .. +31
#pragma unroll
  for (int e = 0; e < 2; ++e) voff[e] = l32 * T::kVRowBytes + (((2 * half + e) ^ swz_v(l32)) * 16);

  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t acc[kDBlocks];
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  // sum of the rounded probabilities of column l%32 (every row of this product holds it; only
  // element 0 is read, so only element 0 is rescaled)
  f32x16_t acc_l = {};
  const i32x8_t ones = {kE4m3Ones, kE4m3Ones, kE4m3Ones, kE4m3Ones, kE4m3Ones, kE4m3Ones, kE4m3Ones, kE4m3Ones};
  f32x16_t s[kSub][2];
  i32x8_t pf[kSub];

  auto m_phase = [&](auto u_tag, int i) __attribute__((always_inline)) {
    using U = decltype(u_tag);
    using Prev = std::integral_constant<int, U::value + STAGES - 1>;
    const PAA_LDS char* kt = kst(U{});
    const PAA_LDS char* vt = vst(Prev{});
    if (i < n_act) {
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub)
#pragma unroll
        for (int t = 0; t < kKSteps; ++t)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            const PAA_LDS char* kr = kt + sub * T::kKTileBytes + mb * 32 * T::kKRowBytes;
            const u32x4_t lo = *(const PAA_LDS u32x4_t*)(kr + koff[t][0]);
            const u32x4_t hi = *(const PAA_LDS u32x4_t*)(kr + koff[t][1]);
            const i32x8_t kf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            s[sub][mb] = t == 0 ? mfma_fp8(kf, qf[t], f32x16_t{}) : mfma_fp8(kf, qf[t], s[sub][mb]);
          }
    }
    if (i >= 1 && i - 1 < n_act) {
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub) {
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db) {
          const PAA_LDS char* vr = vt + sub * T::kVTileBytes + db * 32 * T::kVRowBytes;
          const u32x4_t lo = *(const PAA_LDS u32x4_t*)(vr + voff[0]);
          const u32x4_t hi = *(const PAA_LDS u32x4_t*)(vr + voff[1]);
          const i32x8_t vf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          acc[db] = mfma_fp8(vf, pf[sub], acc[db]);
        }
        acc_l = mfma_fp8(ones, pf[sub], acc_l);
      }
    }
  };

  auto v_phase = [&](int i) __attribute__((always_inline)) {
    if (i < 0 || i >= n_act) return;
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub) {
      const int k0 = (kSub * i + sub) * kBc;
      const bool need_mask = (CAUSAL && (k0 + kBc - 1 > q0)) || (k0 + kBc > a.N);
      if (need_mask) {  // key k0 + 4 half + c, with c a constant per element
        const int lim = (CAUSAL ? min(q0 + l32, a.N - 1) : a.N - 1) - (k0 + 4 * half);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (32 * mb + 8 * (e / 4) + (e % 4) > lim) s[sub][mb][e] = -INFINITY;
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, s[sub][mb][e]);
    tmax = fmaxf(tmax, swap_halves(tmax, half));
    if (__builtin_amdgcn_ballot_w64(tmax > m_run + a.rescale_raw) != 0) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2((m_run - m_new) * a.scale_log2);
      m_run = m_new;
      l_run *= alpha;
      acc_l[0] *= alpha;
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[db][e] *= alpha;
    }
    const float neg_ms = m_run == -INFINITY ? 0.f : kFp8ShiftLog2 - m_run * a.scale_log2;
    float lt = 0.f;  // this lane's share of the iteration's (unrounded) sum, one chain from the first value
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub) {
      int xy[2][4];  // e4m3 of keys 8g + 4 half + 0..3 of block mb (second block: +32) of the tile
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        float p[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          p[e] = fast_exp2(fmaf(s[sub][mb][e], a.scale_log2, neg_ms));
          lt = (sub == 0 && mb == 0 && e == 0) ? p[e] : lt + p[e];
        }
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) xy[mb][gq] = pack_fp8x4(p[4 * gq], p[4 * gq + 1], p[4 * gq + 2], p[4 * gq + 3]);
      }
      // swap the upper half's first block with the lower half's second: the lower half then holds
      // keys 8g .. 8g + 7 (own, then partner) and the upper half keys 32 + 8g .. +7 (partner, then own)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const auto r = __builtin_amdgcn_permlane32_swap(xy[0][gq], xy[1][gq], false, false);
        pf[sub][2 * gq] = r[0];
        pf[sub][2 * gq + 1] = r[1];
      }
    }
    l_run += lt;
  };

  wait_vmcnt<(STAGES - 1) * kLoadsPerStage>();  // Q and stage 0 have landed
  tile_barrier();

  auto run = [&](auto grp_tag) __attribute__((always_inline)) {
    constexpr bool kLead = decltype(grp_tag)::value == 0;
    auto period_pair = [&](auto u_tag, int i) __attribute__((always_inline)) {
      using U = decltype(u_tag);
      using Refill = std::integral_constant<int, U::value + STAGES - 1>;
      if (i >= 1) issue_stage(Refill{}, i - 1 + STAGES);
      if constexpr (kLead) m_phase(U{}, i); else v_phase(i - 1);
      tile_barrier();
      if constexpr (kLead) v_phase(i); else m_phase(U{}, i);
      wait_vmcnt<(STAGES - 2) * kLoadsPerStage>();
      tile_barrier();
    };
    for (int i0 = 0; i0 <= n_iter; i0 += STAGES) for_stages<0, STAGES>(period_pair, i0, n_iter + 1);
  };
  if (grp == 0)
    run(std::integral_constant<int, 0>{});
  else
    run(std::integral_constant<int, 1>{});
  wait_vmcnt<0>();

  // ---- epilogue: O = v_scale * acc / (sum of rounded p), LSE = scale_eff * m + ln(sum of p) - shift ----
  // O leaves through LDS (store_o_tile), wave w's tile in half of one stage array, once every wave is
  // past its last tile (every load landed, every tile read done).
  const int row = q0 + l32;
  const float l_tot = l_run + swap_halves(l_run, half);
  const float f = a.v_scale / acc_l[0];
  static_assert(WAVES * 32 * 2 * D <= 2 * STAGES * kSub * T::kKTileBytes && T::kKTileBytes == T::kVTileBytes &&
                    kSub * T::kKTileBytes == 2 * 32 * 2 * D,
                "two waves' O tiles fill one stage array");
  __syncthreads();
  PAA_LDS char* ot = (wave / 2 == 0   ? (PAA_LDS char*)k_st0
                      : wave / 2 == 1 ? (PAA_LDS char*)k_st1
                      : wave / 2 == 2 ? (PAA_LDS char*)v_st0
                                      : (PAA_LDS char*)v_st1) + (wave % 2) * (32 * 2 * D);
  store_o_tile<D>(ot, acc, f, lane, a.o + (((size_t)b * a.H + head) * N + q0) * D, D, a.N - q0);
  if (row < a.N && a.lse != nullptr && half == 0)
    a.lse[((size_t)b * a.H + head) * N + row] = a.scale_eff * m_run + (__logf(l_tot) - kFp8ShiftLog2 * kLn2);
}

template <typename Kernel>
long long fp8_resident(Kernel kernel) {
  static std::atomic<long long> cached[16];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 16) {
    const long long c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 512, 0) != hipSuccess) return 0;
  const long long c = (long long)cus * per_cu;
  if (dev < 16) cached[dev].store(c, std::memory_order_relaxed);
  return c;
}

template <int D, bool CAUSAL, int HPW>
hipError_t launch_fp8(Fp8Args a, hipStream_t stream) {
  constexpr int kStages = 2;
  constexpr int kTileRows = (8 / HPW) * 32;
  a.n_qtiles = (a.N + kTileRows - 1) / kTileRows;
  a.units_per_qt = a.B * a.Hkv * ((a.H / a.Hkv) / HPW);
  const long long units = (long long)a.n_qtiles * a.units_per_qt;
  if (units > 0x7fffffffLL) return hipErrorInvalidValue;
  const auto kernel = prefill_fp8_kernel<D, CAUSAL, HPW, kStages>;
  a.mirror = CAUSAL && units <= fp8_resident(kernel) ? 1 : 0;
  hipLaunchKernelGGL(kernel, dim3((unsigned)units), dim3(512), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t dispatch_fp8(const Fp8Args& a, hipStream_t stream) {
  const int group = a.H / a.Hkv;
  if (group % 4 == 0) return launch_fp8<D, CAUSAL, 4>(a, stream);
  if (group % 2 == 0) return launch_fp8<D, CAUSAL, 2>(a, stream);
  return launch_fp8<D, CAUSAL, 1>(a, stream);
}

}  // namespace

hipError_t prefill_fp8(const void* q, const void* k, const void* vt, void* o, float* lse, int B, int H, int Hkv,
                       int N, int d, bool causal, float scale, float q_scale, float k_scale, float v_scale,
                       hipStream_t stream) {
  Fp8Args a{};
  a.q = (const uint8_t*)q;
  a.k = (const uint8_t*)k;
  a.vt = (const uint8_t*)vt;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.N = N;
  a.scale_eff = scale * q_scale * k_scale;
  a.scale_log2 = a.scale_eff * kLog2e;
  a.rescale_raw = kFp8RescaleLog2 / a.scale_log2;
  a.v_scale = v_scale;
  if (d == 64) return causal ? dispatch_fp8<64, true>(a, stream) : dispatch_fp8<64, false>(a, stream);
  return causal ? dispatch_fp8<128, true>(a, stream) : dispatch_fp8<128, false>(a, stream);
}

}  // namespace paa
