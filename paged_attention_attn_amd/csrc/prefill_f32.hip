// Exact attention forward with fp32 inputs, outputs and arithmetic (no
// reduced-precision matrix ops), for gfx950.
//
// Same computation and the same online softmax as the bf16 kernel (see
// "Fast Attention Kernels and Operator Fusion", section "FlashAttention-Style
// Kernels", and "Kernel Fusion and Custom Kernels", section 3, v1): K/V tiles
// of 64 keys are staged in LDS and every score stays on chip.  Each lane owns
// one query row: its query vector and output accumulator sit in VGPRs, the
// dot products read K rows from LDS as broadcasts, and the row max / sum are
// lane-local.  This path is for fp32 accuracy, not throughput.

#include "device_common.hpp"
#include "launch.hpp"

namespace paa {

namespace {

constexpr int kRows = 64;  // query rows per workgroup (one wave, one row per lane)
constexpr int kKeys = 32;  // keys per LDS tile

struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int B, H, Hkv, N, n_qtiles;
  float scale, scale_log2;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows) void prefill_f32_kernel(F32Args a) {
  __shared__ float kt[kKeys][D];
  __shared__ float vt[kKeys][D];
  const int lane = threadIdx.x;
  const int qt = a.n_qtiles - 1 - (int)(blockIdx.x % a.n_qtiles);
  const int bh = blockIdx.x / a.n_qtiles;
  const int h = bh % a.H;
  const int b = bh / a.H;
  const int g = h / (a.H / a.Hkv);
  const int row = qt * kRows + lane;
  const size_t N = a.N;
  const float* qrow = a.q + (((size_t)b * a.H + h) * N + (row < a.N ? row : 0)) * D;
  const float* kh = a.k + ((size_t)b * a.Hkv + g) * N * D;
  const float* vh = a.v + ((size_t)b * a.Hkv + g) * N * D;

  float qv[D], acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qv[c] = row < a.N ? qrow[c] : 0.f;
    acc[c] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  const int kv_end = CAUSAL ? min(a.N, (qt + 1) * kRows) : a.N;
  for (int k0 = 0; k0 < kv_end; k0 += kKeys) {
    __syncthreads();
    for (int i = lane; i < kKeys * D; i += kRows) {
      const int r = i / D, c = i % D;
      const bool ok = k0 + r < a.N;
      kt[r][c] = ok ? kh[(size_t)(k0 + r) * D + c] : 0.f;
      vt[r][c] = ok ? vh[(size_t)(k0 + r) * D + c] : 0.f;
    }
    __syncthreads();
    float s[kKeys];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) dot = fmaf(qv[c], kt[j][c], dot);
      const int key = k0 + j;
      const bool visible = key < a.N && (!CAUSAL || key <= row);
      s[j] = visible ? dot : -INFINITY;
      tmax = fmaxf(tmax, s[j]);
    }
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2((m_run - m_use) * a.scale_log2);
    const float neg_ms = -m_use * a.scale_log2;
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] *= alpha;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const float p = fast_exp2(fmaf(s[j], a.scale_log2, neg_ms));
      l_run += p;
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] = fmaf(p, vt[j][c], acc[c]);
    }
  }
  if (row < a.N) {
    const float inv = 1.f / l_run;
    float* orow = a.o + (((size_t)b * a.H + h) * N + row) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) orow[c] = acc[c] * inv;
    if (a.lse != nullptr) a.lse[((size_t)b * a.H + h) * N + row] = a.scale * m_run + __logf(l_run);
  }
}

template <int D, bool CAUSAL>
hipError_t launch_f32(F32Args a, hipStream_t stream) {
  a.n_qtiles = (a.N + kRows - 1) / kRows;
  const long long blocks = (long long)a.B * a.H * a.n_qtiles;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(kRows), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t prefill_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int Hkv,
                       int N, int d, bool causal, float scale, hipStream_t stream) {
  F32Args a{q, k, v, o, lse, B, H, Hkv, N, 0, scale, scale * kLog2e};
  if (d == 64) return causal ? launch_f32<64, true>(a, stream) : launch_f32<64, false>(a, stream);
  return causal ? launch_f32<128, true>(a, stream) : launch_f32<128, false>(a, stream);
}

}  // namespace paa
