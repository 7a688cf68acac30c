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
//  * a workgroup is 4 or 8 waves; each wave owns 32 query rows of one query
//    head.  The waves cover HPW heads of one GQA group x (waves / HPW) row
//    blocks, so all of them read the same K/V head and share its LDS tiles.
//    (The ping-pong kernel further below runs its 8 waves as two groups one
//    phase apart.)
//  * K/V tiles of 64 keys go from global memory straight into LDS
//    (buffer_load_dwordx4 ... lds, no VGPR staging), two stages deep: the
//    loads of tile j+1 are in flight while tile j is computed, one barrier per
//    tile.  Each load goes through a buffer resource that ends at the last
//    valid row, so rows past the end read as zeros.  Each 16-byte chunk c of
//    tile row r is stored at chunk position c ^ swz(r), which keeps both the
//    row-wise K reads and the transposed V reads below free of LDS bank
//    conflicts; the swizzle is applied by choosing which chunk each lane
//    fetches, so the loads stay coalesced.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q kept in
//    VGPRs for the whole kernel), so each lane ends up holding 16 scores of
//    ONE query row (row l%32; the two half-waves split the keys).  A row
//    maximum, when one is taken (below), is a lane-local max plus one
//    permlane32 swap; the row sums stay lane-local until the epilogue.  Two sums are kept: of the fp32 probabilities (for
//    the LSE) and of the same probabilities as rounded to bf16 for P.V (one
//    v_dot2 per packed pair), by which O is divided, so that O is a weighted
//    mean of V rows with exactly the weights its numerator used (a row held
//    by one key returns that key's V row).
//  * O^T = V^T P^T with the same MFMA: B = the lane's own probabilities
//    (bf16), A = V read with ds_read_b64_tr_b16, and the contraction order of
//    keys is permuted to match where the score MFMA left each probability.
//    The accumulator of lane l again belongs to query row l%32, so the
//    rescale by exp(m_old - m_new) is lane-local.
//  * the reference of a row only has to keep the numbers finite, so no row
//    maximum is taken per tile: the probabilities of a tile are computed
//    against the current reference, and only when some lane's share of them
//    exceeds kMaxTileSum (or is not finite, as on a row's first visible
//    tile) does the wave take the exact maximum, move the reference to
//    kRefHeadroomLog2 above it (so that scores may keep rising a long way
//    before it has to move again), rescale its state and recompute them.
//    Numerator and both sums share the reference, so the result is the same
//    softmax; the LSE uses the reference actually kept.
//  * causal: tiles entirely above the diagonal of the workgroup are never
//    loaded; a wave whose rows all precede a tile skips its math; only tiles
//    crossing the diagonal (or the ragged end of the sequence) are masked.
//    Work units are issued heaviest first, and consecutive units (which the
//    dispatcher spreads over the 8 XCDs) differ in their (batch, KV head), so
//    each XCD's L2 keeps serving the same K/V heads (chunked prefill orders
//    its units by sequence instead; see work_unit).

#include <atomic>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"
#include "tile_pipeline.hpp"

namespace paa {

namespace {

template <int D>
struct TileLayout {
  static constexpr int kCpr = D / 8;                       // 16-byte chunks per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileBytes = kBc * kRowBytes;       // one K or V tile
  static constexpr int kRowsPerBlock = 64 / kCpr;          // rows of one wave-wide 16 B/lane load
  static constexpr int kBlocks = kBc / kRowsPerBlock;      // such loads per tile
};

// Chunk position swizzle of tile row r (a function of r % 16 only).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) {
    return 4 * (r & 3) + ((r >> 2) & 3);
  } else {
    const int x = (r >> 1) & 7;  // bit-reversed
    return ((x & 1) << 2) | (x & 2) | ((x >> 2) & 1);
  }
}

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
  float scale_log2;    // scale * log2(e)
  float ref_headroom;  // kRefHeadroomLog2 / scale_log2: a moved reference sits this far above the maximum
  int window;        // sliding window width (kMaskWindow only)
  int n_global;      // leading keys visible to every later query (kMaskWindow only)
  int mirror;        // 1 when the whole grid is resident at once: pair heavy and light units (see below)
  // chunked prefill over a paged cache (kMaskPaged only): q, o [T, H, d] and k, v (the chunk's new
  // keys and values) [T, Hkv, d] hold the sequences' chunks back to back, sequence s owning rows
  // q_start[s] .. q_start[s+1]-1; its first ctx_lens[s] positions are in the caches
  // [num_pages, 16, Hkv, d], where the chunk is appended
  const int* bt;
  const int* ctx_lens;
  const int* q_start;
  uint16_t* kc;
  uint16_t* vc;
  int max_pages, num_pages;
};

// WAVES waves per workgroup, RB blocks of 32 query rows per wave, STAGES-deep K and V rings in LDS.
template <int D, int WAVES, int RB, int STAGES>
struct PrefillCfg {
  static constexpr int kBlocksPerWave = TileLayout<D>::kBlocks / WAVES;  // 1 KB loads per wave per tile
  static_assert(TileLayout<D>::kBlocks % WAVES == 0, "tile rows must split evenly over the waves");
  static_assert(STAGES >= 2 && STAGES <= 4, "2 to 4 stages");
  static_assert(RB == 1 || RB == 2, "one or two 32-row blocks per wave");
  static constexpr int kRowsPerWave = 32 * RB;
  // loads a wave may still have in flight, beyond the ones the next tile needs, at the end of a tile
  static constexpr int kInFlightAfter = (STAGES - 2) * 2 * kBlocksPerWave;
};

// Masks: none, causal (key j visible to query i iff j <= i), causal with a sliding window and
// global tokens (additionally i - j < window or j < n_global), or a chunk of new tokens over a paged
// cache (chunk query i at position ctx + i sees positions 0 .. ctx + i).
enum : int { kMaskNone = 0, kMaskCausal = 1, kMaskWindow = 2, kMaskPaged = 3 };
constexpr int kPageTokens = 16;  // tokens per cache page (the only page size the library accepts)

// The work unit of a workgroup: query tile qt of query heads [g * group + hsub * HPW, + HPW) of
// sequence (batch entry) b.
struct WorkUnit {
  int qt, hsub, g, b;
};

// Sequences ranked for the chunked-prefill order: up to this many are sorted on the device.
constexpr int kMaxRankedSeqs = 256;

// Unit of workgroup `blk`.  Heaviest work first: when the grid is larger than what the chip holds
// at once, workgroups start as others finish and heaviest-first keeps the tail short.  When the
// whole grid is resident at once (a.mirror), the dispatcher gives each CU workgroups a fixed
// distance apart in launch order, so the second half of the grid is laid out in reverse: workgroup
// u of the first half (heavy) and workgroup u + units/2 (light) then carry complementary work.
//   Dense masks: query tiles from the last (most causal keys) to the first, each over every
//   (b, g, hsub).
//   Paged: the sequences' key counts (context + chunk) differ far more than a chunk's query tiles
//   do, so the order is sequence-major, the sequence with the most keys first (ties by index; up
//   to kMaxRankedSeqs sequences, beyond that in the given order), its query tiles last to first,
//   then (g, hsub) innermost: consecutive workgroups go to the chip's dies (XCDs) in turn, so when
//   Hkv * group / HPW is a multiple of their number every query tile of a (b, g) runs on one die
//   at about the same time and reads that head's cache through one L2.
// Paged units call this with every thread of the workgroup (it holds barriers) and `scratch`, LDS
// room for kMaxRankedSeqs + 1 ints that nothing else uses until the call returns.
template <int HPW, bool PAGED>
__device__ __forceinline__ WorkUnit work_unit(const PrefillArgs& a, int blk, PAA_LDS int* scratch) {
  const int units = a.n_qtiles * a.units_per_qt;
  const int half_units = units / 2;
  const int unit = (a.mirror && blk >= half_units) ? units - 1 + half_units - blk : blk;
  const int subgroups = (a.H / a.Hkv) / HPW;
  WorkUnit w;
  if constexpr (!PAGED) {
    w.qt = a.n_qtiles - 1 - unit / a.units_per_qt;
    int rest = unit % a.units_per_qt;
    w.hsub = rest % subgroups;
    rest /= subgroups;
    w.g = rest % a.Hkv;
    w.b = rest / a.Hkv;
  } else {
    const int copies = a.Hkv * subgroups;  // units of one query tile of one sequence
    const int per_seq = a.n_qtiles * copies;
    const int rank = unit / per_seq;
    const int r = unit % per_seq;
    w.qt = a.n_qtiles - 1 - r / copies;
    w.hsub = (r % copies) % subgroups;
    w.g = (r % copies) / subgroups;
    if (a.B > kMaxRankedSeqs) {
      w.b = rank;
    } else {
      const int nthreads = blockDim.x;
      for (int j = threadIdx.x; j < a.B; j += nthreads)
        scratch[j] = max(a.ctx_lens[j], 0) + (a.q_start[j + 1] - a.q_start[j]);
      __syncthreads();
      // the sequence whose rank is `rank`: exactly one candidate has it
      for (int c = threadIdx.x; c < a.B; c += nthreads) {
        const int kc = scratch[c];
        int before = 0;
        for (int j = 0; j < a.B; ++j) {
          const int kj = scratch[j];
          before += (kj > kc) || (kj == kc && j < c);
        }
        if (before == rank) scratch[kMaxRankedSeqs] = c;
      }
      __syncthreads();
      w.b = __builtin_amdgcn_readfirstlane(scratch[kMaxRankedSeqs]);
      __syncthreads();  // every wave has read it before the room is reused
    }
  }
  return w;
}

// Direct loads (16 B per lane, buffer_load ... lds) of a wave's group of consecutive K or V rows
// into LDS.  The group starts at key position row0 (wave-uniform) and has `rows` rows; a lane
// moves 16 B of row row0 + dr, at byte `off` = (dr * stride + 8c) * 2 from the row0 row, where c
// is the lane's piece of the row (`off` is fixed for the whole key loop).  Dense: the n_k rows
// are `stride` elements apart from `src`.  Paged: positions before qoff are in cache page `page`
// (the group lies in one page; a page holds 16 positions of every KV head, head g at `head_off`
// elements into a position) and the rest are the n_k - qoff chunk rows of `src` (position - qoff);
// cache and chunk rows are both `stride` elements apart.
//   A load goes through a buffer resource whose size ends at the last valid row of what it reads:
// rows at or past n_k read as zeros (they are masked) and no access leaves the valid rows.  The
// resource and the group's byte shift are wave-uniform and worked out once per group
// (group_source); each load then costs one vector add.  A paged group that straddles the end of
// the context (once per sequence and stream) takes per-lane addresses instead.
struct GroupSource {
  const uint16_t* base;  // what the resource starts at
  int bytes;             // its size
  int shift;             // byte offset of the group's first row from `base`
  bool straddles;        // paged: the group holds both cache and chunk rows
  const uint16_t* page;  // paged: the group's first row in the cache page
};

template <bool PAGED>
__device__ __forceinline__ GroupSource group_source(const uint16_t* src, const uint16_t* cache, int row0, int rows,
                                                    int n_k, int qoff, int stride, int page, int head_off) {
  const int row_bytes = stride * 2;
  GroupSource gs{src, (n_k - qoff) * row_bytes, (row0 - qoff) * row_bytes, false, nullptr};
  if constexpr (PAGED) {
    if (row0 < qoff) {
      gs.page = cache + ((size_t)page * kPageTokens + row0 % kPageTokens) * stride + head_off;
      gs.straddles = row0 + rows > qoff;
      gs.base = gs.page;
      gs.bytes = rows * row_bytes;
      gs.shift = 0;
    }
  }
  return gs;
}

// STRADDLE selects the path of a straddling paged group; callers branch once per group, not per load.
template <bool PAGED, bool STRADDLE>
__device__ __forceinline__ void group_load(PAA_LDS void* dst, const GroupSource& gs, const uint16_t* src, int row0,
                                           int dr, uint32_t off, int n_k, int qoff, int stride) {
  static_assert(PAGED || !STRADDLE, "only paged groups straddle");
  if constexpr (!STRADDLE) {
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)gs.base, (short)0, gs.bytes, kRawBufferWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, (int)(off + (uint32_t)gs.shift), 0, 0, 0);
  } else {
    // chunk rows at or past n_k repeat row n_k - 1
    const int key = min(row0 + dr, n_k - 1);
    const char* p = key < qoff ? (const char*)gs.page + off
                               : (const char*)(src + (size_t)(key - qoff) * stride) + (off - (uint32_t)(dr * stride * 2));
    __builtin_amdgcn_global_load_lds((const void*)p, dst, 16, 0, 0);
  }
}

// Appending a workgroup's chunk rows (its KV head, its query tile) to the caches.  One workgroup per
// (sequence, KV head, query tile) does it, the one holding the head group's first query heads, so
// every new row is written exactly once.  No workgroup of the launch reads cache positions at or
// past ctx (they read the chunk from k / v), so the writes race with nothing and can go out at any
// time: the kernels issue the reads with their first loads and the writes once those have landed,
// which keeps the append off the end of the workgroup.  Every thread moves up to kPer 16-byte
// pieces; load() issues all of a thread's reads at once (the chunk rows always exist, so the data
// loads do not wait for the page ids), store() writes the pieces whose page id lies in the pool.
template <int D, int ROWS, int THREADS>
struct ChunkAppend {
  static constexpr int kChunks = D / 8;  // 16-byte pieces per row
  static constexpr int kPer = (2 * ROWS * kChunks + THREADS - 1) / THREADS;
  u32x4_t val[kPer];
  uint16_t* dst[kPer];

  __device__ __forceinline__ void load(const PrefillArgs& a, const uint16_t* kh, const uint16_t* vh, size_t kv_stride,
                                       int b, int g, int q0_tile, int rows, int qoff, int tid) {
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int e = tid + r * THREADS;
      dst[r] = nullptr;
      if (e < 2 * rows * kChunks) {
        const bool is_v = e >= rows * kChunks;
        const int f = is_v ? e - rows * kChunks : e;
        const int i = q0_tile + f / kChunks;  // chunk row
        const int c = f % kChunks;
        const int pos = qoff + i;
        const int blk = pos / kPageTokens;
        const int page = blk < a.max_pages ? a.bt[(size_t)b * a.max_pages + blk] : -1;
        val[r] = *(const u32x4_t*)((is_v ? vh : kh) + (size_t)i * kv_stride + c * 8);
        if (page >= 0 && page < a.num_pages)
          dst[r] = (is_v ? a.vc : a.kc) + (((size_t)page * kPageTokens + pos % kPageTokens) * a.Hkv + g) * D + c * 8;
      }
    }
  }
  __device__ __forceinline__ void store() const {
#pragma unroll
    for (int r = 0; r < kPer; ++r)
      if (dst[r] != nullptr) *(u32x4_t*)dst[r] = val[r];
  }
};

template <int D, int MASK, int HPW, int WAVES, int RB, int STAGES>
__global__ __launch_bounds__(64 * WAVES, (RB == 1 ? 2 : 1)) void prefill_bf16_kernel(
    PrefillArgs a) {
  using T = TileLayout<D>;
  using C = PrefillCfg<D, WAVES, RB, STAGES>;
  constexpr bool CAUSAL = MASK != kMaskNone;
  constexpr bool WINDOW = MASK == kMaskWindow;
  constexpr bool PAGED = MASK == kMaskPaged;
  static_assert(!PAGED || STAGES == 2, "the paged page-id prefetch assumes two stages");
  constexpr int kWaveRows = C::kRowsPerWave;
  constexpr int kRowBlocks = WAVES / HPW;              // waves per head in a workgroup
  constexpr int kTileRows = kRowBlocks * kWaveRows;    // query rows per head in a workgroup
  constexpr int kKSteps = D / 16;                      // MFMA k-steps over the head dim
  constexpr int kDBlocks = D / 32;                     // 32-wide blocks of the head dim in O

  // K and V rings, one LDS object per stage, so the compiler can tell that loads landing in one
  // stage never alias the reads of another (stages beyond STAGES are never referenced).
  __shared__ __attribute__((aligned(1024))) char k_st0[T::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char k_st1[T::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char k_st2[T::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char k_st3[T::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_st0[T::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_st1[T::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_st2[T::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_st3[T::kTileBytes];
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
  using I0 = std::integral_constant<int, 0>;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // wave-uniform: group bases stay scalar
  const int lane = tid % 64;
  const int half = lane / 32;  // which half-wave
  const int l32 = lane % 32;
  const int gi = lane % 16;
  const int colhalf = (lane / 16) % 2;

  // ---- work unit (heaviest first) ----
  static_assert(4 * (kMaxRankedSeqs + 1) <= T::kTileBytes, "rank scratch fits a stage buffer");
  const WorkUnit wu = work_unit<HPW, PAGED>(a, (int)blockIdx.x, (PAA_LDS int*)k_st0);
  const int qt = wu.qt, hsub = wu.hsub, g = wu.g, b = wu.b;
  const int group = a.H / a.Hkv;

  const int head = g * group + hsub * HPW + wave / kRowBlocks;
  const int q0_tile = qt * kTileRows;
  const int q0 = q0_tile + (wave % kRowBlocks) * kWaveRows;  // first row of this wave; block rb starts at q0 + 32rb

  // Geometry of this unit: n_q query rows, n_k keys, query row i at key position qoff + i.  The
  // rows of Q / O / LSE and of K / V are q_stride / kv_stride elements apart.
  const size_t N = a.N;
  int n_q = a.N, n_k = a.N, qoff = 0;
  size_t q_base, kv_base, q_stride = D, kv_stride = D;
  if constexpr (PAGED) {
    const int lo = a.q_start[b];
    n_q = a.q_start[b + 1] - lo;
    qoff = max(a.ctx_lens[b], 0);
    n_k = qoff + n_q;
    if (q0_tile >= n_q) return;  // the whole workgroup: this sequence's chunk is shorter
    q_base = (size_t)lo * a.H * D + (size_t)head * D;
    q_stride = (size_t)a.H * D;
    kv_base = (size_t)lo * a.Hkv * D + (size_t)g * D;  // chunk row 0 of k / v
    kv_stride = (size_t)a.Hkv * D;
  } else {
    q_base = ((size_t)b * a.H + head) * N * D;
    kv_base = ((size_t)b * a.Hkv + g) * N * D;
  }
  const uint16_t* qh = a.q + q_base;
  const uint16_t* kh = a.k + kv_base;
  const uint16_t* vh = a.v + kv_base;

  // ---- key tiles ----
  // The workgroup visits key tiles [0, n_glob) and then [j_win, n_tiles) in order; iteration t
  // is tile tile_of(t).  Without a window every tile up to the causal limit is visited.  With one,
  // the tiles between the global tokens and the left edge of the workgroup's lowest row's window
  // hold no visible key and are never loaded.  This wave computes iterations [0, n_act).
  const int kv_end = CAUSAL ? min(n_k, qoff + q0_tile + kTileRows) : n_k;
  const int n_tiles = (kv_end + kBc - 1) / kBc;
  int n_glob = 0, j_win = 0;
  if constexpr (WINDOW) {
    n_glob = min(n_tiles, (a.n_global + kBc - 1) / kBc);
    j_win = max(n_glob, max(0, q0_tile - a.window + 1) / kBc);
  }
  const int n_iter = n_glob + (n_tiles - j_win);
  auto tile_of = [&](int t) __attribute__((always_inline)) { return t < n_glob ? t : j_win + (t - n_glob); };
  const int last_tile = CAUSAL ? min(n_tiles - 1, (qoff + q0 + kWaveRows - 1) / kBc) : n_tiles - 1;
  const int n_act = last_tile < n_glob ? last_tile + 1 : n_glob + max(0, last_tile - j_win + 1);

  // ---- direct global -> LDS load of one tile of K or V; this wave fetches kBlocksPerWave 1 KB blocks ----
  // Paged: the rows this wave fetches lie in one cache page (kWavePage of the tile's four), whose id
  // `page` the caller looked up; positions before qoff come from the cache, the rest from the chunk.
  constexpr int kGroupRows = C::kBlocksPerWave * T::kRowsPerBlock;  // consecutive tile rows one wave loads
  const int group_r0 = wave * kGroupRows;                            // the first of them
  static_assert(kPageTokens % kGroupRows == 0, "a wave's rows of a tile lie in one page");
  const int wave_page = group_r0 / kPageTokens;
  auto dma = [&](const uint16_t* src, uint16_t* cache, int j, int page, PAA_LDS char* dst) __attribute__((always_inline)) {
    const int row0 = j * kBc + group_r0;
    const GroupSource gs = group_source<PAGED>(src, cache, row0, kGroupRows, n_k, qoff, (int)kv_stride, page, g * D);
    auto loads = [&](auto straddle_tag) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < C::kBlocksPerWave; ++i) {
        const int blk = wave * C::kBlocksPerWave + i;
        const int dr = i * T::kRowsPerBlock + lane / T::kCpr;  // tile row written by this lane: group_r0 + dr
        const int c = (lane % T::kCpr) ^ swz<D>(group_r0 + dr);  // data chunk stored at this lane's position
        const uint32_t off = (uint32_t)((dr * kv_stride + c * 8) * 2);
        group_load<PAGED, decltype(straddle_tag)::value>((PAA_LDS void*)(dst + blk * 1024), gs, src, row0, dr, off,
                                                         n_k, qoff, (int)kv_stride);
      }
    };
    if constexpr (PAGED) {
      if (gs.straddles) loads(std::true_type{});
      else loads(std::false_type{});
    } else {
      loads(std::false_type{});
    }
  };
  // cache page holding this wave's rows of tile j (0 when not paged); an id outside the pool is
  // clamped into it, so no access leaves the pool (such a table gives unspecified results).
  // Lane k of pw holds the page of tile pw_t0 + k, so most lookups are a lane read; a refill (once
  // per 64 tiles, or at the jump to a window) is one vector load used at once.  Paged runs use two
  // stages, whose every tile ends with vmcnt(0), so the refill leaves the ring's waits exact.
  int pw = 0, pw_t0 = -(1 << 30);
  auto page_of = [&](int j) __attribute__((always_inline)) -> int {
    if constexpr (PAGED) {
      if (j < pw_t0 || j >= pw_t0 + 64) {
        pw_t0 = j;
        const int blk = min((j + lane) * (kBc / kPageTokens) + wave_page, a.max_pages - 1);
        pw = min(max(a.bt[(size_t)b * a.max_pages + blk], 0), a.num_pages - 1);
        return __builtin_amdgcn_readfirstlane(pw);
      }
      return __builtin_amdgcn_readlane(pw, j - pw_t0);
    } else {
      return 0;
    }
  };

  // ---- paged: the append's reads go out first; its writes follow once the prologue has landed ----
  ChunkAppend<D, kTileRows, 64 * WAVES> app;
  if constexpr (PAGED)
    if (hsub == 0) app.load(a, kh, vh, kv_stride, b, g, q0_tile, min(kTileRows, n_q - q0_tile), qoff, tid);

  // prologue loads: K_0 .. K_{STAGES-1} and V_0 .. V_{STAGES-2}
  auto prologue = [&](auto i_tag, int j) __attribute__((always_inline)) {
    const int page = page_of(j);
    dma(kh, a.kc, j, page, kst(i_tag));
    if (decltype(i_tag)::value + 1 < STAGES) dma(vh, a.vc, j, page, vst(i_tag));
  };
  auto prologue_t = [&](auto i_tag, int t) __attribute__((always_inline)) { prologue(i_tag, tile_of(t)); };
  for_stages<0, STAGES>(prologue_t, 0, n_iter);
  // page ids for the first refills (K of iteration STAGES, V of iteration STAGES - 1), then one
  // iteration ahead of use inside the loop
  int page_k = page_of(tile_of(min(STAGES, n_iter - 1)));
  int page_v = page_of(tile_of(min(STAGES - 1, n_iter - 1)));

  // ---- Q fragments (B operand of S^T = K Q^T): row q0 + 32rb + l32, d = 16t + 8*half + 0..7 ----
  u32x4_t qf[RB][kKSteps];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = q0 + 32 * rb + l32;
#pragma unroll
    for (int t = 0; t < kKSteps; ++t) {
      if (row < n_q)
        qf[rb][t] = *(const u32x4_t*)(qh + (size_t)row * q_stride + 16 * t + 8 * half);
      else
        qf[rb][t] = u32x4_t{0, 0, 0, 0};
    }
  }

  // ---- per-lane LDS byte offsets inside a tile ----
  // K (A operand of the score MFMA): row l32 (+32 for the second key block), chunk 2t + half
  int koff[kKSteps];
#pragma unroll
  for (int t = 0; t < kKSteps; ++t) koff[t] = l32 * T::kRowBytes + (((2 * t + half) ^ swz<D>(l32)) * 16);
  // V (transposed reads): row 4*half + gi/4 (+8 for the second read, +16 per k-step), 8 bytes at column
  // 32*db + 16*colhalf + 4*(gi%4)
  int voff[kDBlocks][2];
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 4 * half + gi / 4 + 8 * e;
      const int col = 32 * db + 16 * colhalf + 4 * (gi % 4);
      voff[db][e] = r * T::kRowBytes + (((col / 8) ^ swz<D>(r)) * 16) + (col % 8) * 2;
    }

  // S^T of one tile for every row block: block (rb, mb) holds keys k0 + 32mb + 8(i/4) + 4*half + i%4
  // of query row q0 + 32rb + l32.  Each K fragment read from LDS feeds RB MFMAs.
  auto scores = [&](const PAA_LDS char* kt, f32x16_t (&s)[RB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int t = 0; t < kKSteps; ++t) {
        const u32x4_t kf = *(const PAA_LDS u32x4_t*)(kt + koff[t] + mb * 32 * T::kRowBytes);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          s[rb][mb] = t == 0 ? mfma32x32x16(kf, qf[rb][t], f32x16_t{}) : mfma32x32x16(kf, qf[rb][t], s[rb][mb]);
      }
    }
  };

  // ---- running state of the lane's row in each block ----
  // reference maximum of raw scores (before scale); this lane's share of the sum of the probabilities
  // (for the LSE) and of the same probabilities as rounded to bf16 (for O, whose numerator uses them)
  float m_run[RB], l_run[RB], lr_run[RB];
  f32x16_t acc[RB][kDBlocks];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
    lr_run[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
      for (int i = 0; i < 16; ++i) acc[rb][db][i] = 0.f;
  }

  // Softmax of tile j, first half, for row block rb: the mask.  Returns -reference * scale_log2, the
  // exponent shift of this tile.  The reference only has to keep the numbers finite: it moves (see
  // rescale) when some lane's share of a tile's probabilities exceeds kMaxTileSum or is not finite,
  // as on a row's first visible tile while the reference is still -inf.  No row maximum is taken
  // otherwise; numerator and both sums share the reference, so the result is the same softmax.
  auto softmax_prep = [&](int j, int rb, f32x16_t (&s)[2]) __attribute__((always_inline)) -> float {
    const int k0 = j * kBc;
    const int rq0 = qoff + q0 + 32 * rb;  // key position of the block's first query row
    // mask: causal keys after the row, keys past the end of the sequence and, with a window, keys
    // left of the row's window that are not global tokens
    const bool need_window = WINDOW && (k0 <= rq0 + 31 - a.window) && (k0 + kBc - 1 >= a.n_global);
    const bool need_mask = (CAUSAL && (k0 + kBc - 1 > rq0)) || (k0 + kBc > n_k) || need_window;
    if (need_mask) {
      // element i of block mb holds key k0 + 4 half + c, c = 32 mb + 8 (i / 4) + i % 4 (a constant);
      // compare c with per-lane bounds relative to k0 + 4 half
      const int row = rq0 + l32;
      const int base = k0 + 4 * half;
      const int lim = (CAUSAL ? min(row, n_k - 1) : n_k - 1) - base;
      const int win = row - a.window - base, glob = a.n_global - base;  // hidden if c <= win and c >= glob
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = 32 * mb + 8 * (i / 4) + (i % 4);
          const bool out_of_window = WINDOW && c <= win && c >= glob;
          if (c > lim || out_of_window) s[mb][i] = -INFINITY;
        }
    }
    return -m_run[rb] * a.scale_log2;  // +inf while the reference is still -inf
  };

  // Moves the reference of row block rb to kRefHeadroomLog2 above the exact running maximum (unless it
  // already sits higher) and rescales the state; returns the new shift.
  auto rescale = [&](int rb, const f32x16_t (&s)[2]) __attribute__((always_inline)) -> float {
    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[mb][i]);
    tmax = fmaxf(tmax, swap_halves(tmax, half));
    const float m_new = fmaxf(m_run[rb], tmax + a.ref_headroom);
    const float alpha = m_new == -INFINITY ? 1.f : fast_exp2((m_run[rb] - m_new) * a.scale_log2);
    m_run[rb] = m_new;
    l_run[rb] *= alpha;
    lr_run[rb] *= alpha;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rb][db][i] *= alpha;
    return m_new == -INFINITY ? 0.f : -m_new * a.scale_log2;
  };

  // Softmax of tile j, second half (no branches, so it can interleave with MFMAs): probabilities
  // relative to the reference and the bf16 B operands of the PV product; returns this lane's share of
  // the tile's probabilities (the sums are only added once the tile is accepted).
  auto softmax_exp = [&](const f32x16_t (&s)[2], float neg_ms, u32x4_t (&pf)[4]) __attribute__((always_inline))
      -> float {
    float lt = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = fast_exp2(fmaf(s[mb][i], a.scale_log2, neg_ms));
        lt = (mb == 0 && i == 0) ? p[i] : lt + p[i];
      }
#pragma unroll
      for (int sh = 0; sh < 2; ++sh)
        pf[2 * mb + sh] = u32x4_t{pack_bf16x2(p[8 * sh + 0], p[8 * sh + 1]), pack_bf16x2(p[8 * sh + 2], p[8 * sh + 3]),
                                  pack_bf16x2(p[8 * sh + 4], p[8 * sh + 5]), pack_bf16x2(p[8 * sh + 6], p[8 * sh + 7])};
    }
    return lt;
  };

  // O^T += V^T P^T for every row block.  PV k-step ks covers keys 16ks..16ks+15 of the tile; logical
  // k = 8*half + jj maps to key 16ks + 8(jj/4) + 4*half + jj%4.  Each A operand (two transposed reads)
  // feeds RB MFMAs.
  auto pv = [&](const PAA_LDS char* vt, const u32x4_t (&pf)[RB][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x2_t lo = lds_read_tr16((const PAA_LDS uint16_t*)(vt + voff[db][0] + 16 * ks * T::kRowBytes));
        const u32x2_t hi = lds_read_tr16((const PAA_LDS uint16_t*)(vt + voff[db][1] + 16 * ks * T::kRowBytes));
        const u32x4_t vf = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb][db] = mfma32x32x16(vf, pf[rb][ks], acc[rb][db]);
      }
    }
  };

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if constexpr (PAGED)
    if (hsub == 0) app.store();
  f32x16_t s_cur[RB][2];
  scores(kst(I0{}), s_cur);  // tile 0 is visible to every row
  __syncthreads();           // everyone is done with K stage 0 before it is refilled

  // Tile j (stage ST = j % STAGES, a template constant, so every LDS address is a register offset
  // plus an immediate): loads of K_{j+STAGES} and V_{j+STAGES-1} go out first, into the stages that
  // held K_j and V_{j-1}; then the scores of tile j+1 (MFMA) sit in one branch-free block with the
  // exponentials of tile j (VALU) and O += P_j V_j.
  auto tile = [&](auto st_tag, int j) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_tag)::value;
    using Next = std::integral_constant<int, ST + 1>;
    using Prev = std::integral_constant<int, ST + STAGES - 1>;
    // near the end the loads repeat the last tile (cached, and never read): issuing them every time
    // keeps the count of loads in flight fixed, so the waits below stay exact
    dma(kh, a.kc, tile_of(min(j + STAGES, n_iter - 1)), page_k, kst(st_tag));
    dma(vh, a.vc, tile_of(min(j + STAGES - 1, n_iter - 1)), page_v, vst(Prev{}));
    if constexpr (PAGED) {  // next iteration's ids; the load retires with this tile's DMA wait
      page_v = page_k;
      page_k = page_of(tile_of(min(j + STAGES + 1, n_iter - 1)));
    }
    if (j < n_act) {
      float neg_ms[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) neg_ms[rb] = softmax_prep(tile_of(j), rb, s_cur[rb]);
      // scores of tile j+1 are computed even past the last active tile, where they are dropped
      f32x16_t s_nxt[RB][2];
      scores(kst(Next{}), s_nxt);
      u32x4_t pf[RB][4];
      float lt[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) lt[rb] = softmax_exp(s_cur[rb], neg_ms[rb], pf[rb]);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (__builtin_amdgcn_ballot_w64(!(lt[rb] <= kMaxTileSum)) != 0)
          lt[rb] = softmax_exp(s_cur[rb], rescale(rb, s_cur[rb]), pf[rb]);
        l_run[rb] += lt[rb];
        lr_run[rb] = add_bf16x16(pf[rb], lr_run[rb]);
      }
      pv(vst(st_tag), pf);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) s_cur[rb][mb] = s_nxt[rb][mb];
    }
    // K_{j+2} and V_{j+1} have landed (own loads, then everyone's) and every wave is done with the
    // stages the next tile refills
    wait_vmcnt<C::kInFlightAfter>();
    tile_barrier();
  };

  for (int j = 0; j < n_iter; j += STAGES) for_stages<0, STAGES>(tile, j, n_iter);
  wait_vmcnt<0>();  // no load may still be writing this workgroup's LDS when it exits

  // ---- epilogue: O = acc / (sum of the rounded probabilities), LSE = scale * m + ln(l) ----
  // O leaves through LDS (store_o_tile); wave w stages each of its row blocks in half of one stage
  // array, once every wave is past its last tile (every load landed, every tile read done).
  static_assert(RB == 1 && WAVES <= 2 * 2 * STAGES, "each wave's O tile is half of its own stage array");
  __syncthreads();
  PAA_LDS char* ot = (wave / 2 == 0   ? (PAA_LDS char*)k_st0
                      : wave / 2 == 1 ? (PAA_LDS char*)k_st1
                      : wave / 2 == 2 ? (PAA_LDS char*)v_st0
                                      : (PAA_LDS char*)v_st1) + (wave % 2) * (32 * T::kRowBytes);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = q0 + 32 * rb + l32;
    const float l_tot = l_run[rb] + swap_halves(l_run[rb], half);
    const float inv_l = 1.f / (lr_run[rb] + swap_halves(lr_run[rb], half));
    store_o_tile<D>(ot, acc[rb], inv_l, lane, a.o + q_base + (size_t)(q0 + 32 * rb) * q_stride, q_stride,
                    n_q - q0 - 32 * rb);
    if (row < n_q) {
      if (a.lse != nullptr && half == 0) {
        const size_t li = PAGED ? q_base / D + (size_t)row * a.H : ((size_t)b * a.H + head) * N + row;
        a.lse[li] = a.scale * m_run[rb] + __logf(l_tot);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Ping-pong variant: 8 waves in two groups of 4 (waves w and w + 4 share a SIMD).  A wave's
// work per key tile is an MFMA phase (scores of tile i, and O += P V of tile i - 1) and a VALU
// phase (mask, exponentials and row sums of tile i).  A single wave cannot overlap its own MFMA
// and VALU work, but a SIMD overlaps an MFMA wave with a VALU wave, so group B runs one phase
// behind group A: in every period one group is in its MFMA phase and the other in its VALU
// phase, and a workgroup barrier ends each period.  Stage s of the LDS ring holds K_s and
// V_{s-1}; both groups read it in periods 2s (A) and 2s + 1 (B), and its refill with stage
// s + STAGES goes out at the start of period 2s + 2.  Every mask of the lock-step kernel is
// supported, the chunked prefill over the paged cache (with its append) included.
//
// Split-key mode (KSPLIT): both groups take the same query rows, group A the even key tiles and
// group B the odd ones, so a short causal sequence's longest rows walk half as many tiles per
// wave.  Stage s then holds K of tiles 2s and 2s + 1 and V of tiles 2s - 2 and 2s - 1 (group g's
// in slot g of the stage); at the end group B hands its (reference max, partial sum,
// accumulator) to group A through LDS, and group A merges them with the rescaling identity of
// the online softmax and writes the rows.
template <int D, int MASK, int HPW, int STAGES, bool KSPLIT = false>
__global__ __launch_bounds__(512, 1) void prefill_pp_kernel(PrefillArgs a) {
  constexpr int WAVES = 8;
  using T = TileLayout<D>;
  constexpr bool CAUSAL = MASK != kMaskNone;
  constexpr bool WINDOW = MASK == kMaskWindow;
  constexpr bool PAGED = MASK == kMaskPaged;
  static_assert(!(KSPLIT && (WINDOW || PAGED)), "split keys: plain and causal masks only");
  static_assert(!PAGED || STAGES == 2, "the paged page-id prefetch assumes two stages");
  constexpr int kRowWaves = KSPLIT ? WAVES / 2 : WAVES;  // waves holding distinct query rows
  constexpr int kRowBlocks = kRowWaves / HPW;          // waves per head in a workgroup
  constexpr int kTileRows = kRowBlocks * 32;           // query rows per head in a workgroup
  constexpr int kKSteps = D / 16;
  constexpr int kDBlocks = D / 32;
  constexpr int kSlots = KSPLIT ? 2 : 1;               // K (and V) tiles per stage
  constexpr int kLoadsPerStage = 2 * kSlots * T::kBlocks / WAVES;
  static_assert((2 * kSlots * T::kBlocks) % WAVES == 0, "tile rows must split evenly over the waves");
  static_assert(STAGES >= 2 && STAGES <= 4, "2 to 4 stages");

  __shared__ __attribute__((aligned(1024))) char k_st0[kSlots * T::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char k_st1[kSlots * T::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char k_st2[kSlots * T::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char k_st3[kSlots * T::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_st0[kSlots * T::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_st1[kSlots * T::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_st2[kSlots * T::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char v_st3[kSlots * T::kTileBytes];
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
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // wave-uniform, so phase branches are scalar
  const int grp = wave / 4;   // 0: group A (leads), 1: group B (one phase behind)
  const int lane = tid % 64;
  const int half = lane / 32;
  const int l32 = lane % 32;
  const int gi = lane % 16;
  const int colhalf = (lane / 16) % 2;

  // ---- work unit (heaviest first) ----
  static_assert(4 * (kMaxRankedSeqs + 1) <= T::kTileBytes, "rank scratch fits a stage buffer");
  const WorkUnit wu = work_unit<HPW, PAGED>(a, (int)blockIdx.x, (PAA_LDS int*)k_st0);
  const int qt = wu.qt, hsub = wu.hsub, g = wu.g, b = wu.b;
  const int group = a.H / a.Hkv;

  const int wrow = KSPLIT ? wave % kRowWaves : wave;  // this wave's row block among the workgroup's
  const int head = g * group + hsub * HPW + wrow / kRowBlocks;
  const int q0_tile = qt * kTileRows;
  const int q0 = q0_tile + (wrow % kRowBlocks) * 32;

  // Geometry (as in the lock-step kernel): n_q query rows, n_k keys, query row i at key position
  // qoff + i; rows of Q / O / LSE and of K / V are q_stride / kv_stride elements apart.
  const size_t N = a.N;
  int n_q = a.N, n_k = a.N, qoff = 0;
  size_t q_base, kv_base, q_stride = D, kv_stride = D;
  if constexpr (PAGED) {
    const int lo = a.q_start[b];
    n_q = a.q_start[b + 1] - lo;
    qoff = max(a.ctx_lens[b], 0);
    n_k = qoff + n_q;
    if (q0_tile >= n_q) return;  // the whole workgroup: this sequence's chunk is shorter
    q_base = (size_t)lo * a.H * D + (size_t)head * D;
    q_stride = (size_t)a.H * D;
    kv_base = (size_t)lo * a.Hkv * D + (size_t)g * D;
    kv_stride = (size_t)a.Hkv * D;
  } else {
    q_base = ((size_t)b * a.H + head) * N * D;
    kv_base = ((size_t)b * a.Hkv + g) * N * D;
  }
  const uint16_t* qh = a.q + q_base;
  const uint16_t* kh = a.k + kv_base;
  const uint16_t* vh = a.v + kv_base;

  // ---- key tiles: iteration t is tile tile_of(t); this wave computes iterations [0, n_act) ----
  const int kv_end = CAUSAL ? min(n_k, qoff + q0_tile + kTileRows) : n_k;
  const int n_tiles = (kv_end + kBc - 1) / kBc;
  int n_glob = 0, j_win = 0;
  if constexpr (WINDOW) {
    n_glob = min(n_tiles, (a.n_global + kBc - 1) / kBc);
    j_win = max(n_glob, max(0, q0_tile - a.window + 1) / kBc);
  }
  const int n_iter = n_glob + (n_tiles - j_win);
  auto tile_of = [&](int t) __attribute__((always_inline)) { return t < n_glob ? t : j_win + (t - n_glob); };
  const int last_tile = CAUSAL ? min(n_tiles - 1, (qoff + q0 + 31) / kBc) : n_tiles - 1;
  // iteration i of this wave works on key tile key_tile(i) (tile_of(i), or 2i + grp when split);
  // it computes iterations [0, n_act) of the n_loop the workgroup runs
  int n_act, n_loop;
  if constexpr (KSPLIT) {
    n_act = last_tile >= grp ? (last_tile - grp) / 2 + 1 : 0;
    n_loop = (n_iter + 1) / 2;
  } else {
    n_act = last_tile < n_glob ? last_tile + 1 : n_glob + max(0, last_tile - j_win + 1);
    n_loop = n_iter;
  }
  auto key_tile = [&](int i) __attribute__((always_inline)) { return KSPLIT ? 2 * i + grp : tile_of(i); };

  // One 1 KB block of a stage: block u of the list [K slot 0, (K slot 1,) V slot 0, (V slot 1)];
  // slot t of a stage holds tile j + t.
  // Paged: a wave's rows of a tile lie in one 16-token page, whose id `page` the caller looked up;
  // positions before qoff come from the cache, the rest from the chunk.
  // The blocks a wave loads in one stage are consecutive rows of one slot (K or V); paged, they
  // also lie in one page.
  constexpr int kGroupRows = kLoadsPerStage * T::kRowsPerBlock;
  static_assert(T::kBlocks % kLoadsPerStage == 0, "a wave's blocks of a stage lie in one slot");
  static_assert(!PAGED || kGroupRows <= kPageTokens, "a wave's rows of a stage lie in one page");
  const bool loads_v = wave * kLoadsPerStage >= kSlots * T::kBlocks;
  const int w0 = loads_v ? wave * kLoadsPerStage - kSlots * T::kBlocks : wave * kLoadsPerStage;
  const int load_slot = w0 / T::kBlocks;
  const int group_r0 = (w0 % T::kBlocks) * T::kRowsPerBlock;  // first tile row of the wave's group
  const int wave_page = group_r0 / kPageTokens;
  const uint16_t* load_src = loads_v ? vh : kh;
  auto load_block = [&](auto straddle_tag, int i, int row0, const GroupSource& gs, PAA_LDS char* kdst, PAA_LDS char* vdst) __attribute__((always_inline)) {
    const int dr = i * T::kRowsPerBlock + lane / T::kCpr;   // tile row written by this lane: group_r0 + dr
    const int c = (lane % T::kCpr) ^ swz<D>(group_r0 + dr);
    const uint32_t off = (uint32_t)((dr * kv_stride + c * 8) * 2);
    PAA_LDS char* dst = (loads_v ? vdst : kdst) + load_slot * T::kTileBytes + (group_r0 / T::kRowsPerBlock + i) * 1024;
    group_load<PAGED, decltype(straddle_tag)::value>((PAA_LDS void*)dst, gs, load_src, row0, dr, off, n_k, qoff,
                                                     (int)kv_stride);
  };
  // Paged: lane k of pw holds the page of this wave's rows of tile pw_t0 + k, so a tile's page is a
  // lane read.  A scalar load per tile would be retired by the next tile barrier's lgkmcnt(0) and
  // stall every period on its latency (400 against 316 us for chunked prefill with no lookup).  A
  // refill (once per 64 tiles) is one vector load whose value is used at once; paged runs use two
  // stages, whose every pair ends with vmcnt(0), so it leaves the ring's exact waits intact.
  int pw = 0, pw_t0 = -(1 << 30);
  auto page_of = [&](int j) __attribute__((always_inline)) -> int {  // page of this wave's rows of tile j
    if constexpr (PAGED) {
      if (j < pw_t0 || j >= pw_t0 + 64) {
        pw_t0 = j;
        const int blk = min((j + lane) * (kBc / kPageTokens) + wave_page, a.max_pages - 1);
        pw = min(max(a.bt[(size_t)b * a.max_pages + blk], 0), a.num_pages - 1);
        return __builtin_amdgcn_readfirstlane(pw);
      }
      return __builtin_amdgcn_readlane(pw, j - pw_t0);
    } else {
      return 0;
    }
  };
  // stage s: K of iteration s and V of iteration s - 1; iterations past the end repeat the last
  // one (the buffer is free and never read), so every stage issues the same number of loads
  auto stage_tiles = [&](int s, int& jk, int& jv) __attribute__((always_inline)) {
    if constexpr (KSPLIT) {  // pairs of tiles; the last pair may reach one tile past the end (masked)
      jk = 2 * min(s, n_loop - 1);
      jv = 2 * min(max(s - 1, 0), n_loop - 1);
    } else {
      jk = tile_of(min(s, n_iter - 1));
      jv = tile_of(min(max(s - 1, 0), n_iter - 1));
    }
  };
  // the page id of this wave's rows of stage s (0 when not paged)
  auto stage_page = [&](int s) __attribute__((always_inline)) -> int {
    int jk, jv;
    stage_tiles(s, jk, jv);
    return page_of(loads_v ? jv : jk);
  };
  int page_next = 0;  // paged: the page id of the next refill, loaded one refill ahead
  auto issue_stage = [&](auto s_tag, int s, int page) __attribute__((always_inline)) {
    using Prev = std::integral_constant<int, decltype(s_tag)::value + STAGES - 1>;
    int jk, jv;
    stage_tiles(s, jk, jv);
    const int row0 = ((loads_v ? jv : jk) + load_slot) * kBc + group_r0;
    const GroupSource gs = group_source<PAGED>(load_src, loads_v ? a.vc : a.kc, row0, kGroupRows, n_k, qoff,
                                               (int)kv_stride, page, g * D);
    auto loads = [&](auto straddle_tag) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < kLoadsPerStage; ++i) load_block(straddle_tag, i, row0, gs, kst(s_tag), vst(Prev{}));
    };
    if constexpr (PAGED) {
      if (gs.straddles) loads(std::true_type{});
      else loads(std::false_type{});
    } else {
      loads(std::false_type{});
    }
  };

  // ---- paged: the append's reads go out first; its writes follow once the first stage has landed ----
  ChunkAppend<D, kTileRows, 512> app;
  if constexpr (PAGED)
    if (hsub == 0) app.load(a, kh, vh, kv_stride, b, g, q0_tile, min(kTileRows, n_q - q0_tile), qoff, tid);
  // ---- Q first, through the idle ring: each wave's 32 rows go to half of one stage array by direct
  // loads (whole rows per instruction, chunk-swizzled as the K tiles are), reach the VGPRs (the MFMA
  // B operand) once landed, and the ring is refilled only after every wave has read its rows ----
  u32x4_t qf[kKSteps];
  if constexpr (KSPLIT) {
    const int row = q0 + l32;
#pragma unroll
    for (int t = 0; t < kKSteps; ++t) {
      if (row < n_q)
        qf[t] = *(const u32x4_t*)(qh + (size_t)row * q_stride + 16 * t + 8 * half);
      else
        qf[t] = u32x4_t{0, 0, 0, 0};
    }
  } else {
    PAA_LDS char* qs = (wave / 2 == 0   ? (PAA_LDS char*)k_st0
                        : wave / 2 == 1 ? (PAA_LDS char*)k_st1
                        : wave / 2 == 2 ? (PAA_LDS char*)v_st0
                                        : (PAA_LDS char*)v_st1) + (wave % 2) * (32 * T::kRowBytes);
    const int rows = max(0, min(32, n_q - q0));
    const int bytes = rows > 0 ? (int)(((size_t)(rows - 1) * q_stride + D) * 2) : 0;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(qh + (size_t)max(0, min(q0, n_q)) * q_stride), (short)0, bytes,
                                          kRawBufferWord3);
#pragma unroll
    for (int k = 0; k < 32 / T::kRowsPerBlock; ++k) {
      const int r = k * T::kRowsPerBlock + lane / T::kCpr;
      const int c = (lane % T::kCpr) ^ swz<D>(r);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (PAA_LDS void*)(qs + k * 1024), 16,
                                               (int)((r * q_stride + c * 8) * 2), 0, 0, 0);
    }
    wait_vmcnt<0>();
#pragma unroll
    for (int t = 0; t < kKSteps; ++t)
      qf[t] = *(const PAA_LDS u32x4_t*)(qs + l32 * T::kRowBytes + (((2 * t + half) ^ swz<D>(l32)) * 16));
    __syncthreads();  // every wave holds its Q before the ring's first loads overwrite it
  }
  // prologue: stages 0 .. STAGES-1 (stage 0's V half repeats tile 0 into a free buffer)
  issue_stage(std::integral_constant<int, 0>{}, 0, stage_page(0));
  auto prologue = [&](auto s_tag, int s) __attribute__((always_inline)) { issue_stage(s_tag, s, stage_page(s)); };
  for_stages<1, STAGES>(prologue, 0, STAGES);
  if constexpr (PAGED) page_next = stage_page(STAGES);

  int koff[kKSteps];
#pragma unroll
  for (int t = 0; t < kKSteps; ++t) koff[t] = l32 * T::kRowBytes + (((2 * t + half) ^ swz<D>(l32)) * 16);
  int voff[kDBlocks][2];
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 4 * half + gi / 4 + 8 * e;
      const int col = 32 * db + 16 * colhalf + 4 * (gi % 4);
      voff[db][e] = r * T::kRowBytes + (((col / 8) ^ swz<D>(r)) * 16) + (col % 8) * 2;
    }

  float m_run = -INFINITY, l_run = 0.f, lr_run = 0.f;  // lr: sum of the probabilities as rounded for P.V
  f32x16_t acc[kDBlocks];
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  f32x16_t s[2];
  u32x4_t pf[4];

  // MFMA phase of iteration i: S^T of iteration i (stage i's K) and O += P_{i-1} V_{i-1} (stage i's V)
  auto m_phase = [&](auto u_tag, int i) __attribute__((always_inline)) {
    using U = decltype(u_tag);
    using Prev = std::integral_constant<int, U::value + STAGES - 1>;
    const PAA_LDS char* kt = kst(U{}) + (KSPLIT ? grp * T::kTileBytes : 0);
    const PAA_LDS char* vt = vst(Prev{}) + (KSPLIT ? grp * T::kTileBytes : 0);
    // each block keeps its LDS reads a few ahead of its MFMAs (not all hoisted to the top, which
    // would take more registers than the wave has)
    if (i < n_act) {
#pragma unroll
      for (int t = 0; t < kKSteps; ++t)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const u32x4_t kf = *(const PAA_LDS u32x4_t*)(kt + koff[t] + mb * 32 * T::kRowBytes);
          s[mb] = t == 0 ? mfma32x32x16(kf, qf[t], f32x16_t{}) : mfma32x32x16(kf, qf[t], s[mb]);
        }
      constexpr int kLead = 4;
      __builtin_amdgcn_sched_group_barrier(0x100, kLead, 0);
#pragma unroll
      for (int k = 0; k < 2 * kKSteps - kLead; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kLead, 0);
    }
    if (i >= 1 && i - 1 < n_act) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db) {
          const u32x2_t lo = lds_read_tr16((const PAA_LDS uint16_t*)(vt + voff[db][0] + 16 * ks * T::kRowBytes));
          const u32x2_t hi = lds_read_tr16((const PAA_LDS uint16_t*)(vt + voff[db][1] + 16 * ks * T::kRowBytes));
          acc[db] = mfma32x32x16(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, pf[ks], acc[db]);
        }
      constexpr int kLead = 4;  // MFMAs whose two reads go out ahead
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kLead, 1);
#pragma unroll
      for (int k = 0; k < 4 * kDBlocks - kLead; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kLead, 1);
    }
  };

  // VALU phase of iteration i: mask, exponentials against the reference (rescaled only on overflow),
  // the two row sums, bf16 P
  auto v_phase = [&](int i) __attribute__((always_inline)) {
    if (i < 0 || i >= n_act) return;
    const int k0 = key_tile(i) * kBc;
    const bool need_window = WINDOW && (k0 <= q0 + 31 - a.window) && (k0 + kBc - 1 >= a.n_global);
    const bool need_mask = (CAUSAL && (k0 + kBc - 1 > qoff + q0)) || (k0 + kBc > n_k) || need_window;
    if (need_mask) {  // as in the lock-step kernel: constant offsets against per-lane bounds
      const int row = qoff + q0 + l32;  // key position of the lane's query row
      const int base = k0 + 4 * half;
      const int lim = (CAUSAL ? min(row, n_k - 1) : n_k - 1) - base;
      const int win = row - a.window - base, glob = a.n_global - base;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int c = 32 * mb + 8 * (e / 4) + (e % 4);
          const bool out_of_window = WINDOW && c <= win && c >= glob;
          if (c > lim || out_of_window) s[mb][e] = -INFINITY;
        }
    }
    // Probabilities against the current reference maximum, then the bf16 B operands of the next P.V.
    auto probs = [&](float neg_ms) __attribute__((always_inline)) -> float {
      float lt = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        float p[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          p[e] = fast_exp2(fmaf(s[mb][e], a.scale_log2, neg_ms));
          lt = (mb == 0 && e == 0) ? p[e] : lt + p[e];
        }
#pragma unroll
        for (int sh = 0; sh < 2; ++sh)
          pf[2 * mb + sh] = u32x4_t{pack_bf16x2(p[8 * sh + 0], p[8 * sh + 1]), pack_bf16x2(p[8 * sh + 2], p[8 * sh + 3]),
                                    pack_bf16x2(p[8 * sh + 4], p[8 * sh + 5]), pack_bf16x2(p[8 * sh + 6], p[8 * sh + 7])};
      }
      return lt;
    };
    // The reference only has to keep the numbers finite: it moves when some lane's share of this tile's
    // probabilities exceeds kMaxTileSum (or is not finite, as on a row's first visible tile, while the
    // reference is still -inf), and then to the exact running maximum.  No row maximum is taken
    // otherwise.  Numerator and both sums share the reference, so the result is the same softmax.
    float lt = probs(-m_run * a.scale_log2);
    if (__builtin_amdgcn_ballot_w64(!(lt <= kMaxTileSum)) != 0) {
      float tmax = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, s[mb][e]);
      tmax = fmaxf(tmax, swap_halves(tmax, half));
      const float m_new = fmaxf(m_run, tmax + a.ref_headroom);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2((m_run - m_new) * a.scale_log2);
      m_run = m_new;
      l_run *= alpha;
      lr_run *= alpha;
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[db][e] *= alpha;
      lt = probs(m_run == -INFINITY ? 0.f : -m_run * a.scale_log2);
    }
    l_run += lt;
    lr_run = add_bf16x16(pf, lr_run);
  };

  // Q and stage 0 have landed (loads after them: stages 1 .. STAGES-1)
  wait_vmcnt<(STAGES - 1) * kLoadsPerStage>();
  tile_barrier();
  if constexpr (PAGED)
    if (hsub == 0) app.store();

  // Periods 2i and 2i + 1 use stage i (u = i % STAGES).  Each group runs its own copy of the loop
  // (same barriers, in the same number), so the state flows straight from one phase to the next.
  auto run = [&](auto grp_tag) __attribute__((always_inline)) {
    constexpr bool kLead = decltype(grp_tag)::value == 0;
    auto period_pair = [&](auto u_tag, int i) __attribute__((always_inline)) {
      using U = decltype(u_tag);
      using Refill = std::integral_constant<int, U::value + STAGES - 1>;  // stage i - 1 + STAGES
      if (i >= 1) {
        issue_stage(Refill{}, i - 1 + STAGES, page_next);
        if constexpr (PAGED) page_next = stage_page(i + STAGES);  // retires with this pair's waits
      }
      if constexpr (kLead) m_phase(U{}, i); else v_phase(i - 1);
      tile_barrier();
      if constexpr (kLead) v_phase(i); else m_phase(U{}, i);
      wait_vmcnt<(STAGES - 2) * kLoadsPerStage>();  // stage i + 1 has landed
      tile_barrier();
    };
    for (int i0 = 0; i0 <= n_loop; i0 += STAGES) for_stages<0, STAGES>(period_pair, i0, n_loop + 1);
  };
  if (grp == 0)
    run(std::integral_constant<int, 0>{});
  else
    run(std::integral_constant<int, 1>{});
  wait_vmcnt<0>();  // no load may still be writing this workgroup's LDS when it exits

  if constexpr (KSPLIT) {
    // group B's partial state to group A, lane for lane (the same rows, the same accumulator
    // layout), through a stage buffer that is idle now: m, l, then the accumulators
    // one stage array per row block: K stages 0 and 1, then V stages 0 and 1
    constexpr int kPerWave = (3 + 16 * kDBlocks) * 64;  // floats
    static_assert(kPerWave * 4 <= kSlots * T::kTileBytes, "a row block's exchange fits in one stage array");
    static_assert(kRowWaves == 4 && STAGES >= 2, "four row blocks, four stage arrays");
    __syncthreads();  // every wave's loads have landed and every tile read is done
    PAA_LDS char* xbase = wrow == 0 ? (PAA_LDS char*)k_st0
                        : wrow == 1 ? (PAA_LDS char*)k_st1
                        : wrow == 2 ? (PAA_LDS char*)v_st0 : (PAA_LDS char*)v_st1;
    PAA_LDS float* xch = (PAA_LDS float*)xbase;
    if (grp == 1) {
      xch[lane] = m_run;
      xch[64 + lane] = l_run;
      xch[128 + lane] = lr_run;
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) xch[192 + (db * 16 + e) * 64 + lane] = acc[db][e];
    }
    __syncthreads();
    if (grp == 1) return;  // group A writes the rows
    const float mb = xch[lane];
    const float lb = xch[64 + lane];
    const float lrb = xch[128 + lane];
    const float m_new = fmaxf(m_run, mb);
    // a group that saw no visible key has m = -inf and contributes nothing
    const float fa = m_run == -INFINITY ? 0.f : fast_exp2((m_run - m_new) * a.scale_log2);
    const float fb = mb == -INFINITY ? 0.f : fast_exp2((mb - m_new) * a.scale_log2);
    m_run = m_new;
    l_run = l_run * fa + lb * fb;
    lr_run = lr_run * fa + lrb * fb;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[db][e] = acc[db][e] * fa + xch[192 + (db * 16 + e) * 64 + lane] * fb;
  }

  // ---- epilogue: O = acc / (sum of the rounded probabilities), LSE = scale * m + ln(l) ----
  const int row = q0 + l32;
  const float l_tot = l_run + swap_halves(l_run, half);
  const float inv_l = 1.f / (lr_run + swap_halves(lr_run, half));
  if constexpr (!KSPLIT) {
    // The ring is idle: the last period pair ended with every load landed and a barrier after
    // every read.  Wave w stages its tile in half of one stage array.
    static_assert(D == 128 && kSlots == 1, "a wave's O tile is half a stage array");
    static_assert(STAGES == 2, "every period pair ends with vmcnt(0) and a barrier only with two stages");
    PAA_LDS char* ot = (wave / 2 == 0   ? (PAA_LDS char*)k_st0
                        : wave / 2 == 1 ? (PAA_LDS char*)k_st1
                        : wave / 2 == 2 ? (PAA_LDS char*)v_st0
                                        : (PAA_LDS char*)v_st1) + (wave % 2) * (32 * T::kRowBytes);
    store_o_tile<D>(ot, acc, inv_l, lane, a.o + q_base + (size_t)q0 * q_stride, q_stride, n_q - q0);
  }
  if (row < n_q) {
    if constexpr (KSPLIT) {
      uint16_t* orow = a.o + q_base + (size_t)row * q_stride;
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
    }
    if (a.lse != nullptr && half == 0) {
      const size_t li = PAGED ? q_base / D + (size_t)row * a.H : ((size_t)b * a.H + head) * N + row;
      a.lse[li] = a.scale * m_run + __logf(l_tot);
    }
  }
}

// Workgroups of one kernel instantiation the current device holds at once (CUs x workgroups per
// CU), 0 if unknown; queried once per device.
template <typename Kernel>
long long resident_workgroups(Kernel kernel, int threads) {
  static std::atomic<long long> cached[16];  // zero: not yet known
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 16) {
    const long long c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return 0;
  const long long c = (long long)cus * per_cu;
  if (dev < 16) cached[dev].store(c, std::memory_order_relaxed);
  return c;
}

template <int D, int MASK, int HPW, int WAVES, int RB, int STAGES>
hipError_t launch_prefill(const PrefillArgs& base, hipStream_t stream) {
  PrefillArgs a = base;
  constexpr int kTileRows = (WAVES / HPW) * 32 * RB;
  a.n_qtiles = (a.N + kTileRows - 1) / kTileRows;
  a.units_per_qt = a.B * a.Hkv * ((a.H / a.Hkv) / HPW);
  const long long units = (long long)a.n_qtiles * a.units_per_qt;
  if (units > 0x7fffffffLL) return hipErrorInvalidValue;
  const auto kernel = prefill_bf16_kernel<D, MASK, HPW, WAVES, RB, STAGES>;
  a.mirror = MASK != kMaskNone && units <= resident_workgroups(kernel, 64 * WAVES) ? 1 : 0;
  hipLaunchKernelGGL(kernel, dim3((unsigned)units), dim3(64 * WAVES), 0, stream, a);
  return hipGetLastError();
}

template <int D, int MASK, int HPW, int STAGES, bool KSPLIT = false>
hipError_t launch_prefill_pp(const PrefillArgs& base, hipStream_t stream) {
  PrefillArgs a = base;
  constexpr int kTileRows = ((KSPLIT ? 4 : 8) / HPW) * 32;
  a.n_qtiles = (a.N + kTileRows - 1) / kTileRows;
  a.units_per_qt = a.B * a.Hkv * ((a.H / a.Hkv) / HPW);
  const long long units = (long long)a.n_qtiles * a.units_per_qt;
  if (units > 0x7fffffffLL) return hipErrorInvalidValue;
  const auto kernel = prefill_pp_kernel<D, MASK, HPW, STAGES, KSPLIT>;
  a.mirror = MASK != kMaskNone && units <= resident_workgroups(kernel, 512) ? 1 : 0;
  hipLaunchKernelGGL(kernel, dim3((unsigned)units), dim3(512), 0, stream, a);
  return hipGetLastError();
}

template <int D, int MASK, bool KSPLIT = false>
hipError_t dispatch_pp(const PrefillArgs& a, hipStream_t stream) {
  constexpr int kStages = 2;
  const int group = a.H / a.Hkv;
  if (group % 4 == 0) return launch_prefill_pp<D, MASK, 4, kStages, KSPLIT>(a, stream);
  if (group % 2 == 0) return launch_prefill_pp<D, MASK, 2, kStages, KSPLIT>(a, stream);
  return launch_prefill_pp<D, MASK, 1, kStages, KSPLIT>(a, stream);
}

template <int D, int MASK, int WAVES>
hipError_t dispatch_group(const PrefillArgs& a, hipStream_t stream) {
  constexpr int kStages = 2;
  const int group = a.H / a.Hkv;
  if constexpr (WAVES % 4 == 0)
    if (group % 4 == 0) return launch_prefill<D, MASK, 4, WAVES, 1, kStages>(a, stream);
  if constexpr (WAVES % 2 == 0)
    if (group % 2 == 0) return launch_prefill<D, MASK, 2, WAVES, 1, kStages>(a, stream);
  return launch_prefill<D, MASK, 1, WAVES, 1, kStages>(a, stream);
}

// Workgroup shape.  Eight waves sharing each K/V tile halve the L2 -> LDS traffic per flop against
// four, and win when the grid still has at least 4 workgroups per CU; for smaller grids (short
// sequences) the critical path is the heaviest causal query tile, and four-wave workgroups (two per
// CU) walk it faster.
template <int D, int MASK>
hipError_t dispatch_hpw(const PrefillArgs& a, hipStream_t stream) {
  const int group = a.H / a.Hkv;
  const int hpw = group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
  const long long rows8 = (8 / hpw) * 32;
  const long long units8 = (long long)a.B * a.Hkv * (group / hpw) * ((a.N + rows8 - 1) / rows8);
  if (units8 >= 1024) {
    // d = 128: the MFMA and VALU halves of a tile are of similar length, and the ping-pong
    // kernel overlaps them across the two waves of each SIMD.  d = 64: the exponentials
    // dominate, and the lock-step kernel is as fast.
    if constexpr (D == 128) return dispatch_pp<D, MASK>(a, stream);
    else return dispatch_group<D, MASK, 8>(a, stream);
  }
  // Small grids (short sequences) at d = 128: the critical path is the longest causal rows, and
  // splitting their key tiles over the two groups of a ping-pong workgroup halves the tiles each
  // wave walks (8 heads x 2048 tokens: 47 -> 39 us).  At d = 64 the split workgroups lose to
  // two four-wave workgroups per CU (causal 16 heads x 1024 tokens: 26.5 against 24.4 us).
  if constexpr (D == 128 && (MASK == kMaskNone || MASK == kMaskCausal)) return dispatch_pp<D, MASK, true>(a, stream);
  return dispatch_group<D, MASK, 4>(a, stream);
}

// Chunked prefill over a paged cache: on large grids the ping-pong kernel at d = 128 and the
// eight-wave lock-step kernel at d = 64; on small grids the four-wave lock-step kernel.
template <int D>
hipError_t dispatch_paged(const PrefillArgs& a, hipStream_t stream) {
  const int group = a.H / a.Hkv;
  const int hpw = group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
  const long long rows8 = (8 / hpw) * 32;
  const long long units8 = (long long)a.B * a.Hkv * (group / hpw) * ((a.N + rows8 - 1) / rows8);
  if (units8 >= 1024) {
    if constexpr (D == 128) return dispatch_pp<D, kMaskPaged>(a, stream);
    else return dispatch_group<D, kMaskPaged, 8>(a, stream);
  }
  return dispatch_group<D, kMaskPaged, 4>(a, stream);
}

}  // namespace

hipError_t paged_prefill_bf16(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              const int* block_table, const int* ctx_lens, const int* q_start, void* o, float* lse,
                              int num_seqs, int H, int Hkv, int d, int max_pages, int num_pages, int max_q_len,
                              float scale, hipStream_t stream) {
  PrefillArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k_new;
  a.v = (const uint16_t*)v_new;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.B = num_seqs;
  a.H = H;
  a.Hkv = Hkv;
  a.N = max_q_len;  // sizes the grid; each sequence's own chunk length is read on the device
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  a.ref_headroom = kRefHeadroomLog2 / a.scale_log2;
  a.bt = block_table;
  a.ctx_lens = ctx_lens;
  a.q_start = q_start;
  a.kc = (uint16_t*)k_cache;
  a.vc = (uint16_t*)v_cache;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  return d == 64 ? dispatch_paged<64>(a, stream) : dispatch_paged<128>(a, stream);
}

hipError_t prefill_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                        int N, int d, bool causal, int window, int n_global, float scale, hipStream_t stream) {
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
  a.ref_headroom = kRefHeadroomLog2 / a.scale_log2;
  a.window = window;
  a.n_global = n_global;
  // a window that covers every earlier key is the plain causal mask
  const int mask = !causal ? kMaskNone : (window > 0 && window < N ? kMaskWindow : kMaskCausal);
  if (d == 64) {
    if (mask == kMaskNone) return dispatch_hpw<64, kMaskNone>(a, stream);
    if (mask == kMaskCausal) return dispatch_hpw<64, kMaskCausal>(a, stream);
    return dispatch_hpw<64, kMaskWindow>(a, stream);
  }
  if (mask == kMaskNone) return dispatch_hpw<128, kMaskNone>(a, stream);
  if (mask == kMaskCausal) return dispatch_hpw<128, kMaskCausal>(a, stream);
  return dispatch_hpw<128, kMaskWindow>(a, stream);
}

}  // namespace paa
