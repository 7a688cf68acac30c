// Pieces of the tiled attention loop shared by the prefill kernels: tile size, the lazy-rescale
// threshold, the buffer resource format, exact vmcnt waits, the tile barrier and compile-time
// unrolling over ring stages.
#pragma once

#include <type_traits>

#include "device_common.hpp"

namespace paa {

constexpr int kBc = 64;               // keys per tile
// bf16 prefill: a lane's share of one tile's probabilities may reach 2^32 before the reference moves
// (so P, the row sums and O stay finite for |V| below 2^64), and a moved reference sits 80 (log2
// units) above the row's running maximum, so later scores may rise by about 107 before it moves
// again.  Keys more than 46 below the running maximum then underflow to 0: their weight is under
// 2^-46 each.  The peaked long workload moved references on many tiles at a headroom of 0 (its
// outlier keys keep setting new maxima): a headroom of 48 took it from 1965 to 1851 us on one box,
// 80 a further 2.6%.
constexpr float kMaxTileSum = 4294967296.0f;
constexpr float kRefHeadroomLog2 = 80.0f;

// Third word of a raw buffer resource (gfx9 family): 32-bit data format, no swizzle, no index.
// The tile loads read K and V through such resources (buffer_load ... lds), sized so that
// anything past the valid rows reads as zeros.
constexpr int kRawBufferWord3 = 0x00020000;


// vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4, lgkmcnt 11:8).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for the tile loop.  The only LDS writes in the loop are direct global->LDS
// loads, whose completion is tracked by vmcnt and awaited explicitly (wait_vmcnt) just before; a
// workgroup-scope fence would make the compiler wait for every one of them (vmcnt(0)), which
// would drain the load ring.  The wavefront-scope fences keep the compiler from moving memory
// accesses across the barrier; lgkmcnt(0) retires this wave's own LDS reads first.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0) only
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int I, int S, typename F>
__device__ __forceinline__ void for_stages(F& f, int j, int n) {
  if (j + I < n) {
    f(std::integral_constant<int, I>{}, j + I);
    if constexpr (I + 1 < S) for_stages<I + 1, S>(f, j, n);
  }
}

}  // namespace paa
