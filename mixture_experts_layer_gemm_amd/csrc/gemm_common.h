// Helpers shared by the grouped GEMM kernels: direct-to-LDS loads, explicit vmcnt
// waits, and the device-side tile map over real-count expert segments.
#pragma once
#include "common.h"

namespace moe {

// One wave-wide direct-to-LDS load: lane j's 16 bytes at gptr land at LDS byte address
// lds_addr + 16 j. Issued as inline asm so that the compiler does not serialize it
// against unrelated LDS reads: completion is awaited explicitly with wait_vmcnt, and the
// workgroup barrier that follows publishes the data to the other waves.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds_addr)
               : "memory", "m0");
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0], expcnt[6:4],
// lgkmcnt[11:8], vmcnt[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

struct TileMap {
  int g, row0, rows, nt;
};

// Builds the per-group tile prefix in LDS and decodes this workgroup's tile; tiles are
// ordered (group, n-tile, m-tile). Returns false for a spare workgroup. All threads of
// the workgroup must call it.
__device__ inline bool decode_tile(const int32_t* __restrict__ offsets, int G, int max_rows, int bm,
                            int n_tiles, int* s_off, int* s_tstart, TileMap& tm) {
  const int tid = threadIdx.x;
  for (int g = tid; g <= G; g += blockDim.x)
    s_off[g] = (offsets != nullptr) ? offsets[g] : (g == 0 ? 0 : max_rows);
  __syncthreads();
  const int cnt = (tid < G) ? ceil_div(s_off[tid + 1] - s_off[tid], bm) * n_tiles : 0;
  s_tstart[tid + 1] = cnt;
  if (tid == 0) s_tstart[0] = 0;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {  // inclusive scan, G <= 256 = blockDim
    const int v = (tid >= off) ? s_tstart[tid + 1 - off] : 0;
    __syncthreads();
    s_tstart[tid + 1] += v;
    __syncthreads();
  }
  const int tile = xcd_remap(blockIdx.x, s_tstart[G]);
  if (tile < 0) return false;
  int lo = 0, hi = G - 1;  // largest g with s_tstart[g] <= tile (a non-empty group)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_tstart[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  const int local = tile - s_tstart[lo];
  const int mtiles = ceil_div(s_off[lo + 1] - s_off[lo], bm);
  tm.g = lo;
  tm.nt = local / mtiles;
  tm.row0 = s_off[lo] + (local - tm.nt * mtiles) * bm;
  tm.rows = min(bm, s_off[lo + 1] - tm.row0);
  return true;
}


}  // namespace moe
