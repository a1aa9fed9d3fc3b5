// gemm_common.h -- pieces shared by the FP4 GEMM kernels (gfx950): buffer
// descriptors, uniform-value helpers and the XCD-aware tile order.  Internal.
#pragma once

#include "fp4_device.h"

namespace fp4 {

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// max(total - off, 0) for uniform values, kept in a scalar register (a
// saturating subtract would otherwise be selected as a vector instruction and
// turn the buffer descriptor into a per-lane value).
__device__ __forceinline__ uint32_t uniform_rem(uint32_t total, uint32_t off) {
  return __builtin_amdgcn_readfirstlane(total > off ? total - off : 0u);
}

// A uniform value the compiler may not strength-reduce into per-step vector
// registers.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+s"(x));
  return __builtin_amdgcn_readfirstlane(x);
}

// Grouped raster: walk tiles in groups of `group_m` tile-rows, so consecutive
// tiles share A rows (within a group) and B columns (across the group).
__device__ __forceinline__ void raster_coords(uint32_t t, uint32_t tilesM, uint32_t tilesN, uint32_t group_m,
                                              uint32_t& tm, uint32_t& tn) {
  const uint32_t group = group_m * tilesN;
  const uint32_t g = t / group, first_m = g * group_m;
  const uint32_t gm = (tilesM - first_m) < group_m ? (tilesM - first_m) : group_m;
  tm = first_m + (t % group) % gm;
  tn = (t % group) / gm;
}

// Tile order: blockIdx.x is dispatched round-robin over the 8 XCDs, so give
// each XCD a contiguous range of tiles, and walk that range with the grouped
// raster so concurrently running tiles share A rows and B columns in the
// XCD's L2.
__device__ __forceinline__ void tile_coords(uint32_t block, uint32_t tilesM, uint32_t tilesN, uint32_t group_m,
                                            uint32_t& tm, uint32_t& tn) {
  const uint32_t ntiles = tilesM * tilesN;
  uint32_t t = block;
  if ((ntiles & 7u) == 0u) t = (block & 7u) * (ntiles >> 3) + (block >> 3);
  raster_coords(t, tilesM, tilesN, group_m, tm, tn);
}

}  // namespace fp4
