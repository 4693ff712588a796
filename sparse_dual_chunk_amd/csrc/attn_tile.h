// Staged-tile layout and softmax helpers shared by the prefill and decode
// attention kernels (gfx950, 64-wide waves, 32x32x16 bf16 MFMA).
#pragma once
#include "common.h"

namespace dca {

// Tiles of 32 keys staged in LDS by direct global->LDS loads, two stages.
// A tile of one tensor is 8 groups of 4 key rows: a group holds its rows one
// after the other (256 bytes each, 1 KiB) and 64 bytes of padding.  Each
// direct load instruction fills one group, 16 consecutive lanes per row, so
// that every 4 lanes read 64 contiguous bytes of one row (the vector memory
// unit serves such requests several times faster than four rows per 4
// lanes).  Inside row r of a group the 16-byte chunk c sits at slot
// c ^ 5(r & 3): with the padding, the K operand reads (16 rows, one chunk)
// and the transposed V reads (4 rows, four chunks) fall on distinct banks
// for 32 as for 64 four-byte banks.
constexpr int BN = 32;
constexpr int GRPB = 1024 + 64;                // bytes per 4-row group
constexpr int TILEB = 8 * GRPB;                // one tensor of one tile

// byte offset of (row, 16-byte chunk) inside a tensor tile
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return (row >> 2) * GRPB + (row & 3) * 256 + ((chunk ^ (5 * (row & 3))) << 4);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum of a value with the one held by lane ^ 32 (the other half of the row)
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace dca
