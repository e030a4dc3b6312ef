// Workgroup id -> output tile mapping, XCD-aware grouped order.
//
// "Hopper/Blackwell architecture features" §12.7.1 maps program ids to tiles in
// groups of GROUP_M tile rows (walk down GROUP_M rows, then move one column) so
// concurrently running tiles reuse the same A rows and B columns from L2.  On
// MI355X the dispatcher hands consecutive workgroup ids to the 8 XCDs in turn and
// each XCD has a private 4 MB L2; without a remap, neighbours in the grouped
// order would land on different XCDs and share nothing.  Here the id is first
// turned into a position in the grouped order in which XCD x owns one contiguous
// slice, so the ~32 tiles resident on an XCD are neighbours.
#pragma once

#include <hip/hip_runtime.h>

namespace fp8gemm {

constexpr int kNumXcd = 8;
constexpr int kGroupM = 4;

// Bijection on [0, total): id -> position in an order where XCD (id % 8) owns a
// contiguous slice.
__device__ __forceinline__ int xcd_linear(int id, int total) {
  const int xcd = id % kNumXcd;
  const int local = id / kNumXcd;
  const int q = total / kNumXcd, r = total % kNumXcd;
  return xcd * q + (xcd < r ? xcd : r) + local;
}

// Grouped order: groups of `group_m` tile rows, column-major inside a group.
__device__ __forceinline__ void grouped_tile(int linear, int tiles_m, int tiles_n, int group_m,
                                             int* tm, int* tn) {
  const int per_group = group_m * tiles_n;
  // a single tile row left over joins the last full group (a one-row group would
  // give each XCD a 1 x 32 block of tiles reading 33 bands instead of about 12)
  const int full = tiles_m / group_m;
  int gid = linear / per_group;
  if (tiles_m % group_m == 1 && full > 0 && gid >= full - 1) gid = full - 1;
  const int first_m = gid * group_m;
  const int rows = (tiles_m % group_m == 1 && full > 0 && gid == full - 1)
                       ? group_m + 1 : min(tiles_m - first_m, group_m);
  const int in_group = linear - gid * per_group;
  *tm = first_m + in_group % rows;
  *tn = in_group / rows;
}

__device__ __forceinline__ void tile_coords(int id, int tiles_m, int tiles_n, int group_m, int* tm,
                                            int* tn) {
  grouped_tile(xcd_linear(id, tiles_m * tiles_n), tiles_m, tiles_n, group_m, tm, tn);
}

}  // namespace fp8gemm
