// Input projection of a layer on the matrix cores, X = x U^T + bias over
// M = T * B rows of x ("Optimizing Performance of Recurrent Neural Networks
// on GPUs", Abstract, single-layer stage).  The arithmetic of a tile is
// project_tile (project_tile.h); this kernel deals the tiles to workgroups:
// workgroup g runs on XCD g % 8, and each XCD takes a rectangle of tiles
// (launch_project), so that its L2 holds the rows of x and U that its tiles
// share.
#include "project_tile.h"

namespace prnn {
namespace {

using proj::kBM;
using proj::kGroups;

template <bool XF32, bool VEC, int BN>
__global__ void __launch_bounds__(proj::kThreads) project_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 lds_all[proj::lds_bytes<BN>() / 2];
  // Workgroup g runs on XCD g % 8.  The XCDs form an xr x (8 / xr) grid over
  // the tiles: XCD (i, j) takes tile rows [i Rm, (i + 1) Rm) and tile columns
  // [j Rn, (j + 1) Rn), so its L2 holds 1 / xr of x and xr / 8 of U (the
  // split that fetches the fewest bytes, chosen by the host).
  const int g = blockIdx.x;
  const int xcd = g & 7, local = g >> 3;
  const int xi = xcd / (8 / a.xcd_rows), xj = xcd % (8 / a.xcd_rows);
  const int lr = local / a.xcd_tile_cols, lc = local - lr * a.xcd_tile_cols;
  const int tm = xi * a.xcd_tile_rows + lr;
  const int tn = xj * a.xcd_tile_cols + lc;
  const int tiles_m = (a.M + kBM - 1) / kBM;
  // whole workgroups leave: the barriers in the tile stay uniform
  if (lr >= a.xcd_tile_rows || tm >= tiles_m || lc >= a.xcd_tile_cols || tn >= a.tiles_n) return;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t ur = make_rsrc(a.U, a.u_bytes);
  const proj::TileRows rows{a.M, 1, 0};
  const bool range_ok =
      proj::project_tile<XF32, VEC, BN>(xr, ur, a.bias, a.X, a.N, rows, tm * kBM, tn * BN, a.N, a.I, lds_all);
  if (XF32 && wave_any(!range_ok) && (threadIdx.x & 63) == 0) report_failure(a.status, a.status_host, kStatusRange);
}

}  // namespace

template <int BN>
const void* pick_project(bool x_f32, bool vec) {
  return x_f32 ? (vec ? reinterpret_cast<const void*>(&project_kernel<true, true, BN>)
                      : reinterpret_cast<const void*>(&project_kernel<true, false, BN>))
               : (vec ? reinterpret_cast<const void*>(&project_kernel<false, true, BN>)
                      : reinterpret_cast<const void*>(&project_kernel<false, false, BN>));
}

// 64 x 128 tiles, or 64 x 64 when 64 x 128 would leave half of the compute
// units idle (fewer than 128 tiles: short sequences, such as one block of a
// stack; measured at N = I = 1792: 256 rows 27.6 -> 22.4 us, while 1024 rows
// are faster with the wide tiles, 31.5 vs 34.5 us).
//
// XCD grid: the 8 XCDs as xr x (8 / xr) rectangles of tiles (xr = 1, 2, 4, 8),
// the split for which the eight L2 caches fetch the fewest bytes (each XCD
// reads the x rows of its tile rows and the U rows of its tile columns);
// among equal splits, the one with the fewest idle workgroups.
hipError_t launch_project(const ProjArgs& a, bool x_f32, bool vec, hipStream_t stream) {
  ProjArgs args = a;
  const long long tiles_m = (a.M + kBM - 1) / kBM;
  const bool narrow = tiles_m * ((a.N + 127) / 128) < 128;
  const int bn = narrow ? 64 : 128;
  args.tiles_n = (a.N + bn - 1) / bn;
  args.tiles = static_cast<int>(tiles_m * args.tiles_n);
  const double xrow_bytes = (double)kBM * a.I * (x_f32 ? 4.0 : 2.0), ucol_bytes = (double)bn * a.I * 2.0;
  long long best_groups = -1;
  double best_bytes = 0.0;
  for (int xr = 1; xr <= 8; xr *= 2) {
    const long long rm = (tiles_m + xr - 1) / xr, rn = (args.tiles_n + (8 / xr) - 1) / (8 / xr);
    const double bytes = 8.0 * ((double)rm * xrow_bytes + (double)rn * ucol_bytes);
    const long long groups = rm * rn;  // workgroups per XCD
    if (best_groups < 0 || bytes < best_bytes * 0.999 || (bytes <= best_bytes * 1.001 && groups < best_groups)) {
      best_groups = groups;
      best_bytes = bytes;
      args.xcd_rows = xr;
      args.xcd_tile_rows = static_cast<int>(rm);
      args.xcd_tile_cols = static_cast<int>(rn);
    }
  }
  args.per_xcd = static_cast<int>(best_groups);
  const void* fn = narrow ? pick_project<64>(x_f32, vec) : pick_project<128>(x_f32, vec);
  void* kargs[] = {&args};
  return hipLaunchKernel(fn, dim3(8u * (unsigned)args.per_xcd), dim3(256 * kGroups), kargs, 0, stream);
}

}  // namespace prnn
