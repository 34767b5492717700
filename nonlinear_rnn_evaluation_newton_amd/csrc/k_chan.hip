// Instantiations and launchers of the channel-parallel kernel family.
#include "k_chan_impl.h"
#include "k_time_impl.h"  // resident_blocks / persistent_grid

namespace pr {

// Tile geometry of the standalone scan: lanes own CPL adjacent channels,
// wavefronts TW steps.
ChanGeomInfo chan_geom(int cell, int n) {
  ChanGeomInfo g;
  if (cell == C_GRU_DIAG) {
    g.CPL = (n % 2 == 0) ? 2 : 1;
    g.TW = 16;
  } else {
    g.CPL = 1;
    g.TW = 8;
  }
  g.CH = 64 * g.CPL;
  g.TT = 4 * g.TW;
  return g;
}

template <auto KERN>
static int chan_grid(const ChanArgs &a, bool stripe_aligned) {
  const int r = resident_blocks<KERN>();
  if (r <= 0) return 0;
  int grid = a.ntiles < r ? a.ntiles : r;
  if (stripe_aligned && a.stripes <= grid) grid = grid / a.stripes * a.stripes;
  return grid;
}

hipError_t launch_chan_reduce_tiles(int cell, ChanArgs &a, double *red, float *dWh, float *dbh, float *dpeep,
                                   float *dbx, hipStream_t s) {
  const ChanGeomInfo gi = chan2_geom(cell, a.n);
  const unsigned blocks = (unsigned)((a.n * CHAN_P + 255) / 256);
  if (gi.CH == 128)
    hipLaunchKernelGGL((k_chan_red_split<128>), dim3(blocks, CHAN_RED_SPLITS), dim3(256), 0, s, a, red);
  else
    hipLaunchKernelGGL((k_chan_red_split<64>), dim3(blocks, CHAN_RED_SPLITS), dim3(256), 0, s, a, red);
  hipLaunchKernelGGL(k_chan_red_final<CHAN_RED_SPLITS>, dim3(blocks), dim3(256), 0, s, a, (const double *)red, dWh,
                     dbh, dpeep, dbx);
  return hipGetLastError();
}

hipError_t launch_chan_scan(int SW, ChanArgs &a, hipStream_t s) {
  if (SW == 1 && a.n % 2 == 0) {
    const int grid = chan_grid<k_chan_scan<1, 2, 16>>(a, false);
    if (grid <= 0) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((k_chan_scan<1, 2, 16>), dim3(grid), dim3(256), 0, s, a);
  } else if (SW == 1) {
    const int grid = chan_grid<k_chan_scan<1, 1, 16>>(a, false);
    if (grid <= 0) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((k_chan_scan<1, 1, 16>), dim3(grid), dim3(256), 0, s, a);
  } else {
    const int grid = chan_grid<k_chan_scan<2, 1, 8>>(a, false);
    if (grid <= 0) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((k_chan_scan<2, 1, 8>), dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pr
