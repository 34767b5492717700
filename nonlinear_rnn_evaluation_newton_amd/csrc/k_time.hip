// Dispatch of the time-parallel kernel family and its standalone scan.
#include "k_time_impl.h"

namespace pr {

int time_padded_n(int n) {
  if (n <= 1) return 1;
  if (n <= 2) return 2;
  if (n <= 4) return 4;
  if (n <= 8) return 8;
  return 0;
}

int time_tile(int N) {
  switch (N) {
    case 1: return time_tile_c<1>();
    case 2: return time_tile_c<2>();
    case 4: return time_tile_c<4>();
    case 8: return time_tile_c<8>();
  }
  return 0;
}

int time_part_count(int cell, int N) {
  const int G = cell_gates(cell);
  return G * N * DX_FUSED + G * N + G * N * N + G * N;  // upper bound over the fused input widths
}

hipError_t launch_time_sweep(int cell, int Nv, const TimeArgs &a, hipStream_t s) {
  switch (cell) {
    case C_TANH: return time_sweep_tanh(Nv, a, s);
    case C_GRU: return time_sweep_gru(Nv, a, s);
    case C_LINEAR: return time_sweep_linear(Nv, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_time_adjoint(int cell, int Nv, TimeArgs &a, hipStream_t s) {
  switch (cell) {
    case C_TANH: return time_adjoint_tanh(Nv, a, s);
    case C_GRU: return time_adjoint_gru(Nv, a, s);
    case C_LINEAR: return time_adjoint_linear(Nv, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_time_elk_jr(int cell, int Nv, const TimeArgs &a, float *jr, hipStream_t s) {
  switch (cell) {
    case C_TANH: return time_elk_jr_tanh(Nv, a, jr, s);
    case C_GRU: return time_elk_jr_gru(Nv, a, jr, s);
    case C_LINEAR: return time_elk_jr_linear(Nv, a, jr, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_time_reduce(int cell, int Nv, const TimeArgs &a, const float *part, float *dWx, float *dbx,
                              float *dWh, float *dbh, hipStream_t s) {
  switch (cell) {
    case C_TANH: return time_reduce_tanh(Nv, a, part, dWx, dbx, dWh, dbh, s);
    case C_GRU: return time_reduce_gru(Nv, a, part, dWx, dbx, dWh, dbh, s);
    case C_LINEAR: return time_reduce_linear(Nv, a, part, dWx, dbx, dWh, dbh, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_time_scan(int Nv, const ScanArgs &a, hipStream_t s) {
  PR_DISPATCH_N(Nv, {
    const int grid = persistent_grid<k_time_scan<N>>(a.ntiles);
    if (grid <= 0) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((k_time_scan<N>), dim3(grid), dim3(256), 0, s, a);
  });
  return hipGetLastError();
}

}  // namespace pr
