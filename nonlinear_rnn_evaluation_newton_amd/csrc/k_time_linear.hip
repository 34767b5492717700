// Time-parallel kernels instantiated for one cell (one translation unit per
// cell keeps compile times short).
#include "k_time_impl.h"

namespace pr {

hipError_t time_sweep_linear(int Nv, const TimeArgs &a, hipStream_t s) { return time_sweep_cell<C_LINEAR>(Nv, a, s); }
hipError_t time_adjoint_linear(int Nv, TimeArgs &a, hipStream_t s) { return time_adjoint_cell<C_LINEAR>(Nv, a, s); }
hipError_t time_reduce_linear(int Nv, const TimeArgs &a, const float *part, float *dWx, float *dbx, float *dWh,
                             float *dbh, hipStream_t s) {
  return time_reduce_cell<C_LINEAR>(Nv, a, part, dWx, dbx, dWh, dbh, s);
}

hipError_t time_elk_jr_linear(int Nv, const TimeArgs &a, float *jr, hipStream_t s) {
  return time_elk_jr_cell<C_LINEAR>(Nv, a, jr, s);
}

}  // namespace pr
