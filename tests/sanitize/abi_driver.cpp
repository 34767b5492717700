// Drives the C ABI's argument validation and workspace planning (every path
// that returns before any HIP call) for a host-side build with
// AddressSanitizer and UndefinedBehaviorSanitizer.  Test infrastructure:
// built and run by tests/test_sanitizers.py, on a machine without a GPU.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "pararnn.h"

static int g_bad = 0;
#define EXPECT(cond)                                                     \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "line %d: %s (%s)\n", __LINE__, #cond, pararnn_last_error()); \
      g_bad = 1;                                                         \
    }                                                                    \
  } while (0)

int main() {
  void *v = (void *)(uintptr_t)256;  // never dereferenced: every call below is refused first
  const int cells[] = {PR_CELL_TANH_RNN, PR_CELL_GRU, PR_CELL_GRU_DIAG, PR_CELL_LSTM_CIFG_DIAG, PR_CELL_LINEAR, 7, -1};
  const int jacs[] = {PR_JAC_DENSE, PR_JAC_DIAG, PR_JAC_BLOCK2, PR_JAC_ZERO, 4};
  const int sizes[][4] = {{2, 256, 2, 4},     {16, 1 << 20, 1, 1}, {8, 4096, 1024, 1024}, {4, 8192, 2048, 2048},
                          {16, 16384, 32, 64}, {1, 1, 1, 1},        {3, 77, 9, 130},       {0, 5, 1, 1},
                          {2, -3, 1, 1},      {65536, 65536, 1, 1}, {1, 1 << 30, 1, 8},    {5, 1000, 7, 64},
                          {2, 100, 3, 20},    {2, 50, 20, 5},       {1, 1, 1, 63},         {65536, 65536, 3, 33}};
  for (int c : cells)
    for (int j : jacs)
      for (int dt = 0; dt < 3; dt++)
        for (const auto &s : sizes) {
          pr_problem p = {c, j, dt, s[0], s[1], s[2], s[3]};
          const size_t w0 = pararnn_workspace_bytes(&p, 0), w1 = pararnn_workspace_bytes(&p, 1);
          EXPECT(w1 >= w0);
          (void)pararnn_elk_workspace_bytes(&p);
          // workspace too small by one byte, or misaligned, or missing
          pr_weights w = {v, nullptr, v, nullptr, v};
          int rc = pararnn_solve(&p, &w, v, nullptr, 1e-6f, 8, v, nullptr, nullptr, 0, v, w0 ? w0 - 1 : 0, nullptr);
          EXPECT(rc < 0);
          rc = pararnn_solve(&p, &w, v, nullptr, 1e-6f, 8, v, nullptr, nullptr, 0, (void *)(uintptr_t)257,
                             w0 + 1024, nullptr);
          EXPECT(rc < 0);
          rc = pararnn_adjoint(&p, &w, v, nullptr, v, v, v, v, v, nullptr, v, w1 ? w1 - 1 : 0, nullptr);
          EXPECT(rc < 0);
          rc = pararnn_solve_adjoint(&p, &w, v, nullptr, 1e-6f, 8, v, nullptr, nullptr, 0, v, v, v, v, nullptr, v,
                                     w1 ? w1 - 1 : 0, nullptr);
          EXPECT(rc < 0);
          rc = pararnn_solve_elk(&p, &w, v, nullptr, 0.1f, 1e-6f, 8, v, nullptr, nullptr, 0, nullptr, 1 << 20, nullptr);
          EXPECT(rc < 0);
          rc = pararnn_solve_elk(&p, &w, v, nullptr, -1.f, 1e-6f, 8, v, nullptr, nullptr, 0, v, (size_t)1 << 40, nullptr);
          EXPECT(rc < 0);
        }
  // missing pointers and bad scalars on a valid problem
  pr_problem p = {PR_CELL_GRU, PR_JAC_DENSE, PR_F32, 2, 64, 1, 1};
  pr_weights w = {v, nullptr, v, nullptr, nullptr}, wn = {nullptr, nullptr, v, nullptr, nullptr};
  const size_t ws = pararnn_workspace_bytes(&p, 1);
  EXPECT(ws > 0);
  EXPECT(pararnn_solve(nullptr, &w, v, nullptr, 1e-6f, 8, v, nullptr, nullptr, 0, v, ws, nullptr) == PR_EINVAL);
  EXPECT(pararnn_solve(&p, &wn, v, nullptr, 1e-6f, 8, v, nullptr, nullptr, 0, v, ws, nullptr) == PR_EINVAL);
  EXPECT(pararnn_solve(&p, &w, nullptr, nullptr, 1e-6f, 8, v, nullptr, nullptr, 0, v, ws, nullptr) == PR_EINVAL);
  EXPECT(pararnn_solve(&p, &w, v, nullptr, 1e-6f, 0, v, nullptr, nullptr, 0, v, ws, nullptr) == PR_EINVAL);
  EXPECT(pararnn_solve(&p, &w, v, nullptr, __builtin_nanf(""), 8, v, nullptr, nullptr, 0, v, ws, nullptr) ==
         PR_EINVAL);
  EXPECT(pararnn_adjoint(&p, &w, v, nullptr, v, nullptr, v, v, v, nullptr, v, ws, nullptr) == PR_EINVAL);
  // scans, lsim, the no-allocation scan, trace categories, status text
  for (int j = -1; j < 4; j++) {
    (void)pararnn_scan_workspace_bytes(j, 3, 1000, 5);
    EXPECT(pararnn_affine_scan(j, 3, 1000, 5, 0, nullptr, (const float *)v, (float *)v, v, 1 << 20, nullptr) < 0);
    EXPECT(pararnn_affine_scan_noalloc(j, 0, 1000, 5, 0, (const float *)v, (const float *)v, (float *)v, nullptr) < 0);
  }
  EXPECT(pararnn_affine_scan_noalloc(PR_JAC_DIAG, 8, 1 << 16, 1024, 0, (const float *)v, (const float *)v, (float *)v,
                                     nullptr) == PR_EWORKSPACE);
  EXPECT(pararnn_affine_scan(PR_JAC_DENSE, 2, 100, 4, 0, (const float *)v, (const float *)v, (float *)v, v, 10,
                             nullptr) == PR_EWORKSPACE);
  for (int nx = 0; nx < 10; nx++) {
    (void)pararnn_lsim_workspace_bytes(4, 5000, nx, 2, 2);
    EXPECT(pararnn_lsim(4, 5000, nx, 2, 2, (const float *)v, (const float *)v, (const float *)v, (const float *)v,
                        0.f, (const float *)v, nullptr, nullptr, (float *)v, v, 1 << 20, nullptr) < 0);
  }
  EXPECT(pararnn_trace_kernel(99, nullptr, nullptr) == PR_EINVAL);
  for (int code = -8; code < 4; code++) EXPECT(pararnn_strerror(code) != nullptr && strlen(pararnn_strerror(code)) > 0);
  EXPECT(strlen(pararnn_last_error()) > 0);
  printf(g_bad ? "abi driver: FAILED\n" : "abi driver: ok\n");
  return g_bad;
}
