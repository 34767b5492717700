// pararnn_affine_scan_noalloc: the linear recurrence of pararnn_affine_scan
// with its scratch (look-back descriptors and the state record) in a static
// device array instead of a caller workspace, for callers that cannot
// allocate device memory at all (code under stream capture, serving loops,
// harnesses that forbid allocation).
//
// Each device that runs this entry point holds its own copy of `scratch`
// until the process ends.  Host code never passes the array's name to a
// kernel or a copy: on the host that name is only a stand-in for the device
// symbol.  The first call on a device, with that device current, asks the
// runtime for the copy's device address (hipGetSymbolAddress), and every
// launch takes that address.  All calls on one device share the array:
// overlapping calls on that device race (each call clears the part it uses
// before its scan).
#include <mutex>

#include "internal.h"
#include "pararnn.h"

namespace {

static __device__ __align__(256) unsigned char scratch[PR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // per device: the address of its copy of `scratch`

// The device address of the current device's `scratch`, looked up once per
// device; nullptr (with the error recorded) on failure.
void *device_scratch(int *code) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *code = pr::fail(PR_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *code = pr::fail(PR_EUNSUPPORTED, "device %d: the static scratch is kept for devices 0..%d", dev,
                     kMaxDevices - 1);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *code = pr::fail(PR_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      return nullptr;
    }
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int pararnn_affine_scan_noalloc(int jac, int B, int T, int n, int reverse, const float *A, const float *b,
                                           float *y, void *stream) {
  pr::clear_error();
  // the sizes first: a problem beyond the static scratch is refused before
  // any HIP call
  if (jac < 0 || jac > 2) return pr::fail(PR_EINVAL, "unknown jac %d", jac);
  if (B < 1 || T < 1 || n < 1) return pr::fail(PR_EINVAL, "sizes must be >= 1");
  if (!A || !b || !y) return pr::fail(PR_EINVAL, "A, b and y are required");
  const size_t need = pararnn_scan_workspace_bytes(jac, B, T, n);
  if (need == 0) return pr::fail(PR_EUNSUPPORTED, "no scan kernel for jac %d n %d", jac, n);
  if (need > (size_t)PR_NOALLOC_SCRATCH_BYTES)
    return pr::fail(PR_EWORKSPACE, "this scan needs %zu bytes of scratch; the static scratch holds %zu", need,
                    (size_t)PR_NOALLOC_SCRATCH_BYTES);
  int code = PR_OK;
  void *ws = device_scratch(&code);
  if (!ws) return code;
  return pr::affine_scan_run(jac, B, T, n, reverse, A, b, y, ws, need, (hipStream_t)stream);
}
