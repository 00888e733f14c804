// Allocation-free loss-only entry point (sdtw_forward_static in
// include/sdtw.h): the inference-mode forward with its workspace in a
// file-scope device array instead of caller memory.
//
// Each GPU the library runs on holds its own copy of `scratch` (allocated
// with the code object, kept until the process ends).  Host code never uses
// the array's name as an address: on the first call on a device, with that
// device current, hipGetSymbolAddress resolves that device's copy, and the
// pointer is kept per device.  Every call on one device shares its copy, so
// calls that overlap on one device race (their control words and hand-off
// rows collide); the forward clears what must start at zero with kernels of
// its own before its sweep.
#include <mutex>

#include "sdtw.h"
#include "sdtw_kernels.h"

namespace sdtw {
namespace {

static_assert(SDTW_STATIC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[SDTW_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_lock;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of `scratch` (resolved once per device), or nullptr.
void* device_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> g(g_scratch_lock);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace sdtw

extern "C" int sdtw_forward_static(const float* x, const float* y, int64_t B, int64_t N,
                                   int64_t M, int64_t D, float gamma, float* loss,
                                   void* stream) {
  if (!x || !y || !loss) return SDTW_ERR_INVALID_ARG;
  const size_t need = sdtw_workspace_bytes(B, N, M, D, SDTW_MODE_INFERENCE);
  if (need == 0) return SDTW_ERR_INVALID_ARG;
  if (need > (size_t)SDTW_STATIC_SCRATCH_BYTES) return SDTW_ERR_WORKSPACE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SDTW_ERR_HIP;
  void* ws = sdtw::device_scratch(dev);
  if (!ws) return SDTW_ERR_HIP;
  sdtw::NoTimingScope no_events_;   // launch timing would create events
  return sdtw::forward_impl(x, y, B, N, M, D, gamma, SDTW_MODE_INFERENCE, ws,
                            (size_t)SDTW_STATIC_SCRATCH_BYTES, loss, stream);
}
