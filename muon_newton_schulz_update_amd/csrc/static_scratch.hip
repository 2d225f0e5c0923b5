// Device scratch for the entry point that allocates nothing
// (muon_update_static): one file-scope array per device, sized for small
// batches, holding the workspace and the launch tables of a call.
//
// In host code the array's name is only a host-side stand-in: its device
// address comes from hipGetSymbolAddress, taken once per device (with that
// device current) when a handle is created, and that address is what the
// kernels receive. Every call on a device shares the device's array and
// leaves its contents behind; calls that overlap on one device race.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

namespace muon {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

size_t static_scratch_bytes() { return kScratchBytes; }

// Device address of `scratch` on device `dev`, which must be current. The
// first call per device looks the symbol up; later calls return the cached
// address.
hipError_t static_scratch_address(int dev, void** out) {
  *out = nullptr;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace muon
