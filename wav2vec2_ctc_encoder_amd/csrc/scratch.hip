// Static device scratch of the allocation-free entry point
// (w2v2_forward_greedy_noalloc): a file-scope device array of fixed size that
// every GPU the library runs on holds for the life of the process.
//
// In host code the array's name is only a host-side stand-in, not a device
// address: its device address is resolved here once per device, with that
// device current, and only that address is handed to the runtime and the
// kernels.
#include <mutex>

#include "common.h"

namespace w2v2 {
namespace {

constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_setup(int device, void** addr) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  if (!g_addr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_addr[device] = p;
  }
  *addr = g_addr[device];
  return hipSuccess;
}

}  // namespace w2v2
