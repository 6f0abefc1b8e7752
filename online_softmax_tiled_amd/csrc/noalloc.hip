// Device scratch of attn_decode_noalloc: the split-KV partial states live in
// a fixed array of device memory that the library owns, for callers that
// cannot allocate (code under HIP graph capture, serving loops that forbid
// allocation). Each GPU the library runs on holds its own copy of the array
// from the first use until the process ends; its device address is looked
// up once per device, with that device current, and used for every launch.
// Calls on one GPU share its array, so calls that overlap in time on one GPU
// race on it.
#include <mutex>

#include "common.h"

namespace attn {
namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;   // 32 MiB of partial states per GPU
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];
std::once_flag g_once[kMaxDevices];

}  // namespace

size_t decode_scratch_bytes() { return kScratchBytes; }

// Device address of the current device's scratch array (looked up on the
// first call for that device).
hipError_t decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = g_status[dev] == hipSuccess ? p : nullptr;
  });
  if (g_status[dev] != hipSuccess) return g_status[dev];
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace attn
