// Scratch memory of the decode entry point that allocates nothing
// (sekv_decode_attn_noalloc): a file-scope device array, one per GPU, held
// for the life of the process.  Host code never passes the array's name to a
// kernel (on the host it is a stand-in, not a device address): the device
// address is looked up once per device with hipGetSymbolAddress, with that
// device current, and the decode kernels take that pointer.
#include <hip/hip_runtime.h>
#include <mutex>

#include "sekv_internal.h"

namespace sekv {

namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch_init(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_ptr[device]) return hipSuccess;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != device) return hipErrorInvalidDevice;  // the caller makes the device current
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_ptr[device] = p;
  return hipSuccess;
}

void* noalloc_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  return g_ptr[device];
}

}  // namespace sekv
