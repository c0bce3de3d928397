// Device-resident decode workspace for pa_decode_noalloc: a fixed array in the
// library's code object, one copy per GPU, so that callers that cannot allocate
// device memory (code under graph capture, serving loops, harnesses that forbid
// allocation) can still run the split-KV decode.
//
// The host never uses the array's name as an address: in host code it names a
// host-side stand-in.  The device address of each GPU's copy is looked up once per
// device (hipGetSymbolAddress, with that device current) and kept; the decode
// kernels then receive that pointer exactly as they receive a caller's workspace.

#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"
#include "pagedattn.h"

// The partials of every split of every (sequence, query head): fp32 O, then (m, l).
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace pa {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_decode_workspace(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace pa
