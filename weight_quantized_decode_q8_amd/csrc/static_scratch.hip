// static_scratch.hip -- the library's one statically allocated device buffer,
// for the entry point that allocates nothing (qgemv_q2_noalloc).
//
// The buffer is a file-scope __device__ array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code the array's name is only a host-side stand-in, so it is never passed
// to a kernel or a copy; the device address is looked up once per device
// with hipGetSymbolAddress (with that device current) and kept here, and
// only that address is handed out.
#include <hip/hip_runtime.h>

#include <mutex>

#include "qg_internal.h"

static __device__ __align__(256) unsigned char scratch[qg::kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device
}  // namespace

namespace qg {

hipError_t static_scratch(void **ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace qg
