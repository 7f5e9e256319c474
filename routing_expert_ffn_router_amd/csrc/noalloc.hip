// Static scratch of the dispatch for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid device allocation).
//
// The dispatch kernels keep two tables in scratch memory: the per-tile expert histogram
// and its per-expert exclusive scan ([ntiles, E] int32 each).  moe_dispatch takes them from
// the caller's workspace; moe_dispatch_no_workspace takes them from the array below, one
// copy per GPU, which the library holds until the process ends.  Both tables are written in
// full by every call before they are read, so nothing needs clearing between calls; calls
// that overlap on one GPU share the array and race.
//
// Host code never uses the array's name as a device address (on the host it names a
// stand-in, not the GPU's copy): the first call on each device asks the runtime for that
// device's address once, with the device current, and every later use goes through it.
#include <mutex>
#include <vector>

#include <hip/hip_runtime.h>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MOE_DISPATCH_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // per device: address of that device's copy

}  // namespace

namespace moe {

hipError_t dispatch_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr.empty()) {
    int n = 0;
    if ((e = hipGetDeviceCount(&n)) != hipSuccess) return e;
    g_scratch_ptr.assign((size_t)n, nullptr);
  }
  if (dev < 0 || (size_t)dev >= g_scratch_ptr.size()) return hipErrorInvalidDevice;
  if (!g_scratch_ptr[(size_t)dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[(size_t)dev] = p;
  }
  *ptr = g_scratch_ptr[(size_t)dev];
  *bytes = MOE_DISPATCH_SCRATCH_BYTES;
  return hipSuccess;
}

}  // namespace moe
