// Statically allocated device scratch for callers that cannot allocate: the
// workspace of dmuon_ns_batched_noalloc (the same launch sequence as
// dmuon_ns_batched, whose workspace the library otherwise allocates with
// hipMalloc) lives in this array instead.  Every device gets its own copy at
// its own address when the code object is loaded there.
//
// In host code the array's name is only a host-side stand-in: the device
// address is obtained once per device with hipGetSymbolAddress and that
// address alone is handed to kernels.

#include "scratch.h"

#include <map>
#include <mutex>

static __device__ __align__(256) char scratch[dmuon::kScratchBytes];

namespace dmuon {
namespace {
std::mutex g_scratch_mu;
std::map<int, char*> g_scratch_ptr;  // device -> address of its scratch array
}  // namespace

hipError_t scratch_address(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    it = g_scratch_ptr.emplace(dev, static_cast<char*>(p)).first;
  }
  *out = it->second;
  return hipSuccess;
}

}  // namespace dmuon
