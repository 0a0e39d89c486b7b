// Device scratch of the allocation-free entry point (dmuon_ns_batched_noalloc).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "dmuon.h"

namespace dmuon {

// Size of the statically allocated scratch array on every device the library
// runs on (held until the process ends).
constexpr size_t kScratchBytes = DMUON_NOALLOC_SCRATCH_BYTES;

// Device address of the scratch array on the current device.  The first call
// on a device resolves it with hipGetSymbolAddress (that device current) and
// keeps it; later calls return the kept address.  Thread-safe.
hipError_t scratch_address(char** out);

}  // namespace dmuon
