// Thread-local error message shared by the host-side translation units.
#pragma once

namespace dmuon {
// Record a printf-style message for dmuon_last_error() and return `code`.
int fail(int code, const char* fmt, ...);
}  // namespace dmuon
