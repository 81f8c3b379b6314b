// int4vh_internal.h -- library-internal helpers shared by the translation
// units of libint4vh.so (not part of the C ABI; hidden from the export table).
#ifndef INT4VH_INTERNAL_H
#define INT4VH_INTERNAL_H

#include <hip/hip_runtime.h>

#include <string>

namespace int4vh_detail {

// Largest device ordinal the library keeps per-device state for.
constexpr int kMaxDevicesPublic = 64;

// Text of the last INT4VH_EHIP error on the calling thread.
extern __attribute__((visibility("hidden"))) thread_local std::string g_last_error;

// Records "what: <HIP error name> (<text>)" as the calling thread's last
// error and returns INT4VH_EHIP.
__attribute__((visibility("hidden"))) int hip_fail(hipError_t e, const char *what);

// Compute units of device `dev` (queried once per device; 256 if unknown).
__attribute__((visibility("hidden"))) int cu_count(int dev);

} // namespace int4vh_detail

#endif // INT4VH_INTERNAL_H
