// int4vh_internal.h -- library-internal helpers shared by the translation
// units of libint4vh.so (not part of the C ABI; hidden from the export table).
#ifndef INT4VH_INTERNAL_H
#define INT4VH_INTERNAL_H

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

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

template <typename T>
struct NoDeduce {
    using type = T;
};

// Launches `kernel` on stream s and returns the launch's status.  With ev0 /
// ev1 (hipEvent_t, either may be null) the events take the start and end
// timestamps of this kernel's own dispatch (hipExtLaunchKernel): their
// elapsed time is the kernel's duration, as a kernel trace measures it,
// without the cost of separate event records on the stream.
template <typename... P>
hipError_t launch_timed(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t s, void *ev0, void *ev1,
                        typename NoDeduce<P>::type... args)
{
    if (ev0 || ev1)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, s, static_cast<hipEvent_t>(ev0), static_cast<hipEvent_t>(ev1),
                              0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
    return hipGetLastError();
}

} // namespace int4vh_detail

#endif // INT4VH_INTERNAL_H
