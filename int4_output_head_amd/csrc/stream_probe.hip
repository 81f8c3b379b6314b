// stream_probe.hip -- read-only HBM streaming kernels: the reference line for
// "how fast can this GPU read a head-sized buffer once", against which the
// verify kernel's weight stream is compared.  Two load paths:
//
//   mode 0  every lane loads 16 bytes per instruction into registers
//           (global_load_dwordx4, non-temporal), 8 loads in flight per lane,
//           and folds them into an xor so that no load is dead;
//   mode 1  the verify kernel's path: global_load_lds_dwordx4 moves 1 KB of
//           consecutive bytes per wave instruction straight into LDS (16
//           slots per wave, at most 13 copies in flight), nothing is read
//           back.
//
// Both walk the buffer in 1 KB blocks, block j handled by wave j mod (grid *
// 8) of a persistent grid (one 512-thread workgroup per CU), so every wave
// instruction covers whole cache lines.  Each wave writes one word (the xor
// of what it read in mode 0, zero in mode 1) to out[global wave index].
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "int4vh_probe.h"
#include "int4vh_internal.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kInFlight = 8;      // register loads in flight per lane (mode 0)
constexpr int kSlots = 16;        // LDS slots of 1 KB per wave (mode 1)

__global__ void __launch_bounds__(kThreads) stream_regs_kernel(const u32x4 *p, size_t n_blocks, uint32_t *out)
{
    const int lane = threadIdx.x & 63;
    const size_t waves = (size_t)gridDim.x * kWaves;
    const size_t w = (size_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    uint32_t acc = 0;
    size_t j = w;
    // kInFlight blocks per iteration, all loads issued before any is used
    for (; j + (kInFlight - 1) * waves < n_blocks; j += kInFlight * waves) {
        u32x4 v[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u)
            v[u] = __builtin_nontemporal_load(p + (j + u * waves) * 64 + lane);
#pragma unroll
        for (int u = 0; u < kInFlight; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; j < n_blocks; j += waves) {
        const u32x4 v = __builtin_nontemporal_load(p + j * 64 + lane);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        acc ^= __shfl_xor(acc, off);
    if (lane == 0)
        out[w] = acc;
}

__device__ __forceinline__ void copy_to_lds16(const uint8_t *src, uint8_t *lds_dst)
{
    __builtin_amdgcn_global_load_lds(src, (lds_void *)lds_dst, 16, 0, 2);
}

__global__ void __launch_bounds__(kThreads) stream_lds_kernel(const uint8_t *p, size_t n_blocks, uint32_t *out)
{
    __shared__ __attribute__((aligned(16))) uint8_t ring[kWaves][kSlots][1024];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const size_t waves = (size_t)gridDim.x * kWaves;
    const size_t w = (size_t)blockIdx.x * kWaves + wv;
    int k = 0;
    for (size_t j = w; j < n_blocks; j += waves, ++k) {
        // slot k % kSlots is free: after the wait below at most 12 later
        // copies are outstanding, so copy k - kSlots has landed
        copy_to_lds16(p + j * 1024 + lane * 16, &ring[wv][k % kSlots][0]);
        __builtin_amdgcn_s_waitcnt((12 & 0xF) | ((12 >> 4) << 14) | (0x7 << 4) | (0xF << 8));   // vmcnt(12)
    }
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));   // vmcnt(0): every copy landed
    if (lane == 0)
        out[w] = 0u;
}

} // namespace

extern "C" {

int int4vh_stream_read(const void *buf, size_t bytes, int mode, uint32_t *out, void *stream,
                       void *event_before, void *event_after)
{
    if (!buf || !out || bytes == 0 || (bytes % 1024) != 0 || (mode != 0 && mode != 1))
        return INT4VH_PROBE_EINVAL;
    if (((uintptr_t)buf % 16) != 0 || ((uintptr_t)out % 4) != 0)
        return INT4VH_PROBE_EINVAL;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return int4vh_detail::hip_fail(e, "hipGetDevice");
    int grid = int4vh_detail::cu_count(dev);
    if (grid * kWaves > INT4VH_PROBE_OUT_WORDS)
        grid = INT4VH_PROBE_OUT_WORDS / kWaves;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t n_blocks = bytes / 1024;
    // the events take the kernel's own start and end (launch_timed)
    if (mode == 0)
        e = int4vh_detail::launch_timed(stream_regs_kernel, dim3(grid), dim3(kThreads), s, event_before,
                                        event_after, static_cast<const u32x4 *>(buf), n_blocks, out);
    else
        e = int4vh_detail::launch_timed(stream_lds_kernel, dim3(grid), dim3(kThreads), s, event_before,
                                        event_after, static_cast<const uint8_t *>(buf), n_blocks, out);
    if (e != hipSuccess)
        return int4vh_detail::hip_fail(e, "stream kernel launch");
    return 0;
}

} // extern "C"
