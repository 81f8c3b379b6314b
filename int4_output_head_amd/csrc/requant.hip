// requant.hip -- offline requantisation of the output head into the
// calibrated int4 format of the verify kernels, for MI355X (gfx950).
//
// The step is the requantisation of "Qwen3.8-27B on a Single RTX 3090: How
// Calibrated Quantization and Speculative Decoding Hit 1,000 tok/s",
// Technical Insight (requantisation listing): one scale per hidden channel,
// the largest |activation| of that channel over the calibration rows divided
// by 7, then every weight divided by its channel's scale, rounded to the
// nearest integer (ties to even) and clamped to [-7, 7].  The head is then
// packed two values per byte in the verify layout.
//
// All three kernels stream HBM once:
//
//  amax_kernel   column maxima of |acts| [N, H]: a workgroup owns a strip of
//      512 channels (16 bytes = 8 channels per lane, 1 KB per wave
//      instruction) and 256 rows; its 4 waves take every fourth row, combine
//      in LDS, and merge into the float32 maxima with an integer atomic
//      maximum (non-negative binary32 values order like their bit patterns);
//      one atomic per channel and workgroup (each costs a 32-byte write).
//
//  scales_kernel amax / 7 in binary32, rounded to binary16.
//
//  pack_kernel   each wave instruction reads 1 KB of contiguous weights and
//      writes 256 contiguous bytes of the packed head; every lane keeps the same channels for its whole life
//      (the wave stride is a multiple of the row length) and holds their
//      reciprocal scales in registers.
//
// The codes equal those of the binary32 definition clamp(round_half_even(
// fl32(W / s)), -7, 7) bit for bit, without a division: a = W * (1/s)
// (reciprocal rounded once per channel) lies within 2^-20 of W / s wherever
// |W / s| <= 8, and a quotient of a binary16 or bfloat16 weight by a
// binary16 scale with |W / s| <= 7.5 is either exactly a half-integer or at
// least 2^-12 away from every half-integer (its numerator 2W - (2k+1)s is a
// multiple of the scale's last place or of the weight's, and the case
// analysis over the two formats' significand widths bounds it).  So a is
// clamped to [-7, 7], rounded to a multiple of 2^-14 (which puts every exact
// tie back on its half-integer and moves nothing across one), and rounded to
// the nearest integer, ties to even, by adding 1.5 * 2^23; the low four
// mantissa bits of that sum are the two's-complement code.  A zero or
// infinite scale has reciprocal 0 and gives code 0.  The identity is checked
// exhaustively over every binary16 scale and every binary16 and bfloat16
// weight by the test suite.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "int4vh.h"
#include "int4vh_internal.h"
#include "int4vh_requant.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

using int4vh_detail::cu_count;
using int4vh_detail::launch_timed;
using int4vh_detail::hip_fail;

constexpr int kAmaxThreads = 256;               // 4 waves
constexpr int kAmaxWaves = kAmaxThreads / 64;
constexpr int kAmaxStrip = 64 * 8;              // channels per workgroup strip
constexpr int kAmaxRows = 256;                  // calibration rows per workgroup
constexpr int kPackThreads = 256;               // 4 waves
constexpr int kPackLoads = 2;                   // 16-byte loads per lane and step
constexpr int kPackWavesPerCU = 16;             // waves per compute unit (measured best)
constexpr int kPackWave = kPackLoads * 512;     // elements per wave step (loads x 64 lanes x 8)
constexpr float kSnap = 768.0f;                 // 1.5 * 2^9: a + kSnap rounds a to a multiple of 2^-14
constexpr float kRoundAfterSnap = 12582144.0f;  // 1.5 * 2^23 - kSnap: then to the nearest integer

template <int kDtype>
__device__ __forceinline__ float decode(uint32_t bits16)
{
    if constexpr (kDtype == INT4VH_F16)
        return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
    else
        return __uint_as_float(bits16 << 16);
}

// 16-bit element j (0..7) of a 16-byte vector.
__device__ __forceinline__ uint32_t elem16(const u32x4 &v, int j)
{
    const uint32_t w = v[j >> 1];
    return (j & 1) ? (w >> 16) : (w & 0xFFFFu);
}

__device__ __forceinline__ float half_bits(uint32_t b)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

__global__ void fill_zero_f32(float *p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = 0.0f;
}

// grid (ceil(N / kAmaxRows), ceil(H / 512))
template <int kDtype>
__global__ void __launch_bounds__(kAmaxThreads)
amax_kernel(const uint16_t *acts, int N, int H, uint32_t *amax_bits)
{
    __shared__ float red[kAmaxWaves][kAmaxStrip];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int h0 = blockIdx.y * kAmaxStrip + lane * 8;
    const bool col = h0 < H;                     // H % 32 == 0: all 8 channels or none
    const long long r0 = (long long)blockIdx.x * kAmaxRows;
    const int nr = (int)((long long)N - r0 < kAmaxRows ? (long long)N - r0 : kAmaxRows);
    float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (col) {
        const uint16_t *base = acts + (size_t)r0 * H + h0;
        int r = wave;
        constexpr int kUnroll = 4;
        for (; r + (kUnroll - 1) * kAmaxWaves < nr; r += kUnroll * kAmaxWaves) {
            u32x4 v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                v[u] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4 *>(base + (size_t)(r + u * kAmaxWaves) * H));
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    m[j] = fmaxf(m[j], fabsf(decode<kDtype>(elem16(v[u], j))));
        }
        for (; r < nr; r += kAmaxWaves) {
            const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(base + (size_t)r * H));
#pragma unroll
            for (int j = 0; j < 8; ++j)
                m[j] = fmaxf(m[j], fabsf(decode<kDtype>(elem16(v, j))));
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
        red[wave][j * 64 + lane] = m[j];
    __syncthreads();
    if (wave == 0 && col) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float x = red[0][j * 64 + lane];
#pragma unroll
            for (int w = 1; w < kAmaxWaves; ++w)
                x = fmaxf(x, red[w][j * 64 + lane]);
            if (x > 0.0f)
                __hip_atomic_fetch_max(&amax_bits[h0 + j], __float_as_uint(x), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

__global__ void scales_kernel(const float *amax, int H, uint16_t *scales)
{
    const int h = blockIdx.x * blockDim.x + threadIdx.x;
    if (h < H)
        scales[h] = __builtin_bit_cast(uint16_t, (_Float16)(amax[h] / 7.0f));
}

// One wave step covers 1024 consecutive elements of the flattened head
// [V*H]: load k (0..1) of lane l reads the 8 elements at base + 512k + 8l,
// so each load instruction reads 1 KB of contiguous memory, and the 8 codes
// of a load become one 32-bit word of the packed head (each store
// instruction writes 256 contiguous bytes).  Waves take chunks w, w + S,
// w + 2S, ... with S*1024 a multiple of H, so the channels of every load of
// a lane never change and their reciprocal scales stay in registers.  Two
// register sets alternate: the loads of the next step are in flight while
// the current one is converted.
template <int kDtype>
__global__ void __launch_bounds__(kPackThreads)
pack_kernel(const uint16_t *W, const uint16_t *scales, int H, long long n_elems, long long n_chunks,
            long long wave_stride, uint32_t *out)
{
    const int lane = threadIdx.x & 63;
    const long long wv = (long long)blockIdx.x * (kPackThreads / 64) + (threadIdx.x >> 6);
    if (wv >= n_chunks)
        return;
    float rcp[kPackLoads][8];
#pragma unroll
    for (int k = 0; k < kPackLoads; ++k) {
        const int h = (int)((wv * kPackWave + k * 512 + lane * 8) % H);
        const u32x4 sv = *reinterpret_cast<const u32x4 *>(scales + h);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float s = half_bits(elem16(sv, j));
            rcp[k][j] = (s > 0.0f && s < __builtin_huge_valf()) ? 1.0f / s : 0.0f;
        }
    }
    // Loads are never predicated (a predicated load leaves the compiler
    // unable to count the loads in flight, and it then waits for all of
    // them): addresses past the head are clamped to its last 8 elements,
    // whose codes are never stored.
    const long long e_last = n_elems - 8;
    auto load = [&](long long c, u32x4 (&x)[kPackLoads]) {
#pragma unroll
        for (int k = 0; k < kPackLoads; ++k) {
            const long long e = c * kPackWave + lane * 8 + k * 512;
            x[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(W + (e < e_last ? e : e_last)));
        }
    };
    auto convert_store = [&](long long c, const u32x4 (&x)[kPackLoads]) {
#pragma unroll
        for (int k = 0; k < kPackLoads; ++k) {
            uint32_t acc = 0u;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float a = __builtin_amdgcn_fmed3f(decode<kDtype>(elem16(x[k], j)) * rcp[k][j],
                                                        -7.0f, 7.0f);
                const float t = (a + kSnap) + kRoundAfterSnap;
                acc |= (__float_as_uint(t) & 0xFu) << (4 * j);
            }
            const long long e = c * kPackWave + lane * 8 + k * 512;
            if (e < n_elems)
                __builtin_nontemporal_store(acc, out + e / 8);
        }
    };
    u32x4 xa[kPackLoads], xb[kPackLoads];
    load(wv, xa);
    for (long long c = wv; c < n_chunks; c += 2 * wave_stride) {
        load(c + wave_stride, xb);
        convert_store(c, xa);
        if (c + wave_stride >= n_chunks)
            break;
        load(c + 2 * wave_stride, xa);
        convert_store(c + wave_stride, xb);
    }
}

bool aligned(const void *p, size_t al)
{
    return ((uintptr_t)p % al) == 0;
}

bool dtype_ok(int d)
{
    return d == INT4VH_F16 || d == INT4VH_BF16;
}

bool h_ok(int H)
{
    return H >= 32 && (H % 32) == 0;
}

int launched(const char *what)
{
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? INT4VH_OK : hip_fail(e, what);
}

int do_amax(const void *acts, int dtype, int N, int H, float *amax, int accumulate, void *stream)
{
    if (!acts || !amax || N < 1 || !h_ok(H) || !dtype_ok(dtype))
        return INT4VH_EINVAL;
    if ((unsigned long long)N * (unsigned long long)H >= (1ull << 40))
        return INT4VH_EUNSUPPORTED;
    if (!aligned(acts, 16) || !aligned(amax, 4))
        return INT4VH_EALIGN;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (!accumulate) {
        hipLaunchKernelGGL(fill_zero_f32, dim3((H + 255) / 256), dim3(256), 0, s, amax, H);
        const int st = launched("amax clear launch");
        if (st != INT4VH_OK)
            return st;
    }
    const dim3 grid((unsigned)((N + kAmaxRows - 1) / kAmaxRows), (unsigned)((H + kAmaxStrip - 1) / kAmaxStrip));
    const uint16_t *a = static_cast<const uint16_t *>(acts);
    uint32_t *bits = reinterpret_cast<uint32_t *>(amax);
    if (dtype == INT4VH_F16)
        hipLaunchKernelGGL(amax_kernel<INT4VH_F16>, grid, dim3(kAmaxThreads), 0, s, a, N, H, bits);
    else
        hipLaunchKernelGGL(amax_kernel<INT4VH_BF16>, grid, dim3(kAmaxThreads), 0, s, a, N, H, bits);
    return launched("amax kernel launch");
}

int do_scales(const float *amax, int H, void *scales, void *stream)
{
    if (!amax || !scales || !h_ok(H))
        return INT4VH_EINVAL;
    if (!aligned(amax, 4) || !aligned(scales, 16))
        return INT4VH_EALIGN;
    hipLaunchKernelGGL(scales_kernel, dim3((H + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream),
                       amax, H, static_cast<uint16_t *>(scales));
    return launched("scales kernel launch");
}

int do_pack(const void *W, int dtype, int V, int H, const void *scales, uint8_t *packed, void *stream,
            void *ev0, void *ev1)
{
    if (!W || !scales || !packed || V < 1 || !h_ok(H) || !dtype_ok(dtype))
        return INT4VH_EINVAL;
    if ((long long)V * (H / 32) >= (1ll << 31))
        return INT4VH_EUNSUPPORTED;
    if (!aligned(W, 16) || !aligned(scales, 16) || !aligned(packed, 16))
        return INT4VH_EALIGN;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    const long long n_elems = (long long)V * H;
    const long long n_chunks = (n_elems + kPackWave - 1) / kPackWave;
    // wave stride S: S * kPackWave a multiple of H (fixed channels per lane)
    // and S a multiple of the 4 waves of a workgroup, about 16 waves per
    // compute unit
    long long g = H, b = kPackWave;
    while (b) {
        const long long r = g % b;
        g = b;
        b = r;
    }
    long long unit = H / g;                                        // H / gcd(H, kPackWave)
    if (unit % 4)
        unit *= (unit % 2) ? 4 : 2;                                // lcm(unit, 4)
    const long long target = (long long)kPackWavesPerCU * cu_count(dev);
    const long long stride = unit * ((target + unit - 1) / unit);
    const long long waves = n_chunks < stride ? n_chunks : stride;
    const unsigned blocks = (unsigned)((waves + 3) / 4);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t *w = static_cast<const uint16_t *>(W);
    const uint16_t *sc = static_cast<const uint16_t *>(scales);
    uint32_t *out = reinterpret_cast<uint32_t *>(packed);
    // ev0 / ev1 take the pack kernel's own start and end (launch_timed)
    e = launch_timed(dtype == INT4VH_F16 ? pack_kernel<INT4VH_F16> : pack_kernel<INT4VH_BF16>, dim3(blocks),
                     dim3(kPackThreads), s, ev0, ev1, w, sc, H, n_elems, n_chunks, stride, out);
    return e == hipSuccess ? INT4VH_OK : hip_fail(e, "pack kernel launch");
}

} // namespace

extern "C" {

int requant_lm_head_int4_amax(const void *acts, int dtype, int N, int H, float *amax, int accumulate,
                              void *stream)
{
    return do_amax(acts, dtype, N, H, amax, accumulate, stream);
}

int requant_lm_head_int4_scales(const float *amax, int H, void *scales, void *stream)
{
    return do_scales(amax, H, scales, stream);
}

int requant_lm_head_int4_pack(const void *W, int dtype, int V, int H, const void *scales,
                              uint8_t *packed, void *stream)
{
    return do_pack(W, dtype, V, H, scales, packed, stream, nullptr, nullptr);
}

int requant_lm_head_int4_pack_timed(const void *W, int dtype, int V, int H, const void *scales,
                                    uint8_t *packed, void *stream, void *event_before,
                                    void *event_after)
{
    return do_pack(W, dtype, V, H, scales, packed, stream, event_before, event_after);
}

int requant_lm_head_int4(const void *W, int w_dtype, int V, int H, const void *acts, int acts_dtype,
                         int N, float *amax, void *scales, uint8_t *packed, void *stream)
{
    // validate everything before the first launch
    if (!W || !acts || !amax || !scales || !packed || V < 1 || N < 1 || !h_ok(H) ||
        !dtype_ok(w_dtype) || !dtype_ok(acts_dtype))
        return INT4VH_EINVAL;
    if ((long long)V * (H / 32) >= (1ll << 31) ||
        (unsigned long long)N * (unsigned long long)H >= (1ull << 40))
        return INT4VH_EUNSUPPORTED;
    if (!aligned(W, 16) || !aligned(acts, 16) || !aligned(amax, 4) || !aligned(scales, 16) ||
        !aligned(packed, 16))
        return INT4VH_EALIGN;
    int st = do_amax(acts, acts_dtype, N, H, amax, 0, stream);
    if (st != INT4VH_OK)
        return st;
    st = do_scales(amax, H, scales, stream);
    if (st != INT4VH_OK)
        return st;
    return do_pack(W, w_dtype, V, H, scales, packed, stream, nullptr, nullptr);
}

} // extern "C"
