// context_copy.hip -- the context-copy (prompt lookup) drafter for MI355X
// (gfx950): proposes the verify positions that are copied from the
// request's own prompt ("Qwen3.8-27B on a Single RTX 3090: How Calibrated
// Quantization and Speculative Decoding Hit 1,000 tok/s", Technical Insight,
// the draft-from-context optimisation).
//
// One workgroup (1024 threads) per request.  Thread t scores the prompt end
// positions e = 1 + t, 1 + t + 1024, ...: it compares the prompt backwards
// from e with the key (held in LDS) until the first mismatch, so consecutive
// threads read consecutive prompt tokens and most positions cost one load;
// the first tokens of 8 positions are loaded before any is compared.
// A position's score is the 64-bit key (match length << 32 | e); the
// workgroup's maximum (shuffles, then LDS) is the longest match, latest
// occurrence on ties, and its first n_out threads copy the proposal.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "int4vh.h"
#include "int4vh_drafter.h"
#include "int4vh_internal.h"

namespace {

using int4vh_detail::hip_fail;
using int4vh_detail::launch_timed;

constexpr int kThreads = 1024;
constexpr int kMaxKey = 64;
constexpr int kBatch = 8;                 // positions per thread whose loads are in flight together

__global__ void __launch_bounds__(kThreads)
context_copy_kernel(const int32_t *prompts, const int64_t *offsets, const int32_t *keys, int n_max,
                    int n_min, int n_out, int32_t *out_tokens, int32_t *out_count,
                    int32_t *out_match_end, int32_t *out_match_len)
{
    __shared__ int32_t s_key[kMaxKey];
    __shared__ unsigned long long s_best[kThreads / 64];
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t base = offsets[r];
    const int L = (int)(offsets[r + 1] - base);
    const int32_t *P = prompts + base;
    if (tid < n_max)
        s_key[tid] = keys[(size_t)r * n_max + tid];
    __syncthreads();

    // kBatch positions per thread at a time: their first tokens are loaded
    // before any is compared (most positions stop at the first token)
    unsigned long long best = 0ull;
    const int32_t last_key = s_key[n_max - 1];
    for (int e0 = 1 + tid; e0 < L; e0 += kThreads * kBatch) {
        int32_t first[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int e = e0 + u * kThreads;
            first[u] = e < L ? P[e - 1] : 0;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int e = e0 + u * kThreads;
            if (e >= L || first[u] != last_key)
                continue;
            int ell = 1;
            const int lim = n_max < e ? n_max : e;
            while (ell < lim && P[e - 1 - ell] == s_key[n_max - 1 - ell])
                ++ell;
            if (ell >= n_min) {
                const unsigned long long k = ((unsigned long long)ell << 32) | (uint32_t)e;
                best = k > best ? k : best;
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)best, off);
        const uint32_t hi = __shfl_xor((uint32_t)(best >> 32), off);
        const unsigned long long o = ((unsigned long long)hi << 32) | lo;
        best = o > best ? o : best;
    }
    if ((tid & 63) == 0)
        s_best[tid >> 6] = best;
    __syncthreads();
    best = s_best[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w)
        best = s_best[w] > best ? s_best[w] : best;

    const int e = best ? (int)(uint32_t)best : -1;
    const int cnt = best ? (n_out < L - e ? n_out : L - e) : 0;
    if (tid < n_out)
        out_tokens[(size_t)r * n_out + tid] = tid < cnt ? P[e + tid] : -1;
    if (tid == 0) {
        out_count[r] = cnt;
        out_match_end[r] = e;
        out_match_len[r] = best ? (int)(best >> 32) : 0;
    }
}

bool aligned(const void *p, size_t al)
{
    return ((uintptr_t)p % al) == 0;
}

} // namespace

extern "C" {

int context_copy_propose_timed(const int32_t *prompts, const int64_t *prompt_offsets, int R,
                               const int32_t *keys, int n_max, int n_min, int n_out,
                               int32_t *out_tokens, int32_t *out_count, int32_t *out_match_end,
                               int32_t *out_match_len, void *stream, void *event_before,
                               void *event_after)
{
    if (R < 1 || n_max < 1 || n_max > kMaxKey || n_min < 1 || n_min > n_max || n_out < 1 ||
        n_out > 64)
        return INT4VH_EINVAL;
    if (!prompts || !prompt_offsets || !keys || !out_tokens || !out_count || !out_match_end ||
        !out_match_len)
        return INT4VH_EINVAL;
    if (!aligned(prompts, 4) || !aligned(prompt_offsets, 8) || !aligned(keys, 4) ||
        !aligned(out_tokens, 4) || !aligned(out_count, 4) || !aligned(out_match_end, 4) ||
        !aligned(out_match_len, 4))
        return INT4VH_EALIGN;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // the events take the kernel's own start and end (launch_timed)
    const hipError_t e = launch_timed(context_copy_kernel, dim3(R), dim3(kThreads), s, event_before, event_after,
                                      prompts, prompt_offsets, keys, n_max, n_min, n_out, out_tokens, out_count,
                                      out_match_end, out_match_len);
    return e == hipSuccess ? INT4VH_OK : hip_fail(e, "context-copy kernel launch");
}

int context_copy_propose(const int32_t *prompts, const int64_t *prompt_offsets, int R,
                         const int32_t *keys, int n_max, int n_min, int n_out, int32_t *out_tokens,
                         int32_t *out_count, int32_t *out_match_end, int32_t *out_match_len,
                         void *stream)
{
    return context_copy_propose_timed(prompts, prompt_offsets, R, keys, n_max, n_min, n_out,
                                      out_tokens, out_count, out_match_end, out_match_len, stream,
                                      nullptr, nullptr);
}

} // extern "C"
