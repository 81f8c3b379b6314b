// int4vh.hip -- int4 lm_head speculative verification for MI355X (gfx950).
//
// One call computes, for a verify block of M <= 16 rows of final hidden
// states (up to 64 in token groups of 16, below), every logit of a
// calibrated int4 head, the greedy argmax of each row and the
// accepted-prefix length of each request.  The head is the
// requantised lm_head of "Qwen3.8-27B on a Single RTX 3090: How Calibrated
// Quantization and Speculative Decoding Hit 1,000 tok/s", Technical Insight
// (values in [-7, 7], one scale per hidden channel); the greedy compare of a
// drafted block is the verify step of the same section; blocks of up to 16
// positions are from "HyperQwen on one RTX 3090: a first-time developer's
// guide to the 381-token claim", "What actually became faster?".
//
// Two launches on the caller's stream (one for a block of one or two rows,
// whose staging runs inside verify_kernel):
//
//  stage_kernel  turns hidden*scale (exact in binary32) into a 24-bit
//      fixed-point code per token (power-of-two step from the token's largest
//      |hidden*scale|), splits each code into three signed bytes (limbs) and
//      writes them to the workspace already laid out as MFMA A-operand
//      fragments, together with each token's step exponent.
//
//  verify_kernel  streams the head once.  Persistent workgroups (one per CU)
//      walk vocabulary tiles of 16 rows b, b+G, b+2G, ...  A tile (16 rows x
//      H/2 bytes, contiguous in memory) is copied straight into an LDS ring
//      with global_load_lds_dwordx4: each instruction moves 1 KB of
//      consecutive bytes (whole cache lines, non-temporal), and the ring holds
//      several tiles in flight without using registers.  The 16-byte chunks
//      are XOR-swizzled inside each 1 KB block so that the fragment reads
//      below hit distinct LDS banks.  The 8 waves split the hidden dimension;
//      each keeps its slice of the activation limbs in registers for the whole
//      call.  A weight nibble becomes the int8 value 16*q by moving it to the
//      high half of a byte (two bit operations per 8 weights) and
//      v_mfma_i32_16x16x64_i8 accumulates exactly in int32.  Each wave
//      combines its limbs (weights 2^16, 2^8, 1) into partial sums -- integers
//      below 2^44, held exactly in binary64 -- and stores them in LDS; after
//      the next barrier the lanes that own a token add the 8 waves' partials
//      (exact, so independent of order) and round the logit to binary32 once.
//      Each wave folds two tokens' logits into a running argmax.  The last
//      workgroup to finish (two-level atomic ticket) merges the per-workgroup
//      winners, writes the outputs, counts accepted drafts and resets the
//      tickets.
//
//  Blocks of 17 to 64 rows run the same two kernels in token groups of 16:
//  the registers of a workgroup hold the activation codes of 16 rows (all 24
//  bits of 16 rows x 5120 channels fill half the register file), so each
//  group gets its own workgroups, one per tile set, and the workgroups of a
//  set (one per group, 8 blockIdx apart: the same XCD) walk the same tiles
//  at the same time, so a tile comes from HBM once and from that XCD's L2
//  for the others.  Each group's workgroup repeats the per-tile compute
//  (the int8 MFMAs, at the rate the matrix cores sustain under this load,
//  plus the nibble conversion and the cross-wave reduction), so the call
//  costs about 46 us more per group; above 64 rows the matrix-core batch
//  kernels below are faster.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <type_traits>
#include <string>

#include "int4vh.h"
#include "int4vh_internal.h"

namespace int4vh_detail {

thread_local std::string g_last_error;

int hip_fail(hipError_t e, const char *what)
{
    g_last_error = std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
    return INT4VH_EHIP;
}

namespace {
constexpr int kMaxDevices = kMaxDevicesPublic;
int g_cu_count[kMaxDevices];
std::once_flag g_cu_once[kMaxDevices];
} // namespace

int cu_count(int dev)
{
    if (dev < 0 || dev >= kMaxDevices)
        return 256;
    std::call_once(g_cu_once[dev], [dev] {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        g_cu_count[dev] = n;
    });
    return g_cu_count[dev];
}

} // namespace int4vh_detail

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWaves = 8;                 // waves per workgroup
constexpr int kThreads = 64 * kWaves;     // 512
constexpr int kTileRows = 16;             // vocabulary rows per tile (MFMA N)
constexpr int kUnitH = 128;               // hidden channels per unit (16 rows x 64 B = 1 KB)
constexpr int kMaxUnitsPerWave = 8;       // 8 waves x 8 units x 128 = 8192 channels
constexpr int kMaxRows = 16;              // rows per token group (MFMA M)
constexpr int kMaxGroups = 4;             // token groups per launch: up to 64 rows in the weight stream
constexpr int kCodeMax = 8355711;         // |code| bound: all three limbs stay in int8
constexpr int kMaxGrid = 1024;            // partial slots in the workspace
constexpr int kStageThreads = 512;        // threads of stage_kernel (one 16-channel chunk each)

constexpr int kBatchMaxRows = 4096;       // rows per launch of the batch path

// Workspace layout (bytes from the 256-byte aligned base).  The control block
// (tickets, per-row keys, the sampled epilogue's draft flags) is zeroed by
// workspace_init and left zeroed by every call; the rest is written before it
// is read.
constexpr size_t kWsTicket = 0;                                   // uint32 ticket
constexpr size_t kWsKeys = 256;                                   // uint64 [4096] batch winner keys
// Atomics on one 128-byte line serialise at the memory side (about 13 ns
// each), so a ticket taken by every workgroup at once costs microseconds;
// the tickets are two-level, one line per group of 16 workgroups.
constexpr int kGroupWgs = 16;                                     // workgroups per ticket group
constexpr int kTicketStride = 32;                                 // uint32 per group ticket (128 B)
constexpr size_t kWsGroupTk = kWsKeys + (size_t)kBatchMaxRows * 8;   // uint32 [64][32] group tickets
constexpr size_t kWsDraftSeen = kWsGroupTk + (size_t)(kMaxGrid / kGroupWgs) * kTicketStride * 4;
                                                                  // int32 [64] draft logit written
constexpr size_t kWsDraftLogit = kWsDraftSeen + 256;                  // float [64] the draft's logit
constexpr size_t kWsCtlBytes = kWsDraftSeen + 512;
constexpr size_t kWsExp = kWsCtlBytes;                            // int32 [4096] step exponents
constexpr size_t kWsPart = kWsExp + (size_t)kBatchMaxRows * 4;    // uint64 [kMaxGrid][16]
constexpr size_t kWsFrag = kWsPart + (size_t)kMaxGrid * kMaxRows * 8;   // activation fragments
constexpr size_t kFragBytes = (size_t)kWaves * kMaxUnitsPerWave * 2 * 3 * 64 * 16;
constexpr int kMaxTopK = 16;              // largest k of the sampled epilogue
constexpr int kSampledMaxGrid = 256;      // workgroups of a sampled call (16 groups of 16)
constexpr size_t kWsTopK = kWsFrag + kFragBytes;                  // uint64 [256][16][kMaxTopK]
constexpr size_t kWsGroupTopK = kWsTopK + (size_t)kSampledMaxGrid * kMaxRows * kMaxTopK * 8;
constexpr size_t kWsLse = kWsGroupTopK + (size_t)(kSampledMaxGrid / 16) * kMaxRows * kMaxTopK * 8;
constexpr size_t kWsGroupLse = kWsLse + (size_t)kSampledMaxGrid * kMaxRows * 8;   // (m, s) pairs
constexpr size_t kWsBytes = kWsGroupLse + (size_t)(kSampledMaxGrid / 16) * kMaxRows * 8;
static_assert(kWsCtlBytes % 256 == 0 && kWsExp % 256 == 0 && kWsPart % 256 == 0 &&
                  kWsFrag % 256 == 0 && kWsTopK % 256 == 0 && kWsGroupTopK % 256 == 0,
              "workspace regions stay 256-byte aligned");

#ifndef INT4VH_WEIGHT_AUX
#define INT4VH_WEIGHT_AUX 2                // cache policy of the weight stream: non-temporal
#endif

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8).
constexpr int waitcnt_vm(int n)
{
    return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}
constexpr int kWaitLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);

// Workgroup barrier without the release/acquire fences of __syncthreads (a
// fence would also wait for the weight copies still in flight).  The caller
// issues the s_waitcnt that its protocol needs; the empty asm statements keep
// the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void barrier_no_fence()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// LDS writes of the partial sums go through inline asm: the compiler orders
// every LDS write it can see after all LDS copies still in flight (a full
// vmcnt(0) drain of the weight stream), although the partial sums and the
// ring never overlap.  Completion of these writes is covered by the explicit
// lgkmcnt(0) before each barrier.
typedef __attribute__((address_space(3))) unsigned long long lds_u64;

__device__ __forceinline__ uint32_t lds_offset(unsigned long long *p)
{
    return (uint32_t)(size_t)(lds_u64 *)p;
}

__device__ __forceinline__ void lds_store_u64(unsigned long long *p, unsigned long long v)
{
    asm volatile("ds_write_b64 %0, %1" ::"v"(lds_offset(p)), "v"(v) : "memory");
}
// One 16-byte-per-lane copy from global memory straight into LDS (lane l
// lands at lds_dst + 16*l).  Kept out of line of the kernels' bodies.
template <int kAux>
__device__ __forceinline__ void copy_to_lds16(const uint8_t *src, uint8_t *lds_dst)
{
    __builtin_amdgcn_global_load_lds(src, (lds_void *)lds_dst, 16, 0, kAux);
}

// A value the compiler cannot prove uniform but the caller knows is (the
// wave index), moved to a scalar register.
__device__ __forceinline__ int wave_uniform(int v)
{
    return __builtin_amdgcn_readfirstlane(v);
}

// Cross-lane moves within a 16-lane DPP row (no LDS traffic, unlike
// __shfl): row_ror:n gives each lane the value of the lane n places before
// it in its row, cyclically.
template <int kCtl>
__device__ __forceinline__ float dpp_f32(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtl, 0xF, 0xF, false));
}
template <int kCtl>
__device__ __forceinline__ int dpp_i32(int x)
{
    return __builtin_amdgcn_update_dpp(0, x, kCtl, 0xF, 0xF, false);
}
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;

// Maximum of x over the wave, in every lane (rotations within the rows,
// then the four row results).  Called by all lanes.
__device__ __forceinline__ float wave_max(float x)
{
    x = fmaxf(x, dpp_f32<kRowRor1>(x));
    x = fmaxf(x, dpp_f32<kRowRor2>(x));
    x = fmaxf(x, dpp_f32<kRowRor4>(x));
    x = fmaxf(x, dpp_f32<kRowRor8>(x));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Three 8-byte LDS reads, complete on return.  Written as one asm block:
// reads of a ring slot that the weight copies also fill would otherwise
// make the compiler wait for every copy in flight (it cannot tell the
// slots apart).
__device__ __forceinline__ void lds_load3_u64(const void *p0, const void *p1, const void *p2, uint2 &v0, uint2 &v1,
                                              uint2 &v2)
{
    asm volatile("ds_read_b64 %0, %3\n\t"
                 "ds_read_b64 %1, %4\n\t"
                 "ds_read_b64 %2, %5\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v0), "=&v"(v1), "=&v"(v2)
                 : "v"(lds_offset(reinterpret_cast<unsigned long long *>(const_cast<void *>(p0)))),
                   "v"(lds_offset(reinterpret_cast<unsigned long long *>(const_cast<void *>(p1)))),
                   "v"(lds_offset(reinterpret_cast<unsigned long long *>(const_cast<void *>(p2))))
                 : "memory");
}

// Element `hi` (0 or 1) of a wave-uniform pair of int32 in global memory,
// loaded through the scalar unit and complete on return (it counts against
// lgkmcnt only, so no vector load in flight is waited for).
__device__ __forceinline__ int load_exp_pair(const int32_t *p, int hi)
{
    unsigned long long xy;
    asm volatile("s_load_dwordx2 %0, %1, 0x0\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=s"(xy)
                 : "s"(p)
                 : "memory");
    return (int)(uint32_t)(hi ? xy >> 32 : xy);
}

__device__ __forceinline__ void lds_store_u32(void *p, uint32_t v)
{
    asm volatile("ds_write_b32 %0, %1" ::"v"(lds_offset(reinterpret_cast<unsigned long long *>(p))), "v"(v)
                 : "memory");
}

struct Args {
    const uint16_t *hidden;   // [M, H] binary16
    const uint8_t *w;         // [V, H/2]
    const uint16_t *scales;   // [H]
    const int32_t *draft;     // [R, T-1] or null
    float *logits_max;        // [M]
    int32_t *argmax;          // [M]
    int32_t *n_acc;           // [R]
    float *logits_out;        // [M, V] or null
    const int32_t *vmap;      // [V] token id of each head row, or null (identity)
    uint64_t *part;           // [grid, M] packed (index << 32 | value bits)
    // sampled epilogue (top-k sampling at a temperature; unused when off)
    unsigned long long *part_topk;   // [groups * sets, rows per workgroup, kTopK] per-workgroup top-k keys
    unsigned long long *group_topk;  // [merge groups, rows per workgroup, kTopK] per-merge-group keys
    uint32_t *group_ticket;          // [64][kTicketStride] per-group tickets (word 0), zero between calls
    int top_k;                // k <= kTopK
    float tau;                // temperature > 0
    const float *dprob;       // [R, T-1] drafter probability of each draft
    const float *unif;        // [R, T-1] uniforms in [0, 1)
    int32_t *topk_ids;        // [M, k] (unused when top_k == 0)
    float *topk_logits;       // [M, k]
    float *p_draft;           // [R, T-1]
    float *lse_out;           // [M] log sum exp(logit / tau), or null
    uint64_t *part_lse;       // [groups * sets, rows per workgroup] per-workgroup (max, sum) of exp2 terms
    uint64_t *group_lse;      // [merge groups, rows per workgroup]
    int32_t *draft_seen;      // [M <= 64] set when the draft's logit was written; zero between calls
    float *draft_logit;       // [M]
    uint32_t *ticket;
    int32_t *exps;            // [16]
    const u32x4 *frag;        // activation fragments
    u32x4 *frag_out;
    int R, T, M, V, H;
    int n_units;              // ceil(H / 128)
    int n_tiles;              // ceil(V / 16)
    unsigned long long w_bytes;
    // Blocks of more than 16 rows: groups of 16 rows, each with its own
    // workgroups (one per tile set) and activation fragments
    int n_groups;             // ceil(M / 16); 1 up to 16 rows
    int n_sets;               // workgroups per group; grid = n_groups * n_sets
    size_t group_words;       // 16-byte fragment words per group
};

__device__ __forceinline__ float half_bits_to_float(uint32_t b)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// (value, index) order: larger value first, lower index on equal values.
// -0.0 == +0.0 compare equal, so they tie and the lower index wins.
__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2)
{
    return v1 > v2 || (v1 == v2 && i1 < i2);
}

// The better (value, index) pair over the lane's 16-lane row, in every lane
// of the row (rotations: each step doubles the window a lane has seen).
__device__ __forceinline__ void row_best16(float &v, int &i)
{
#define INT4VH_ROW_BEST_STEP(C)                                        \
    {                                                                  \
        const float ov = dpp_f32<C>(v);                                \
        const int oi = dpp_i32<C>(i);                                  \
        const bool take = better(ov, oi, v, i);                        \
        v = take ? ov : v;                                             \
        i = take ? oi : i;                                             \
    }
    INT4VH_ROW_BEST_STEP(kRowRor1)
    INT4VH_ROW_BEST_STEP(kRowRor2)
    INT4VH_ROW_BEST_STEP(kRowRor4)
    INT4VH_ROW_BEST_STEP(kRowRor8)
#undef INT4VH_ROW_BEST_STEP
}

// (max, sum) pairs of exp2 terms and plain sums over the lane's 16-lane row,
// in every lane of the row.
__device__ __forceinline__ void lse_combine(float &m, float &s, float mo, float so);
__device__ __forceinline__ void row_lse16(float &m, float &s)
{
    lse_combine(m, s, dpp_f32<kRowRor1>(m), dpp_f32<kRowRor1>(s));
    lse_combine(m, s, dpp_f32<kRowRor2>(m), dpp_f32<kRowRor2>(s));
    lse_combine(m, s, dpp_f32<kRowRor4>(m), dpp_f32<kRowRor4>(s));
    lse_combine(m, s, dpp_f32<kRowRor8>(m), dpp_f32<kRowRor8>(s));
}
__device__ __forceinline__ float row_sum16(float x)
{
    x += dpp_f32<kRowRor1>(x);
    x += dpp_f32<kRowRor2>(x);
    x += dpp_f32<kRowRor4>(x);
    x += dpp_f32<kRowRor8>(x);
    return x;
}

__device__ __forceinline__ uint64_t pack_pair(float v, int i)
{
    return ((uint64_t)(uint32_t)i << 32) | (uint64_t)__float_as_uint(v);
}

// Key of a (value, index) pair whose unsigned order is the argmax order:
// larger value first, then lower index.  -0.0 is keyed as +0.0.
__device__ __forceinline__ unsigned long long order_key(float v, int i)
{
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u)
        u = 0u;
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)u << 32) | (unsigned long long)(~(uint32_t)i);
}

__device__ __forceinline__ float key_value(unsigned long long k)
{
    const uint32_t u = (uint32_t)(k >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

__device__ __forceinline__ int key_index(unsigned long long k)
{
    return (int)(~(uint32_t)k);
}


// Top-k lists of the sampled epilogue are distributed over an aligned group
// of 16 lanes (one DPP row): lane j of the group holds the rank-j order key
// (best first; keys are unique because the index is part of the key, and key
// 0, below every real key, marks an empty rank).

__device__ __forceinline__ unsigned long long key_readlane(unsigned long long k, int src)
{
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)k, src);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(k >> 32), src);
    return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ unsigned long long key_shfl(unsigned long long k, int src)
{
    const uint32_t lo = __shfl((uint32_t)k, src);
    const uint32_t hi = __shfl((uint32_t)(k >> 32), src);
    return ((unsigned long long)hi << 32) | lo;
}

// The key of the previous lane of the DPP row (row_shr:1; lane 0 of the row
// gets 0).
__device__ __forceinline__ unsigned long long key_row_prev(unsigned long long k)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)k, 0x111, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(k >> 32), 0x111, 0xF, 0xF, false);
    return ((unsigned long long)hi << 32) | lo;
}

// Insert `key` (equal on the group's lanes) into the distributed list whose
// rank-j entry this lane holds; the last entry drops out.
__device__ __forceinline__ unsigned long long dlist_insert(unsigned long long mine, unsigned long long key)
{
    const bool first = (threadIdx.x & 15) == 0;          // rank 0 of the group
    const unsigned long long up = key_row_prev(mine);    // rank j-1 (an empty rank is 0)
    return (!first && key > up) ? up : (key > mine ? key : mine);
}

// 64-bit DPP move within a row of 16 lanes (lanes whose source is outside
// the row get 0).
template <int kCtrl>
__device__ __forceinline__ unsigned long long key_dpp(unsigned long long k)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)k, kCtrl, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(k >> 32), kCtrl, 0xF, 0xF, false);
    return ((unsigned long long)hi << 32) | lo;
}

// The key of lane j ^ S of the row: quad_perm for S = 1, 2; row_shl:4 /
// row_shr:4 for S = 4; row_ror:8 for S = 8.
template <int S>
__device__ __forceinline__ unsigned long long key_row_xor(unsigned long long k, int j)
{
    if constexpr (S == 1)
        return key_dpp<0xB1>(k);
    else if constexpr (S == 2)
        return key_dpp<0x4E>(k);
    else if constexpr (S == 4) {
        // both moves with every lane active (a DPP move inside a divergent
        // branch reads inactive source lanes as 0), then the select
        const unsigned long long from_above = key_dpp<0x104>(k);
        const unsigned long long from_below = key_dpp<0x114>(k);
        return (j & 4) ? from_below : from_above;
    } else
        return key_dpp<0x128>(k);
}

// Compare-exchange with lane j ^ S: keep the larger key or the smaller one.
template <int S>
__device__ __forceinline__ unsigned long long key_cex(unsigned long long c, int j, bool keep_max)
{
    const unsigned long long o = key_row_xor<S>(c, j);
    return (keep_max == (c > o)) ? c : o;
}

// Sort the 16 keys of a row best first (bitonic network, 10 stages).
__device__ __forceinline__ unsigned long long row_sort16(unsigned long long c, int j)
{
    c = key_cex<1>(c, j, ((j & 1) == 0) == ((j & 2) == 0));
    c = key_cex<2>(c, j, ((j & 2) == 0) == ((j & 4) == 0));
    c = key_cex<1>(c, j, ((j & 1) == 0) == ((j & 4) == 0));
    c = key_cex<4>(c, j, ((j & 4) == 0) == ((j & 8) == 0));
    c = key_cex<2>(c, j, ((j & 2) == 0) == ((j & 8) == 0));
    c = key_cex<1>(c, j, ((j & 1) == 0) == ((j & 8) == 0));
    c = key_cex<8>(c, j, (j & 8) == 0);
    c = key_cex<4>(c, j, (j & 4) == 0);
    c = key_cex<2>(c, j, (j & 2) == 0);
    return key_cex<1>(c, j, (j & 1) == 0);
}

// Top 16 of two distributed lists: a = rank-j key of list A, b_rev = rank
// (15-j) key of list B.  max(A[j], B[15-j]) is a bitonic sequence holding the
// 16 largest keys; four compare-exchange stages sort it (the lower lane of
// each pair keeps the larger key).
__device__ __forceinline__ unsigned long long dlist_merge(unsigned long long a, unsigned long long b_rev,
                                                          int lane)
{
    const int j = lane & 15;
    const unsigned long long c = a > b_rev ? a : b_rev;
    return key_cex<1>(key_cex<2>(key_cex<4>(key_cex<8>(c, j, (j & 8) == 0), j, (j & 4) == 0), j,
                                 (j & 2) == 0),
                      j, (j & 1) == 0);
}

// Running sums of exp2 terms, (m, s) = (maximum exponent, sum of
// exp2(z - m)); an empty pair is (-inf, 0).  Combination scales each sum to
// the larger maximum (factor 1 when the maxima are equal, including two
// empty pairs).
__device__ __forceinline__ void lse_combine(float &m, float &s, float mo, float so)
{
    const float mn = fmaxf(m, mo);
    const float f1 = m == mn ? 1.0f : __builtin_amdgcn_exp2f(m - mn);
    const float f2 = mo == mn ? 1.0f : __builtin_amdgcn_exp2f(mo - mn);
    s = s * f1 + so * f2;
    m = mn;
}

// Adds one term exp2(z) to a running (m, s) pair: one exp2.
__device__ __forceinline__ void lse_add(float &m, float &s, float z)
{
    const float mn = fmaxf(m, z);
    const float e = __builtin_amdgcn_exp2f(fminf(m, z) - mn);   // exp2 of (smaller - larger)
    s = z > m ? s * e + 1.0f : s + e;
    m = mn;
}

__device__ __forceinline__ uint64_t lse_pack(float m, float s)
{
    return ((uint64_t)__float_as_uint(s) << 32) | (uint64_t)__float_as_uint(m);
}

// (m, s) pairs [n <= 16] of one row, stored [n][stride] from `pairs`: lane
// j of each 16-lane group loads pair j of row `row` (all loads in flight at
// once) and a fixed sequence of row rotations combines them; every lane of
// the group ends with the same pair.  Called by all lanes of the wave.
__device__ __forceinline__ uint64_t lse_load16(const uint64_t *pairs, int n, int stride, int row)
{
    const int j = threadIdx.x & 15;
    return __hip_atomic_load(&pairs[(size_t)(j < n ? j : 0) * stride + row], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void lse_combine16(uint64_t pr, int n, float &m, float &s)
{
    const int j = threadIdx.x & 15;
    m = j < n ? __uint_as_float((uint32_t)pr) : -__builtin_huge_valf();
    s = j < n ? __uint_as_float((uint32_t)(pr >> 32)) : 0.0f;
    row_lse16(m, s);
}

// Merge up to 16 published top-k lists ([n_lists][stride][kTopK] keys, rank
// order) per token of the first M <= 16; a workgroup of 512 threads, wave w
// handling tokens 2w and 2w+1 with 32 lanes each.  Each half of the 32 lanes
// folds the lists of its parity (all loads issued first), then the halves
// merge; every lane returns the rank-(lane & 15) key of its token's merged
// list.
template <int kTopK>
__device__ __forceinline__ unsigned long long merge_topk_lists(const unsigned long long *lists, int n_lists,
                                                               int stride, int M, int lane)
{
    const int wave = threadIdx.x >> 6;
    const int m = 2 * wave + (lane >> 5);
    const int mm = m < M ? m : M - 1;
    const int h = (lane >> 4) & 1;
    const int j = lane & 15;
    // lists 2i + h, even i by rank and odd i reversed; every load issued
    // before any is used (clamped to a valid slot, zero = empty when absent)
    unsigned long long e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int w = 2 * i + h;
        const int r = (i & 1) == 0 ? j : 15 - j;
        const bool live = w < n_lists && r < kTopK;
        const unsigned long long v = __hip_atomic_load(&lists[((size_t)(live ? w : 0) * stride + mm) * kTopK + (live ? r : 0)],
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        e[i] = live ? v : 0ull;
    }
    // a merge tree (empty lists merge harmlessly): depth 3 instead of 7
    const unsigned long long c0 = dlist_merge(e[0], e[1], lane);
    const unsigned long long c1 = dlist_merge(e[2], e[3], lane);
    const unsigned long long c2 = dlist_merge(e[4], e[5], lane);
    const unsigned long long c3 = dlist_merge(e[6], e[7], lane);
    const unsigned long long d0 = dlist_merge(c0, key_dpp<0x140>(c1), lane);   // row_mirror: reversed
    const unsigned long long d1 = dlist_merge(c2, key_dpp<0x140>(c3), lane);
    const unsigned long long c = dlist_merge(d0, key_dpp<0x140>(d1), lane);
    return dlist_merge(c, key_shfl(c, ((lane ^ 16) & ~15) | (15 - j)), lane);
}

// 16 consecutive hidden*scale products (binary32, exact) of one row.
__device__ __forceinline__ void load_xs16(const uint16_t *hrow, const uint16_t *scales, int h0,
                                          float (&xs)[16])
{
    const u32x4 *hp = reinterpret_cast<const u32x4 *>(hrow + h0);
    const u32x4 *sp = reinterpret_cast<const u32x4 *>(scales + h0);
    u32x4 hx[2] = {hp[0], hp[1]};
    u32x4 sx[2] = {sp[0], sp[1]};
    // all four loads in flight before the first use (left alone, the
    // scheduler waits for one of them before issuing the others)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        uint32_t hw = hx[j >> 3][(j >> 1) & 3], sw = sx[j >> 3][(j >> 1) & 3];
        uint32_t hb = (j & 1) ? (hw >> 16) : (hw & 0xFFFF);
        uint32_t sb = (j & 1) ? (sw >> 16) : (sw & 0xFFFF);
        xs[j] = half_bits_to_float(hb) * half_bits_to_float(sb);
    }
}

// Slot order of one K-step fragment (4 registers x 4 bytes), matching the
// weight dequantisation below: register v, byte b holds hidden offset
// 8*(v>>1) + 2*b + (v&1) within the 16 channels of the fragment.
__device__ __forceinline__ int frag_offset(int v, int b)
{
    return 8 * (v >> 1) + 2 * b + (v & 1);
}

// Rows of the 16-row MFMA operand A are (token, limb) slots: slot s of group
// g (s = 16*g + row) holds limb s / kP of token s % kP, so every lane carries
// one token (row % kP) and the three limbs of all tokens need
// ceil(3*kP / 16) MFMAs per K-step: kP = 5 (<= 5 rows, 1 MFMA), 8 (<= 8
// rows, 2 MFMAs) or 16 (<= 16 rows, 3 MFMAs).
template <int kP>
struct Slots {
    static constexpr int kGroups = (3 * kP + 15) / 16;
};

// Index of the fragment (wave, unit i, K-step t, group g, lane) in the workspace.
template <int kP, int kUnits>
__device__ __forceinline__ size_t frag_index(int wave, int i, int t, int g, int lane)
{
    return ((((size_t)wave * kUnits + i) * 2 + t) * Slots<kP>::kGroups + g) * 64 + lane;
}

// Smallest e with amax / 2^e <= kCodeMax (0 for amax == 0).
__device__ __forceinline__ int code_exponent(float amax)
{
    if (!(amax > 0.0f))
        return 0;
    int ex;
    frexpf(amax, &ex);                    // amax = f * 2^ex, f in [0.5, 1)
    int e = ex - 23;                      // amax / 2^e in [2^22, 2^23)
    if (ldexpf(amax, -e) > (float)kCodeMax)
        ++e;
    return e;
}

// Codes of 16 products (step 2^e, round to nearest even) split into three
// signed bytes, high limb first (code = 2^16*l0 + 2^8*l1 + l2), packed in
// fragment slot order: limbw[l][v] byte b holds limb l of the product at
// frag_offset(v, b).
__device__ __forceinline__ void split_limbs(const float (&xs)[16], int e, uint32_t (&limbw)[3][4])
{
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        uint32_t w0 = 0, w1 = 0, w2 = 0;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const int cval = (int)rintf(ldexpf(xs[frag_offset(v, bb)], -e));
            const int lo = (int)(int8_t)(cval & 0xFF);
            const int c1 = (cval - lo) >> 8;
            const int mid = (int)(int8_t)(c1 & 0xFF);
            const int hi = (c1 - mid) >> 8;
            w0 |= (uint32_t)(uint8_t)hi << (8 * bb);
            w1 |= (uint32_t)(uint8_t)mid << (8 * bb);
            w2 |= (uint32_t)(uint8_t)lo << (8 * bb);
        }
        limbw[0][v] = w0;
        limbw[1][v] = w1;
        limbw[2][v] = w2;
    }
}

// Accepted-prefix lengths from one wave's ballot of per-row decisions (bit
// r*T + t: draft t of request r accepted; R*T <= 64): request r accepts up
// to its first rejected draft.  Lane r < R writes n_acc[r].
__device__ __forceinline__ void accept_from_ballot(unsigned long long bits, int T, int R, int lane, int32_t *n_acc)
{
    if (lane < R) {
        const unsigned long long drafts = (1ull << (T - 1)) - 1ull;     // T - 1 <= 15 draft bits
        const unsigned long long rb = (bits >> (lane * T)) & drafts;
        n_acc[lane] = rb == drafts ? T - 1 : __builtin_ctzll(~rb);
    }
}

// ---------------------------------------------------------------- stage_kernel
// One workgroup per token slot tau < kP.  Thread c owns the 16-channel chunk
// c of the token's row: it loads x and s for its chunk once, the block finds
// the token's largest |x*s|, and the thread turns its 16 products into codes
// and writes every fragment word that holds this chunk (one per lane row
// n16 = tau, tau + kP, ... and lane group).  Slots tau >= M, and rows whose
// limb index is 3, get zeros.
template <int kP, int kUnits>
__global__ void __launch_bounds__(kStageThreads) stage_kernel(Args a)
{
    constexpr int kGroups = Slots<kP>::kGroups;
    __shared__ float s_red[kStageThreads / 64];
    // slot tau of token group blockIdx.x / kP (one group when kP < 16)
    const int tau = (int)blockIdx.x % kP;
    const int tok = (int)blockIdx.x;
    u32x4 *frag_out = a.frag_out + (size_t)(tok / kP) * a.group_words;
    const int H = a.H;
    const bool live = tok < a.M;
    const uint16_t *hrow = a.hidden + (size_t)(live ? tok : 0) * H;
    const int n_chunks = kWaves * kUnits * 8;              // 16-channel chunks in the padded row
    constexpr int kIter = (kWaves * kMaxUnitsPerWave * 8 + kStageThreads - 1) / kStageThreads;

    float xs[kIter][16];
    float am = 0.0f;
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
        const int c = threadIdx.x + kStageThreads * it;
        const bool ok = live && c < n_chunks && c * 16 < H;
        if (ok) {
            load_xs16(hrow, a.scales, c * 16, xs[it]);
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j)
                xs[it][j] = 0.0f;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j)
            am = fmaxf(am, fabsf(xs[it][j]));
    }
    am = wave_max(am);
    if ((threadIdx.x & 63) == 0)
        s_red[threadIdx.x >> 6] = am;
    __syncthreads();
    am = s_red[0];
#pragma unroll
    for (int w = 1; w < kStageThreads / 64; ++w)
        am = fmaxf(am, s_red[w]);
    const int e = code_exponent(am);
    if (threadIdx.x == 0)
        a.exps[tok] = e;

#pragma unroll
    for (int it = 0; it < kIter; ++it) {
        const int c = threadIdx.x + kStageThreads * it;
        if (c >= n_chunks)
            break;
        // chunk c = channels 16c..16c+15: unit u = c / 8, lane group grp =
        // (c % 8) / 2, K-step t = c % 2; unit u belongs to wave u / kUnits
        const int u = c / 8, grp = (c % 8) / 2, t = c % 2;
        const int wave = u / kUnits, i = u % kUnits;
        uint32_t limbw[3][4];
        split_limbs(xs[it], e, limbw);
        for (int n16 = tau; n16 < 16; n16 += kP) {
#pragma unroll
            for (int g = 0; g < kGroups; ++g) {
                const int limb = (16 * g + n16) / kP;
                u32x4 word = {0u, 0u, 0u, 0u};
                if (limb < 3)
                    word = u32x4{limbw[limb][0], limbw[limb][1], limbw[limb][2], limbw[limb][3]};
                frag_out[frag_index<kP, kUnits>(wave, i, t, g, grp * 16 + n16)] = word;
            }
        }
    }
}

// ---------------------------------------------------------------- verify_kernel
template <int kP, int kUnits, int kRing, bool kLogits, int kTopK, bool kLse, bool kFused,
          int kAux = INT4VH_WEIGHT_AUX>
__global__ void __launch_bounds__(kThreads)
verify_kernel(Args a)
{
    static_assert(kTopK == 0 || (kTopK <= kMaxTopK && !kLogits), "sampled epilogue");
    static_assert(!kLse || kTopK > 0, "the log-sum-exp belongs to the sampled epilogue");
    static_assert(!kFused || (kP == 5 && kTopK == 0), "fused staging: one MFMA row group, greedy");
    constexpr int kGroups = Slots<kP>::kGroups;
    constexpr int kTileBytes = kUnits * kWaves * 1024;     // LDS image of one tile (max H)
    // All LDS lives in one object: the weight ring, then the per-wave
    // partial sums (exact integers held in binary64, per D row and column,
    // two buffers).  The final merge reuses the ring once it is dead.
    struct Merge {
        float fv[kWaves][kMaxRows];
        int fi[kWaves][kMaxRows];
        int draft[kMaxGroups * kMaxRows];
        int accept[kMaxGroups * kMaxRows];
        int last;
        int arg_g[kMaxGroups * kMaxRows];     // several token groups: ids of every row
        int draft_g[kMaxGroups * kMaxRows];   // and the drafts of every request
    };
    // Sampled epilogue: a per-token buffer of candidate keys, sorted into the
    // top-k list 16 at a time -- where the LDS budget leaves room for it
    // (otherwise candidates are inserted into the list directly).
    constexpr bool kCBuf = kTopK > 0 && (size_t)kRing * kTileBytes + 2 * kWaves * kTileRows * kTileRows * 8 +
                                                (size_t)kWaves * 2 * 16 * 8 <= 160 * 1024;
    struct Lds {
        uint8_t ring[kRing][kTileBytes];
        unsigned long long part[2][kWaves][kTileRows][kTileRows];
        unsigned long long cbuf[kCBuf ? kWaves : 0][2][16];   // [wave][token 2w / 2w+1][slot]
    };
    static_assert(sizeof(Merge) <= sizeof(uint8_t[kRing][kTileBytes]), "merge area");
    static_assert(sizeof(Lds) <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) Lds lds;
    auto &s_ring = lds.ring;
    auto &s_part = lds.part;
    Merge &mg = *reinterpret_cast<Merge *>(&lds.ring[0][0]);
    auto &s_fv = mg.fv;
    auto &s_fi = mg.fi;
    auto &s_draft = mg.draft;
    auto &s_accept = mg.accept;
    auto &s_last = mg.last;

    const int lane = threadIdx.x & 63;
    const int wave = wave_uniform((int)threadIdx.x >> 6);   // in an SGPR: scalar address math
    const int n16 = lane & 15;   // MFMA row of A / column of B and D
    const int grp = lane >> 4;   // 16-lane group: K sub-block, D rows 4*grp..4*grp+3
    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int M = a.M, V = a.V, H = a.H;
    // Token groups (more than 16 rows): one workgroup of each group per tile
    // set, all walking the same tiles.  With whole sets of 8 workgroups the
    // members of a set are 8 blockIdx apart, so they run on one XCD (blockIdx
    // b runs on XCD b % 8) at the same time and a tile comes from HBM once,
    // then from that XCD's L2.
    const int n_g = a.n_groups, n_sets = a.n_sets;
    const int tgrp = n_g == 1 ? 0 : (n_sets % 8 == 0 ? (b / 8) % n_g : b / n_sets);
    const int tset = n_g == 1 ? b : (n_sets % 8 == 0 ? (b % 8) + 8 * (b / (8 * n_g)) : b % n_sets);
    const int Mg = n_g == 1 ? M : min(kMaxRows, M - kMaxRows * tgrp);   // rows of this group
    const int pstride = n_g == 1 ? M : kMaxRows;                        // winners per workgroup
    const int n_my = (a.n_tiles - tset + n_sets - 1) / n_sets;
    const int chunks_per_row = H / 32;                     // 16-byte chunks per weight row

    // ---------------- weight stream into the LDS ring
    // Wave w copies 1 KB blocks jj = w*kUnits + m of the tile (m < kUnits);
    // lane l of a block fetches chunk l ^ (jj & 7) so that LDS holds the
    // tile image with chunk c of block jj at position c ^ (jj & 7).  Blocks
    // past the tile and bytes past the head are clamped (their values are
    // never used: zero activation codes or masked rows), which keeps every
    // wave's number of copies per tile fixed.
    const unsigned long long w_last = a.w_bytes - 16;
    const unsigned long long tile_bytes = (unsigned long long)kTileRows * (H / 2);
    const unsigned long long span_bytes = (unsigned long long)a.n_units * 1024;   // bytes a tile's copies touch
    unsigned int loff[kUnits];                               // lane offsets within a tile, per block
#pragma unroll
    for (int m = 0; m < kUnits; ++m) {
        const int jj = min(wave * kUnits + m, a.n_units - 1);
        loff[m] = (unsigned int)(jj * 1024 + (lane ^ (jj & 7)) * 16);
    }
    // The first kRing tiles go out without the branch (clamped addresses
    // throughout): the compiler then counts the copies in flight exactly and
    // does not wait for all of them before the first use of the fragments.
    auto issue_tile = [&](int k, bool branch_free = false) {
        const int tile = tset + k * n_sets;
        const unsigned long long base = (unsigned long long)tile * tile_bytes;
        uint8_t *dst = s_ring[k % kRing];
        if (!branch_free && base + span_bytes <= a.w_bytes) {   // all of the tile's copies inside the head
            const uint8_t *src = a.w + base;
#pragma unroll
            for (int m = 0; m < kUnits; ++m) {
                const int jj = min(wave * kUnits + m, a.n_units - 1);
                copy_to_lds16<kAux>(src + loff[m], dst + jj * 1024);
            }
        } else {
#pragma unroll
            for (int m = 0; m < kUnits; ++m) {
                const int jj = min(wave * kUnits + m, a.n_units - 1);
                const unsigned long long off = base + loff[m];
                copy_to_lds16<kAux>(a.w + (off < w_last ? off : w_last), dst + jj * 1024);
            }
        }
    };
    // ---------------- activation fragments and step exponents
    const int rtok = 2 * wave + ((lane >> 4) & 1);         // token (of the group) reduced by this lane
    const bool rlane = lane < 32 && rtok < Mg;
    i32x4 afr[kUnits][2][kGroups];
    int rexp;
    // sampled epilogue: the draft id of the lane's token (loaded ahead of the
    // weight copies, like every other register the main loop reads)
    int my_draft = -1;
    const int grow = kMaxRows * tgrp + rtok;                 // the lane's row of the call
    if (kTopK > 0 && rlane && a.T > 1 && (grow % a.T) < a.T - 1)
        my_draft = a.draft[(grow / a.T) * (a.T - 1) + grow % a.T];
    if constexpr (!kFused) {
        // Tile 0's copies go out first, so that HBM starts streaming while
        // the fragments (245 KB per workgroup at 16 rows, from L2) pass the
        // CU's in-order memory pipeline; the next prologue tiles follow them,
        // so that waiting for tile 0 at the first step also covers the
        // fragments.  (Issuing every prologue tile first delays the fragments
        // by a second tile and measured slower.)
        issue_tile(0, true);
        // fragments from stage_kernel, in the workspace
#pragma unroll
        for (int i = 0; i < kUnits; ++i)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int g = 0; g < kGroups; ++g)
                    afr[i][t][g] = __builtin_bit_cast(
                        i32x4, a.frag[(size_t)tgrp * a.group_words + frag_index<kP, kUnits>(wave, i, t, g, lane)]);
        // the other prologue tiles, unconditional like the first step's (a
        // tile past the head reads clamped bytes into a ring slot that is
        // never used; every copy has landed before the workgroup publishes)
#pragma unroll
        for (int k = 1; k < kRing - 1; ++k)
            issue_tile(k, true);
        // the step exponents of the wave's two tokens, by a scalar load once
        // the copies are out (a vector load would make the compiler wait for
        // every copy in flight where it is first used); lanes of tokens >= M
        // never use theirs
        rexp = load_exp_pair(a.exps + kMaxRows * tgrp + 2 * wave, (lane >> 4) & 1) - 4;   // weights carry a factor 16
    } else {
        // Staging done here for M <= 2 rows.  The scale row and the hidden
        // rows are copied into the last ring slot (unused until the main loop
        // refills it) with the same LDS copies as the weights, ahead of the
        // weight prologue, so one count of outstanding copies covers both.
        // While the weights stream, the workgroup turns the rows into codes
        // (each wave its slice of the hidden dimension, same arithmetic as
        // stage_kernel) in the partial-sum area of LDS (free until the main
        // loop), and every lane reads its A fragments from there.
        constexpr int kSliceCh = kUnits * kUnitH;           // channels of a wave's slice
        constexpr int kHPad = kWaves * kSliceCh;              // padded hidden dimension
        constexpr int kRowBlocks = kHPad * 2 / 1024;          // 1 KB blocks of one padded fp16 row
        static_assert(3 * kHPad * 2 <= kTileBytes, "scale and hidden rows fit one ring slot");
        uint8_t *rows = s_ring[kRing - 1];                    // [scales | hidden 0 | hidden 1], kHPad each
        uint8_t *codes = reinterpret_cast<uint8_t *>(&s_part[0][0][0][0]);     // [3][M][kHPad]
        float *wmax = reinterpret_cast<float *>(codes + 3 * M * kHPad);      // [kWaves][2]
        {
            const unsigned long long row_bytes = (unsigned long long)H * 2;
            for (int q = wave; q < (M + 1) * kRowBlocks; q += kWaves) {
                const int arr = q / kRowBlocks;               // 0: scales, 1 + m: hidden row m
                const unsigned long long off = (unsigned long long)(q % kRowBlocks) * 1024 + lane * 16;
                const uint16_t *src = arr == 0 ? a.scales : a.hidden + (size_t)(arr - 1) * H;
                // bytes past the row: clamped, masked below
                copy_to_lds16<0>(reinterpret_cast<const uint8_t *>(src) + (off < row_bytes ? off : row_bytes - 16),
                                 rows + q * 1024);
            }
        }
        // the prologue tiles, unconditional (a tile past the head reads
        // clamped bytes into a ring slot that is never used), so that the
        // count below is exactly this wave's weight copies
#pragma unroll
        for (int k = 0; k < kRing - 1; ++k)
            issue_tile(k, true);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm((kRing - 1) * kUnits));
        barrier_no_fence();

        // Thread t takes the 4-channel chunks t, t + 512, ... of the padded
        // row (an even share per SIMD); channels past H give zero codes.
        constexpr int kChunks4 = kHPad / 4;
        constexpr int kR4 = (kChunks4 + kThreads - 1) / kThreads;
        float xs[2][kR4][4];
        float mx[2] = {0.0f, 0.0f};
#pragma unroll
        for (int r = 0; r < kR4; ++r) {
            const int c = (int)threadIdx.x + kThreads * r;
            const bool in_pad = c < kChunks4;
            const int ch = in_pad ? 4 * c : 0;
            uint2 sx, hxm[2];
            lds_load3_u64(rows + 2 * ch, rows + 2 * (kHPad + ch), rows + 2 * ((M > 1 ? 2 : 1) * kHPad + ch), sx,
                          hxm[0], hxm[1]);
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const bool ok = m < M && in_pad && 4 * c < H;
                const uint2 hx = hxm[m];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t hw = j < 2 ? hx.x : hx.y, sw = j < 2 ? sx.x : sx.y;
                    const uint32_t hb = (j & 1) ? (hw >> 16) : (hw & 0xFFFF);
                    const uint32_t sb = (j & 1) ? (sw >> 16) : (sw & 0xFFFF);
                    xs[m][r][j] = ok ? half_bits_to_float(hb) * half_bits_to_float(sb) : 0.0f;
                    mx[m] = fmaxf(mx[m], fabsf(xs[m][r][j]));
                }
            }
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            mx[m] = wave_max(mx[m]);
            if (lane == 0)
                lds_store_u32(&wmax[2 * wave + m], __float_as_uint(mx[m]));
        }
        // (no fence: the weight copies stay in flight)
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        barrier_no_fence();
        int e[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            float am = wmax[m];
#pragma unroll
            for (int w = 1; w < kWaves; ++w)
                am = fmaxf(am, wmax[2 * w + m]);
            e[m] = code_exponent(am);
        }
        // Codes, as three signed bytes each, stored per (limb, token) row of
        // the padded hidden dimension.  |code| <= kCodeMax = 0x7F7F7F, so
        // code + 0x808080 lies in [0, 2^24) and its bytes are the limbs
        // (low first) offset by 128: byte i of the biased value, xor 0x80, is
        // the signed limb of weight 2^(8i) -- the same split as stage_kernel.
        // Four codes' bytes of one limb are gathered with byte permutes.
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < kR4; ++r) {
                const int c = (int)threadIdx.x + kThreads * r;
                if (m < M && c < kChunks4) {
                    uint32_t u[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        u[j] = (uint32_t)((int)rintf(ldexpf(xs[m][r][j], -e[m])) + 0x808080);
#pragma unroll
                    for (int l = 0; l < 3; ++l) {            // limb l: 0 = high (byte 2) ... 2 = low (byte 0)
                        const uint32_t bi = 2 - l;
                        const uint32_t sel = ((4 + bi) << 8) | bi;
                        const uint32_t p01 = __builtin_amdgcn_perm(u[1], u[0], sel);
                        const uint32_t p23 = __builtin_amdgcn_perm(u[3], u[2], sel);
                        lds_store_u32(codes + (size_t)(l * M + m) * kHPad + 4 * c,
                                      __builtin_amdgcn_perm(p23, p01, 0x05040100u) ^ 0x80808080u);
                    }
                }
            }
        // (no fence: the weight copies stay in flight)
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        barrier_no_fence();
        // A fragment of slot n16 = (limb n16 / 5, token n16 % 5): 16 channels
        // in the register order of the weight dequantisation (register v, byte
        // b <- channel 8*(v>>1) + 2*b + (v&1))
        const int slot_tok = n16 % 5, slot_limb = n16 / 5;
        const bool slot_live = slot_tok < M && slot_limb < 3;
        const uint8_t *slot_codes = codes + (size_t)(slot_live ? slot_limb * M + slot_tok : 0) * kHPad;
#pragma unroll
        for (int i = 0; i < kUnits; ++i)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int ch0 = (wave * kUnits + i) * kUnitH + 32 * grp + 16 * t;
                const u32x4 d = *reinterpret_cast<const u32x4 *>(slot_codes + ch0);
                const i32x4 f = {(int32_t)__builtin_amdgcn_perm(d[1], d[0], 0x06040200u),
                                 (int32_t)__builtin_amdgcn_perm(d[1], d[0], 0x07050301u),
                                 (int32_t)__builtin_amdgcn_perm(d[3], d[2], 0x06040200u),
                                 (int32_t)__builtin_amdgcn_perm(d[3], d[2], 0x07050301u)};
                afr[i][t][0] = slot_live ? f : i32x4{0, 0, 0, 0};
            }
        rexp = e[rtok < M ? rtok : 0] - 4;
    }

    // LDS byte offsets of this lane's B fragments (swizzled), per unit
    int boff[kUnits];
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
        const int gc = n16 * chunks_per_row + (wave * kUnits + i) * 4 + grp;
        const int jj = gc >> 6;
        boff[i] = (jj * 64 + ((gc & 63) ^ (jj & 7))) * 16;
    }
    // limb weight (2^16, 2^8, 1; 0 for rows past the three limbs) of each
    // group's D rows this lane receives
    double limb_w[kGroups][4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        const int row = grp * 4 + r4;
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
            const int l = kP == 16 ? g : (16 * g + row) / kP;   // row < 16: group g is limb g
            limb_w[g][r4] = l < 3 ? (double)(1 << (8 * (2 - l))) : 0.0;
        }
    }

    float bv = -__builtin_huge_valf();
    int bi = 0x7FFFFFFF;
    // sampled epilogue: the token's distributed top-k list (lanes 0-15: token
    // 2*wave, lanes 16-31: token 2*wave+1; rank = n16) and the lane's running
    // (max, sum) of exp2(logit * log2(e) / tau)
    unsigned long long dl = 0ull;
    float lm = -__builtin_huge_valf(), ls = 0.0f;
    const float zscale = 1.4426950408889634f / a.tau;
    int cnt0 = 0, cnt1 = 0;             // buffered candidates of the wave's two tokens (wave-uniform)
    // A flush of the buffered candidates into the lists is a chain of
    // dependent cross-lane steps that holds the whole workgroup at the next
    // barrier, so it is split over two tiles: the buffer is sorted on one
    // tile and merged into the lists at the start of the next.  Until then
    // the bar a key must pass is the older, lower one: a superset of the
    // candidates, so the lists stay exact.  (pend is wave-uniform.)
    unsigned long long srt_pend = 0ull;
    bool pend = false;
    auto merge_pending = [&]() {
        if constexpr (kCBuf) {
            if (pend) {
                dl = dlist_merge(dl, key_dpp<0x140>(srt_pend), lane);      // row_mirror: rank 15-j
                pend = false;
            }
        }
    };
    // sort the buffered candidates of both tokens (all lanes); the merge
    // follows on the next tile
    auto flush_cand = [&]() {
        if constexpr (kCBuf) {
            merge_pending();
            const int cnt = lane < 16 ? cnt0 : cnt1;
            const unsigned long long v = (lane < 32 && n16 < cnt) ? lds.cbuf[wave][(lane >> 4) & 1][n16] : 0ull;
            srt_pend = row_sort16(v, n16);
            pend = true;
            cnt0 = 0;
            cnt1 = 0;
        }
    };
    // Rows of D that hold limbs of token t are t, t + kP, t + 2*kP (those
    // with a limb index below 3).  Every lane loads (clamped to a valid
    // token) so the loads are straight-line and all in flight together.
    constexpr int kRowsPerTok = (16 + kP - 1) / kP < 3 ? (16 + kP - 1) / kP : 3;
    const int rt = rlane ? rtok : 0;
    // In token groups the lanes of a partial group's missing rows take the
    // epilogue's steps as well (on token 0's sums and the step exponent
    // staged for an empty row; nothing of theirs is published).  Every
    // group's workgroups then spend the same time per tile and stay in step:
    // a partial group that runs ahead drifts out of the window of tiles the
    // XCD's L2 still holds, and the full groups fetch those tiles again.
    const bool rwork = lane < 32 && (rtok < Mg || n_g > 1);
    auto reduce_tile = [&](int k) {
        const int buf = k & 1;
        double code = 0.0;                 // integer-valued, |code| < 2^47: exact
#pragma unroll
        for (int j = 0; j < kRowsPerTok; ++j)
#pragma unroll
            for (int w = 0; w < kWaves; ++w)
                code += __longlong_as_double((long long)s_part[buf][w][rt + kP * j][n16]);
        unsigned long long key = 0ull;
        if (rwork) {
            const int v = (tset + k * n_sets) * kTileRows + n16;
            const float val = (float)ldexp(code, rexp);   // the one rounding
            if (v < V) {
                if constexpr (kTopK == 0) {       // (the sampled epilogue's winner is its list's rank 0)
                    if (better(val, v, bv, bi)) {
                        bv = val;
                        bi = v;
                    }
                }
                if constexpr (kTopK > 0) {
                    key = order_key(val, v);
                    if constexpr (kLse)
                        lse_add(lm, ls, val * zscale);      // one exp2 per logit
                    if (kLse && v == my_draft) {      // one lane of one workgroup per token
                        __hip_atomic_store(&a.draft_logit[grow], val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        __hip_atomic_store(&a.draft_seen[grow], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
                if (kLogits && rlane)
                    a.logits_out[(size_t)(kMaxRows * tgrp + rtok) * V + v] = val;
            }
        }
        if (kCBuf && k == 0) {
            // the first tile: the lists are empty, so its 16 keys per token,
            // sorted, are the lists (wave-uniform control flow)
            dl = row_sort16(key, n16);
        } else if constexpr (kCBuf) {
            merge_pending();                       // the previous tile's sorted flush, if any
            // the tile's keys that beat the list's last kept rank go to the
            // token's candidate buffer; a full buffer is sorted first (and
            // merged on the next tile) (wave-uniform control flow)
            const unsigned long long th0 = key_readlane(dl, kTopK - 1);
            const unsigned long long th1 = key_readlane(dl, 16 + kTopK - 1);
            const bool is_cand = key > (lane < 16 ? th0 : th1);
            const unsigned long long cand = __ballot(is_cand);
            const uint32_t m0 = (uint32_t)cand & 0xFFFFu, m1 = (uint32_t)(cand >> 16) & 0xFFFFu;
            const int n0 = __builtin_popcount(m0), n1 = __builtin_popcount(m1);
            if (cnt0 + n0 > 16 || cnt1 + n1 > 16)
                flush_cand();
            if (is_cand) {
                const uint32_t mrow = lane < 16 ? m0 : m1;
                const int slot = (lane < 16 ? cnt0 : cnt1) + __builtin_popcount(mrow & ((1u << n16) - 1u));
                lds.cbuf[wave][(lane >> 4) & 1][slot] = key;
            }
            cnt0 += n0;
            cnt1 += n1;
        } else if constexpr (kTopK > 0) {
            // insert the tile's keys that beat the list's last kept rank: a
            // sort and one merge when a group has more than two, else one per
            // group and iteration (wave-uniform control flow, all lanes active)
            const unsigned long long th0 = key_readlane(dl, kTopK - 1);
            const unsigned long long th1 = key_readlane(dl, 16 + kTopK - 1);
            const bool is_cand = key > (lane < 16 ? th0 : th1);
            unsigned long long cand = __ballot(is_cand);
            if (__builtin_popcount((uint32_t)cand & 0xFFFFu) > 2 ||
                __builtin_popcount((uint32_t)(cand >> 16) & 0xFFFFu) > 2) {
                // many: sort the tile's candidates and merge them in at once
                const unsigned long long srt = row_sort16(is_cand ? key : 0ull, n16);
                dl = dlist_merge(dl, key_dpp<0x140>(srt), lane);      // row_mirror: rank 15-j
                cand = 0ull;
            }
            while (cand) {
                const uint32_t m0 = (uint32_t)cand & 0xFFFFu;
                const uint32_t m1 = (uint32_t)(cand >> 16) & 0xFFFFu;
                const unsigned long long k0 = key_readlane(key, m0 ? __builtin_ctz(m0) : 0);
                const unsigned long long k1 = key_readlane(key, m1 ? 16 + __builtin_ctz(m1) : 16);
                const bool in0 = lane < 16, in1 = lane >= 16 && lane < 32;
                const unsigned long long kk = in0 ? k0 : k1;
                const unsigned long long nd = dlist_insert(dl, kk);
                dl = ((in0 && m0) || (in1 && m1)) ? nd : dl;
                cand &= ~((unsigned long long)(m0 & (0u - m0)) | ((unsigned long long)(m1 & (0u - m1)) << 16));
            }
        }
    };

    // ---------------- main loop over this workgroup's tiles
    // One step per tile.  The first step runs ahead of the loop: the
    // compiler waits for every copy in flight at the entry of a loop that
    // uses registers loaded before it (the activation fragments), which would
    // hold tile 0 until tile 1 has landed and tile 2 back until then; peeled,
    // the step's own count of copies in flight covers the fragments.
    auto step = [&](int k) {
        // this wave's copies of tile k are done (later tiles may be in flight);
        // after the barrier every wave's copies are, and tile k-1's partial
        // sums are complete in s_part
        // copies issued after tile k's: min(kRing - 2, n_my - 1 - k) tiles,
        // kRing - 2 at the first step (the prologue is unconditional; the
        // fragment loads, issued between tile 0's copies and tile 1's, are
        // done once tile 0's are)
        static_assert(kRing >= 2 && kRing <= 4, "ring depth");
        const int later = k == 0 ? kRing - 2 : min(kRing - 2, n_my - 1 - k);
        if (later >= 2)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kUnits));
        else if (later == 1)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(kUnits));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        barrier_no_fence();
        if (k == 0)                                // (straight-line first step)
            issue_tile(kRing - 1, true);
        else if (k + kRing - 1 < n_my)
            issue_tile(k + kRing - 1);

        const uint8_t *tile = s_ring[k % kRing];
        u32x4 q[kUnits];
#pragma unroll
        for (int i = 0; i < kUnits; ++i)
            q[i] = *reinterpret_cast<const u32x4 *>(tile + boff[i]);
        i32x4 acc[kGroups];
#pragma unroll
        for (int g = 0; g < kGroups; ++g)
            acc[g] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < kUnits; ++i) {
            // nibble -> high half of a byte: the int8 value is 16*q
            const i32x4 b0 = {(int32_t)((q[i][0] << 4) & 0xF0F0F0F0u), (int32_t)(q[i][0] & 0xF0F0F0F0u),
                              (int32_t)((q[i][1] << 4) & 0xF0F0F0F0u), (int32_t)(q[i][1] & 0xF0F0F0F0u)};
            const i32x4 b1 = {(int32_t)((q[i][2] << 4) & 0xF0F0F0F0u), (int32_t)(q[i][2] & 0xF0F0F0F0u),
                              (int32_t)((q[i][3] << 4) & 0xF0F0F0F0u), (int32_t)(q[i][3] & 0xF0F0F0F0u)};
#pragma unroll
            for (int g = 0; g < kGroups; ++g)
                acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(afr[i][0][g], b0, acc[g], 0, 0, 0);
#pragma unroll
            for (int g = 0; g < kGroups; ++g)
                acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(afr[i][1][g], b1, acc[g], 0, 0, 0);
        }

        if (k > 0)
            reduce_tile(k - 1);

        // this wave's partial codes, limbs combined, one per D row: binary64
        // holds them exactly (|value| < 2^44), and the combination is three
        // conversions and two fused multiply-adds instead of 64-bit shifts
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            double val = (double)acc[0][r4] * limb_w[0][r4];
#pragma unroll
            for (int g = 1; g < kGroups; ++g)
                val = __builtin_fma((double)acc[g][r4], limb_w[g][r4], val);
            // rows of tokens >= M hold zero activation codes, so val is 0
            lds_store_u64(&s_part[k & 1][wave][grp * 4 + r4][n16], (unsigned long long)__double_as_longlong(val));
        }
    };
    step(0);
    for (int k = 1; k < n_my; ++k)
        step(k);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    barrier_no_fence();
    reduce_tile(n_my - 1);
    if (cnt0 + cnt1 > 0)
        flush_cand();
    merge_pending();

    // ---------------- per-workgroup best per token
    if constexpr (kTopK == 0)
        row_best16(bv, bi);
    if constexpr (kTopK > 0) {
        // lane n16 = j publishes the rank-j key of the workgroup's list;
        // the 16 lanes' (max, sum) pairs combine (fixed rotations) and lane
        // 0 of the token publishes them.  Slots are ordered by (token group,
        // tile set), so each merge group's lists are contiguous.
        const size_t pslot = (size_t)tgrp * n_sets + tset;
        if (rlane && n16 < kTopK)
            __hip_atomic_store(&a.part_topk[(pslot * pstride + rtok) * kTopK + n16], dl,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (kLse) {
            row_lse16(lm, ls);
            if (rlane && n16 == 0)
                __hip_atomic_store(&a.part_lse[pslot * pstride + rtok], lse_pack(lm, ls), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // Publication without device-scope fences: a fence here writes back and
    // invalidates the whole L2 of the XCD, which costs tens of microseconds
    // when every workgroup does it.  The winners and the ticket are
    // agent-scope atomics, which are coherent across XCDs by themselves; each
    // wave waits until its store is acknowledged before the barrier, so every
    // store has landed before the ticket is incremented, and the last
    // workgroup reads them with agent-scope atomic loads.
    if (kTopK == 0 && rlane && n16 == 0)           // (the sampled epilogue's winners are in its lists)
        __hip_atomic_store(&a.part[(size_t)b * pstride + rtok], pack_pair(bv, bi), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    if constexpr (kTopK == 0) {
        // With 8 or more tiles per workgroup the workgroups finish spread over
        // microseconds and one ticket does not queue: the last one takes a
        // single round trip.  Otherwise they finish together, and the last
        // workgroup of each group of 16 takes the top-level ticket.
        if (threadIdx.x == 0) {
            bool last;
            if (a.n_tiles >= 8 * n_sets) {
                last = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                       (uint32_t)(G - 1);
            } else {
                const int grp = b / kGroupWgs;
                const int gsz = min(kGroupWgs, G - kGroupWgs * grp);
                uint32_t *gt = a.group_ticket + (size_t)grp * kTicketStride;
                last = __hip_atomic_fetch_add(gt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                       (uint32_t)(gsz - 1);
                if (last) {
                    __hip_atomic_store(gt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    last = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                           (uint32_t)((G + kGroupWgs - 1) / kGroupWgs - 1);
                }
            }
            s_last = last;
        }
        __syncthreads();
        if (!s_last)
            return;
    } else {
        // Two levels, so that most of the merging overlaps the weight stream
        // of the workgroups still running: the last workgroup of each merge
        // group (up to 16 tile sets of one token group) merges the group's
        // lists into one, and the last merge group to finish runs the final
        // merge.
        const int n_mg = (n_sets + 15) / 16;          // merge groups per token group
        const int grp = tgrp * n_mg + tset / 16;
        const int gsz = min(16, n_sets - 16 * (tset / 16));
        const int n_grp = n_g * n_mg;
        if (threadIdx.x == 0) {
            const uint32_t prev = __hip_atomic_fetch_add(&a.group_ticket[(size_t)grp * kTicketStride], 1u,
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last = (prev == (uint32_t)(gsz - 1));
        }
        __syncthreads();
        if (!s_last)
            return;
        {
            const int m = 2 * wave + (lane >> 5);
            const size_t first = (size_t)tgrp * n_sets + 16 * (tset / 16);   // the group's first slot
            // the pairs' loads go out with the lists' (one round trip)
            const uint64_t lse_pr =
                kLse ? lse_load16(a.part_lse + first * pstride, gsz, pstride, m < Mg ? m : 0) : 0;
            const unsigned long long mine =
                merge_topk_lists<kTopK>(a.part_topk + first * pstride * kTopK, gsz, pstride, Mg, lane);
            if (m < Mg && ((lane >> 4) & 1) == 0 && n16 < kTopK)
                __hip_atomic_store(&a.group_topk[((size_t)grp * pstride + m) * kTopK + n16], mine,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if constexpr (kLse) {
                // lane n16 of the token's 16-lane group loads workgroup n16's
                // pair; fixed row rotations combine the 16
                float gm, gs;
                lse_combine16(lse_pr, gsz, gm, gs);
                if (m < Mg && (lane & 31) == 0)
                    __hip_atomic_store(&a.group_lse[(size_t)grp * pstride + m], lse_pack(gm, gs), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __syncthreads();
        if (threadIdx.x == 0) {
            __hip_atomic_store(&a.group_ticket[(size_t)grp * kTicketStride], 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t prev = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            s_last = (prev == (uint32_t)(n_grp - 1));
        }
        __syncthreads();
        if (!s_last)
            return;
    }

    // ---------------- last workgroup, several token groups (greedy only)
    // Four threads per row m: they load the winners of the n_sets workgroups
    // of group m / 16 (every load issued before any is used), reduce them,
    // and the rows' ids and the drafts go to LDS for the acceptance count.
    if (kTopK == 0 && n_g > 1) {
        constexpr int kPerThread = kMaxGrid / kMaxGroups / 4;    // winners per thread, at most
        const int m = (int)threadIdx.x >> 2, sub = (int)threadIdx.x & 3;
        const int mm = m < M ? m : M - 1;
        const int gm = mm / kMaxRows, l = mm % kMaxRows;
        float v0 = -__builtin_huge_valf();
        int i0 = 0x7FFFFFFF;
        uint64_t p[kPerThread];
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int js = sub + 4 * j;
            const int jj = js < n_sets ? js : n_sets - 1;   // repeats are harmless for a maximum
            const int bb = n_sets % 8 == 0 ? 8 * (n_g * (jj / 8) + gm) + jj % 8 : gm * n_sets + jj;
            p[j] = __hip_atomic_load(&a.part[(size_t)bb * kMaxRows + l], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const float pv = __uint_as_float((uint32_t)p[j]);
            const int pi = (int)(uint32_t)(p[j] >> 32);
            if (better(pv, pi, v0, i0)) {
                v0 = pv;
                i0 = pi;
            }
        }
#pragma unroll
        for (int off = 1; off <= 2; off <<= 1) {
            const float ov = __shfl_xor(v0, off);
            const int oi = __shfl_xor(i0, off);
            if (better(ov, oi, v0, i0)) {
                v0 = ov;
                i0 = oi;
            }
        }
        const int n_draft = a.R * (a.T - 1);
        if (sub == 0 && m < M) {
            const int id = a.vmap ? a.vmap[i0] : i0;    // row -> token id
            a.logits_max[m] = v0;
            a.argmax[m] = id;
            mg.arg_g[m] = id;
        }
        if ((int)threadIdx.x < n_draft)
            mg.draft_g[threadIdx.x] = a.draft[threadIdx.x];
        __syncthreads();
        for (int i = threadIdx.x; i < a.R; i += kThreads) {
            const int T = a.T;
            int n = 0;
            while (n < T - 1 && mg.arg_g[i * T + n] == mg.draft_g[i * (T - 1) + n])
                ++n;
            a.n_acc[i] = n;
        }
        if (threadIdx.x == 0)
            __hip_atomic_store(a.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }

    // ---------------- last workgroup: merge, write, accept, reset
    // One memory round trip: every load below is issued before any is used.
    // Thread (slot, m) takes the winners of workgroups slot, slot+32, ... for
    // token m (agent-scope loads: the lines may be stale in this XCD's L2);
    // the threads below R*(T-1) also fetch one draft id each.  (The sampled
    // epilogue takes its winners from the merged top-k lists instead.)
    {
        const int m = threadIdx.x & 15;
        const int slot = threadIdx.x >> 4;   // 0..31
        const int mm = m < M ? m : M - 1;    // rows past M repeat a real one (never written out)
        const int n_draft = a.R * (a.T - 1);
        const int dft = (int)threadIdx.x < n_draft ? a.draft[threadIdx.x] : 0;
        if constexpr (kTopK == 0) {
            float v0 = -__builtin_huge_valf();
            int i0 = 0x7FFFFFFF;
            constexpr int kPerThread = kMaxGrid / 32;
            constexpr int kBatch = 8;
#pragma unroll
            for (int j0 = 0; j0 < kPerThread; j0 += kBatch) {
                if (32 * j0 >= G)
                    break;
                uint64_t p[kBatch];
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    int bb = slot + 32 * (j0 + j);
                    bb = bb < G ? bb : G - 1;    // repeats are harmless for a maximum
                    p[j] = __hip_atomic_load(&a.part[(size_t)bb * M + mm], __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
                }
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    const float pv = __uint_as_float((uint32_t)p[j]);
                    const int pi = (int)(uint32_t)(p[j] >> 32);
                    if (better(pv, pi, v0, i0)) {
                        v0 = pv;
                        i0 = pi;
                    }
                }
            }
            // the four slots of this wave (lanes m, m+16, m+32, m+48)
#pragma unroll
            for (int off = 16; off <= 32; off <<= 1) {
                const float ov = __shfl_xor(v0, off);
                const int oi = __shfl_xor(i0, off);
                if (better(ov, oi, v0, i0)) {
                    v0 = ov;
                    i0 = oi;
                }
            }
            const int wv = threadIdx.x >> 6;
            if ((threadIdx.x & 63) < 16) {
                s_fv[wv][m] = v0;
                s_fi[wv][m] = i0;
            }
        }
        if ((int)threadIdx.x < n_draft)
            s_draft[threadIdx.x] = dft;
    }
    __syncthreads();
    if constexpr (kTopK == 0) {
        // wave 0 (all M <= 16 rows): thread m takes row m's winner, and the
        // acceptance of every request comes from one ballot of the
        // draft matches
        if (threadIdx.x < 64) {
            const int m = threadIdx.x;
            const int T = a.T;
            bool match = false;
            if (m < M) {
                float fv[kWaves];
                int fi[kWaves];
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    fv[w] = s_fv[w][m];
                    fi[w] = s_fi[w][m];
                }
                float v0 = fv[0];
                int i0 = fi[0];
#pragma unroll
                for (int w = 1; w < kWaves; ++w)
                    if (better(fv[w], fi[w], v0, i0)) {
                        v0 = fv[w];
                        i0 = fi[w];
                    }
                const int id = a.vmap ? a.vmap[i0] : i0;    // row -> token id
                a.logits_max[m] = v0;
                a.argmax[m] = id;
                const int req = m / T, t = m % T;
                match = t < T - 1 && id == s_draft[req * (T - 1) + t];
            }
            accept_from_ballot(__ballot(match), T, a.R, m, a.n_acc);
        }
    } else {
        // Sampled epilogue, final merge over the merge groups' lists, then
        // the token's target probability of its draft from the k logits
        // (top-k sampling at temperature tau): lane j of the token's first
        // 16-lane group holds rank j; sums are fixed rotations over the 16
        // lanes.  One pass per token group of 16 rows.
        const int n_mg = (n_sets + 15) / 16;          // merge groups per token group
        const int T = a.T;
        for (int tg = 0; tg < n_g; ++tg) {
            const int Mt = min(kMaxRows, M - kMaxRows * tg);           // rows of token group tg
            const int ml = 2 * wave + (lane >> 5);                     // row within the group
            const int slot = lane & 31;                                // 0..15: first 16 lanes of the row
            const int mml = ml < Mt ? ml : Mt - 1;
            const int m = kMaxRows * tg + ml, mm = kMaxRows * tg + mml;  // rows of the call
            const int req = mm / T, t = mm % T;
            const bool drafted = t < T - 1;
            const int di = drafted ? req * (T - 1) + t : 0;
            // every load of this pass is issued before the lists' (one round trip)
            const float u_d = drafted ? a.unif[di] : 1.0f, q_d = drafted ? a.dprob[di] : 1.0f;
            uint64_t lse_pr = 0;
            int seen_d = 0;
            float logit_d = 0.0f;
            if constexpr (kLse) {
                lse_pr = lse_load16(a.group_lse + (size_t)tg * n_mg * pstride, n_mg, pstride, mml);
                seen_d = __hip_atomic_load(&a.draft_seen[mm], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                logit_d = __hip_atomic_load(&a.draft_logit[mm], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            const unsigned long long mine = merge_topk_lists<kTopK>(
                a.group_topk + (size_t)tg * n_mg * pstride * kTopK, n_mg, pstride, Mt, lane);
            const int d = drafted ? s_draft[di] : -1;
            const float hv = key_value(mine);
            const int hi = key_index(mine);
            const bool live = ml < Mt;
            if (slot == 0 && live) {                      // rank 0: the greedy winner
                a.logits_max[m] = hv;
                a.argmax[m] = a.vmap ? a.vmap[hi] : hi;
            }
            const float lmax = key_value(key_shfl(mine, lane & ~15));
            const float e = n16 < a.top_k ? expf((hv - lmax) / a.tau) : 0.0f;
            float sum = e, e_d = (n16 < a.top_k && hi == d) ? e : 0.0f;
            sum = row_sum16(sum);
            e_d = row_sum16(e_d);
            if (slot < a.top_k && live) {
                a.topk_ids[m * a.top_k + slot] = hi;
                a.topk_logits[m * a.top_k + slot] = hv;
            }
            // log sum exp(logit / tau) over the whole vocabulary, from the
            // merge groups' pairs (lane-parallel loads, fixed row rotations)
            float lse = 0.0f;
            if constexpr (kLse) {
                float gm, gs;
                lse_combine16(lse_pr, n_mg, gm, gs);
                lse = (gm + __log2f(gs)) * 0.6931471805599453f;
            }
            if (slot == 0 && live) {
                if (kLse && a.lse_out)
                    a.lse_out[m] = lse;
                int ok = 0;
                if (drafted) {
                    float p;
                    if (!kLse || a.top_k > 0)
                        p = e_d / sum;
                    else
                        p = seen_d != 0 ? expf(logit_d / a.tau - lse) : 0.0f;
                    a.p_draft[di] = p;
                    ok = u_d * q_d < p;
                }
                s_accept[m] = ok;
                if constexpr (kLse)
                    __hip_atomic_store(&a.draft_seen[m], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __syncthreads();
        if (threadIdx.x < 64)
            accept_from_ballot(__ballot((int)threadIdx.x < M && s_accept[threadIdx.x] != 0), T, a.R,
                               (int)threadIdx.x, a.n_acc);
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(a.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ================================================================ batch path
//
// Blocks of more than 64 rows (up to 4096: many requests sharing one head).
// The contraction is then a GEMM of (token, limb) rows against the head,
// 3M x H times H x V, on the same int8 MFMA and with the same numerics as the
// single-block kernels (identical codes, exact integer sums, one
// rounding), so a row's results do not depend on the path or the batch it ran
// in.  The step count grows with M: at M = 256 the 16x16x64 int8 MFMAs, not
// the weight stream, bound the call.
//
//  stage_rows_kernel  codes and step exponents of all rows, written as MFMA
//      A-operand fragments: for each 16-token block, K step of 128 channels,
//      half (64 channels) and limb, 64 lanes x 16 bytes contiguous.
//
//  verify_rows_kernel  work item = 128 tokens x 128 vocabulary rows over the
//      whole hidden dimension; workgroups (one per CU) take items
//      round-robin.  Each of the 8 waves (two per SIMD) owns one 16-token
//      block (three limb row blocks) and all 128 rows (8 column blocks): 24
//      int32 accumulator tiles.  The packed weights of a K step (128 rows x
//      64 bytes) are loaded once per workgroup, one 16-byte chunk per thread,
//      turned into int8 B fragments by the thread that loaded them and
//      written to LDS (16 KB, double-buffered), where every wave reads them:
//      the nibble conversion happens once per workgroup, not once per wave.
//      The activation fragments, private to a wave, go from memory (L2:
//      every workgroup reads them) straight to registers.  Steps of
//      consecutive items form one stream, prefetched two steps ahead.  At the
//      end of an item each wave turns its accumulators into logits, reduces
//      them per token and merges the winner into a per-token 64-bit key with
//      an atomic maximum (value order in the high word, inverted index in the
//      low word, so the larger value and then the lower index wins).  The
//      last workgroup decodes the keys, counts accepted drafts and clears the
//      keys for the next call.
//
// Alternatives that measured slower on MI355X: four waves of 32 tokens (one
// per SIMD: LDS and memory latency exposed with no second wave to cover
// it), per-wave nibble conversion from a packed LDS tile (the VALU work
// equals the MFMA issue time), a four-deep register ring (no gain: the stalls
// are not latency), and activation re-loads interleaved between MFMAs (a
// load into a register that in-flight MFMAs still read stalls the wave).

constexpr int kRWaves = 8;                              // waves per workgroup
constexpr int kRThreads = 64 * kRWaves;
constexpr int kRTbPerWave = 8 / kRWaves;                // 16-token blocks per wave (128-token kernel)
constexpr int kRTbPerTile = kRTbPerWave * kRWaves;      // 16-token blocks per work item (128-token kernel)
constexpr int kRTokTile = 16 * kRTbPerTile;             // tokens per work item (128-token kernel)
constexpr int kRVocTile = 128;                          // vocabulary rows per work item
constexpr int kRVBlocks = kRVocTile / 16;               // MFMA column blocks per wave
constexpr int kRStepH = 128;                            // hidden channels per K step
constexpr int kRStepBytes = kRVocTile * kRStepH / 2;    // packed weight bytes of one K step
constexpr int kRTileBytes = kRVocTile * kRStepH;        // the same weights as int8 MFMA fragments
constexpr int kRStageSteps = 8;                         // K steps per stage workgroup
constexpr int kRStageThreads = kRStageSteps * 2 * 64;   // one (step, half, lane) per thread
static_assert(kRStageThreads % (16 * 64) == 0, "whole waves per token in the exponent pass");
constexpr int kRChunks = kRStepBytes / (kRThreads * 16);   // 16-byte weight chunks per thread and step
static_assert(kRChunks * kRWaves == kRVBlocks, "each wave stages whole column blocks");

struct RArgs {
    const uint16_t *hidden;   // [M, H] binary16
    const uint8_t *w;         // [V, H/2]
    const uint16_t *scales;   // [H]
    const int32_t *draft;     // [R, T-1] or null
    float *logits_max;        // [M]
    int32_t *argmax;          // [M]
    int32_t *n_acc;           // [R]
    float *logits_out;        // [M, V] or null
    unsigned long long *item_keys;   // [M, ceil(V / 128)] each row's best key per vocabulary tile, or null
    const int32_t *vmap;      // [V] token id of each head row, or null (identity)
    unsigned long long *keys; // [M] per-token winner keys, zero between calls
    uint32_t *ticket;
    uint32_t *group_ticket;   // [64][kTicketStride] per-group tickets (word 0), zero between calls
    int32_t *exps;            // [n_mt * token tile] step exponents
    const u32x4 *frag;        // activation fragments
    u32x4 *frag_out;
    int R, T, M, V, H;
    int n_steps;              // K steps of 128 channels, rounded up to even
    int n_tb;                 // 16-token blocks that hold real rows: ceil(M / 16)
    int n_mt;                 // token tiles of 32, 64 or 128 tokens: ceil(M / tile)
    int n_items;              // n_mt * ceil(V / 128)
    unsigned long long w_bytes;
};

// Index (in 16-byte words) of a fragment: token block tb, K step s, half h,
// limb l, lane.
__device__ __forceinline__ size_t rfrag_index(int tb, int n_steps, int s, int h, int l, int lane)
{
    return ((((size_t)tb * n_steps + s) * 2 + h) * 3 + l) * 64 + lane;
}

// ---------------------------------------------------------------- stage_rows_kernel
// Grid (token blocks of the padded tiles, groups of kRStageSteps K steps).
// Every workgroup finds the step exponents of its 16 tokens (the largest
// |x*s| over the whole row: 64 threads per token, all of a thread's loads in
// flight at once), then writes the fragments of its K steps, one
// (step, half, lane) word triple per thread.  Tokens >= M and channels >= H
// get zero codes.
__global__ void __launch_bounds__(kRStageThreads) stage_rows_kernel(RArgs a)
{
    __shared__ float s_am[16][kRStageThreads / 16 / 64];
    __shared__ int s_e[16];
    const int tb = blockIdx.x;
    const int tid = threadIdx.x;
    const int H = a.H;
    {
        constexpr int kPerTok = kRStageThreads / 16;           // threads per token
        constexpr int kChunks = (INT4VH_MAX_H / 16 + kPerTok - 1) / kPerTok;
        const int n = tid / kPerTok, sub = tid % kPerTok;
        const int tok = tb * 16 + n;
        const uint16_t *hrow = a.hidden + (size_t)(tok < a.M ? tok : 0) * H;
        float xs[kChunks][16];
#pragma unroll
        for (int j = 0; j < kChunks; ++j) {
            const int c = sub + kPerTok * j;
            if (tok < a.M && c * 16 < H) {
                load_xs16(hrow, a.scales, c * 16, xs[j]);
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    xs[j][i] = 0.0f;
            }
        }
        float am = 0.0f;
#pragma unroll
        for (int j = 0; j < kChunks; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                am = fmaxf(am, fabsf(xs[j][i]));
        am = wave_max(am);
        if ((tid & 63) == 0)
            s_am[n][sub / 64] = am;
        __syncthreads();
        if (tid < 16) {
            float m = s_am[tid][0];
#pragma unroll
            for (int w = 1; w < kPerTok / 64; ++w)
                m = fmaxf(m, s_am[tid][w]);
            const int e = code_exponent(m);
            s_e[tid] = e;
            if (blockIdx.y == 0)
                a.exps[tb * 16 + tid] = e;
        }
    }
    __syncthreads();
    const int L = tid & 63, n16 = L & 15, grp = L >> 4;
    const int tok = tb * 16 + n16;
    const bool live = tok < a.M;
    const uint16_t *hrow = a.hidden + (size_t)(live ? tok : 0) * H;
    const int e = s_e[n16];
    const int p = tid >> 6;                                  // (step, half) pair of this thread
    const int s = blockIdx.y * kRStageSteps + (p >> 1), h = p & 1;
    if (s >= a.n_steps)
        return;
    // lane group grp, half h: channels 32*grp + 16*h .. +15 of the step
    const int ch0 = s * kRStepH + 32 * grp + 16 * h;
    float xs[16];
    if (live && ch0 < H) {
        load_xs16(hrow, a.scales, ch0, xs);
    } else {
#pragma unroll
        for (int j = 0; j < 16; ++j)
            xs[j] = 0.0f;
    }
    uint32_t limbw[3][4];
    split_limbs(xs, e, limbw);
#pragma unroll
    for (int l = 0; l < 3; ++l)
        a.frag_out[rfrag_index(tb, a.n_steps, s, h, l, L)] =
            u32x4{limbw[l][0], limbw[l][1], limbw[l][2], limbw[l][3]};
}

// ---------------------------------------------------------------- verify_rows_kernel
template <bool kLogits>
__global__ void __launch_bounds__(kRThreads) verify_rows_kernel(RArgs a)
{
    struct Lds {
        uint8_t wt[2][kRTileBytes];     // int8 weight fragments of the current and the next K step
        int exp[kBatchMaxRows];         // step exponents of the rows
        int arg[kBatchMaxRows];         // last workgroup: argmax ids
        int draft[kBatchMaxRows];       // last workgroup: draft ids
        int last;
    };
    __shared__ __attribute__((aligned(16))) Lds lds;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int n16 = lane & 15;   // MFMA row of A / column of B and D
    const int grp = lane >> 4;   // 16-lane group: K sub-block, D rows 4*grp..4*grp+3
    const int G = gridDim.x;
    // Item order: workgroups are dispatched to the 8 XCDs round-robin, so
    // blockIdx b runs on XCD b % 8.  Renumbering b -> (b % 8) * (G / 8) + b / 8
    // gives neighbouring item numbers -- the token tiles of one vocabulary
    // tile -- to workgroups of the same XCD, which then read that tile's
    // weights at the same time through one L2.
    const int b = (G % 8 == 0) ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8)
                               : (int)blockIdx.x;
    const int n_steps = a.n_steps, n_mt = a.n_mt;
    const int n_my = b < a.n_items ? (a.n_items - 1 - b) / G + 1 : 0;

    for (int m = tid; m < n_mt * kRTokTile; m += kRThreads)
        lds.exp[m] = a.exps[m];
    __syncthreads();

    // Weight chunks of this thread in every K step: 16 bytes (32 channels)
    // of rows 16*(wave + kRWaves*j) + n16 of the item's tile, chunk grp of
    // the step's 64 bytes, j < kRChunks.  The chunk becomes exactly the B fragment
    // words of this lane for column block wave + kRWaves*j, halves 0 and 1, so
    // each wave converts and stores whole 1 KB fragments.  Addresses past
    // the head are clamped (such rows are masked, and channels past H meet
    // zero codes).
    const unsigned long long w_last = a.w_bytes - 16;
    const unsigned long long row_bytes = (unsigned long long)(a.H / 2);
    auto load_w = [&](int k, int s, u32x4 (&q)[kRChunks]) {
        const int nt = (b + k * G) / n_mt;
#pragma unroll
        for (int j = 0; j < kRChunks; ++j) {
            unsigned long long off =
                (unsigned long long)(nt * kRVocTile + 16 * (wave + kRWaves * j) + n16) * row_bytes +
                (unsigned long long)(s * 64 + grp * 16);
            off = off < w_last ? off : w_last;
            q[j] = *reinterpret_cast<const u32x4 *>(a.w + off);
        }
    };
    // nibble -> high half of a byte: the int8 value is 16*q; fragment word
    // (half h, column block vb) of lane L sits at byte ((8h + vb) * 64 + L) * 16
    auto store_w = [&](uint8_t *wt, const u32x4 (&q)[kRChunks]) {
#pragma unroll
        for (int j = 0; j < kRChunks; ++j) {
            const int vb = wave + kRWaves * j;
            const i32x4 b0 = {(int32_t)((q[j][0] << 4) & 0xF0F0F0F0u), (int32_t)(q[j][0] & 0xF0F0F0F0u),
                              (int32_t)((q[j][1] << 4) & 0xF0F0F0F0u), (int32_t)(q[j][1] & 0xF0F0F0F0u)};
            const i32x4 b1 = {(int32_t)((q[j][2] << 4) & 0xF0F0F0F0u), (int32_t)(q[j][2] & 0xF0F0F0F0u),
                              (int32_t)((q[j][3] << 4) & 0xF0F0F0F0u), (int32_t)(q[j][3] & 0xF0F0F0F0u)};
            *reinterpret_cast<i32x4 *>(wt + (vb * 64 + lane) * 16) = b0;
            *reinterpret_cast<i32x4 *>(wt + ((8 + vb) * 64 + lane) * 16) = b1;
        }
    };
    // activation fragments of one half (64 channels) of a K step
    auto load_a = [&](int k, int s, int h, i32x4 (&A)[kRTbPerWave][2][3]) {
        const int tb0 = ((b + k * G) % n_mt) * kRTbPerTile + wave * kRTbPerWave;
#pragma unroll
        for (int t = 0; t < kRTbPerWave; ++t)
#pragma unroll
            for (int l = 0; l < 3; ++l)
                A[t][h][l] = __builtin_bit_cast(
                    i32x4, a.frag[rfrag_index(tb0 + t, n_steps, s, h, l, lane)]);
    };

    i32x4 acc[kRTbPerWave][3][kRVBlocks];
    auto zero_acc = [&]() {
#pragma unroll
        for (int t = 0; t < kRTbPerWave; ++t)
#pragma unroll
            for (int l = 0; l < 3; ++l)
#pragma unroll
                for (int vb = 0; vb < kRVBlocks; ++vb)
                    acc[t][l][vb] = i32x4{0, 0, 0, 0};
    };
    // One half (64 channels) of a K step over all column blocks.  The eight
    // B fragments are read from LDS before the first MFMA needs one (the
    // schedule is pinned: left alone, the compiler keeps only two reads in
    // flight and waits on each).
    auto mma_half = [&](const uint8_t *wt, int h, const i32x4 (&A)[kRTbPerWave][2][3]) {
        i32x4 bf[kRVBlocks];
#pragma unroll
        for (int vb = 0; vb < kRVBlocks; ++vb)
            bf[vb] = *reinterpret_cast<const i32x4 *>(wt + ((8 * h + vb) * 64 + lane) * 16);
#pragma unroll
        for (int vb = 0; vb < kRVBlocks; ++vb)
#pragma unroll
            for (int t = 0; t < kRTbPerWave; ++t)
#pragma unroll
                for (int l = 0; l < 3; ++l)
                    acc[t][l][vb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[t][h][l], bf[vb], acc[t][l][vb], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x0100, kRVBlocks, 0);                    // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x0008, kRVBlocks * kRTbPerWave * 3, 0);  // MFMAs
    };
    // End of an item: logits of this wave's 32 tokens x 128 rows, the best
    // per token into its key.  The limbs combine exactly in binary64
    // (|code| < 2^53); the one rounding to binary32 happens before the
    // power-of-two step is applied, which gives the same value because the
    // scaled logits stay in the normal range.  Within a lane the column
    // index grows with vb, so a strict > keeps the lowest index on ties.
    // Winners of consecutive items of the same token tile merge here first
    // (with G a multiple of the number of token tiles, a workgroup keeps one
    // token tile throughout), so each workgroup takes one atomic per token
    // and tile change: atomics on one line serialise at the memory side, and
    // a wave's later loads wait behind its outstanding atomics.
    unsigned long long run[kRTbPerWave][4];
#pragma unroll
    for (int t = 0; t < kRTbPerWave; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            run[t][r] = 0ull;
    auto finish_item = [&](int it, bool flush) {
        const int vcol = (it / n_mt) * kRVocTile + n16;
#pragma unroll
        for (int t = 0; t < kRTbPerWave; ++t) {
            const int tok0 = ((it % n_mt) * kRTbPerTile + wave * kRTbPerWave + t) * 16 + 4 * grp;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = tok0 + r;
                const int e = lds.exp[tok] - 4;   // weights carry a factor 16
                float bv = -__builtin_huge_valf();
                int bi = 0x7FFFFFFF;
#pragma unroll
                for (int vb = 0; vb < kRVBlocks; ++vb) {
                    const double code = __builtin_fma((double)acc[t][0][vb][r], 65536.0,
                                                      __builtin_fma((double)acc[t][1][vb][r], 256.0,
                                                                    (double)acc[t][2][vb][r]));
                    const float u = (float)code;          // the one rounding
                    const int v = vcol + vb * 16;
                    const bool take = v < a.V && u > bv;
                    bv = take ? u : bv;
                    bi = take ? v : bi;
                    if (kLogits && tok < a.M && v < a.V)
                        a.logits_out[(size_t)tok * a.V + v] = ldexpf(u, e);
                }
                row_best16(bv, bi);
                const unsigned long long key = order_key(ldexpf(bv, e), bi);
                if (kLogits && a.item_keys && n16 == 0 && tok < a.M)
                    a.item_keys[(size_t)tok * ((a.V + kRVocTile - 1) / kRVocTile) + it / n_mt] = key;
                run[t][r] = key > run[t][r] ? key : run[t][r];
                if (flush) {
                    if (n16 == 0 && tok < a.M)
                        __hip_atomic_fetch_max(&a.keys[tok], run[t][r], __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                    run[t][r] = 0ull;
                }
            }
        }
    };

    // ---------------- the (item, K step) stream, two steps per iteration
    // Registers: activation fragments of the even and the odd step in
    // flight (aE, aO), the packed weight chunks staged for the step after
    // next (wE, wO).  Steps past the end of the stream re-load the last one
    // (valid addresses, results unused), which keeps the sequence of memory
    // operations the same in every iteration.  n_steps is even, so items
    // start at an even step.
    zero_acc();
    if (n_my > 0) {
        i32x4 aE[kRTbPerWave][2][3], aO[kRTbPerWave][2][3];
        u32x4 wE[kRChunks], wO[kRChunks];
        load_a(0, 0, 0, aE);
        load_a(0, 0, 1, aE);
        load_w(0, 0, wE);
        load_a(0, 1, 0, aO);
        load_a(0, 1, 1, aO);
        load_w(0, 1, wO);
        store_w(lds.wt[0], wE);
        int kn = n_steps == 2 ? 1 : 0;     // item and step of the next even step
        int sn = n_steps == 2 ? 0 : 2;
        for (int k = 0; k < n_my; ++k) {
            const bool active =
                ((b + k * G) % n_mt) * kRTbPerTile + wave * kRTbPerWave < a.n_tb;
            for (int s = 0; s < n_steps; s += 2) {
                const int kp = kn < n_my ? kn : n_my - 1;
                const int sp = kn < n_my ? sn : n_steps - 2;
                // even step: weights in LDS tile 0, activations in aE
                __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                barrier_no_fence();
                load_w(kp, sp, wE);
                if (active)
                    mma_half(lds.wt[0], 0, aE);
                load_a(kp, sp, 0, aE);
                if (active)
                    mma_half(lds.wt[0], 1, aE);
                load_a(kp, sp, 1, aE);
                store_w(lds.wt[1], wO);
                // odd step: weights in LDS tile 1, activations in aO
                __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                barrier_no_fence();
                load_w(kp, sp + 1, wO);
                if (active)
                    mma_half(lds.wt[1], 0, aO);
                load_a(kp, sp + 1, 0, aO);
                if (active)
                    mma_half(lds.wt[1], 1, aO);
                load_a(kp, sp + 1, 1, aO);
                store_w(lds.wt[0], wE);
                sn += 2;
                if (sn == n_steps) {
                    sn = 0;
                    ++kn;
                }
            }
            finish_item(b + k * G, k == n_my - 1 || (b + (k + 1) * G) % n_mt != (b + k * G) % n_mt);
            zero_acc();
        }
    }

    // ---------------- completion: the last workgroup decodes the keys
    // Each wave's atomics are acknowledged before the ticket is taken (see
    // verify_kernel for why no fence is used).
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    if (tid == 0) {
        // two levels: the last workgroup of each group of 16 takes the top ticket
        const int gi = (int)blockIdx.x / kGroupWgs;
        const int gsz = min(kGroupWgs, G - kGroupWgs * gi);
        uint32_t *gt = a.group_ticket + (size_t)gi * kTicketStride;
        bool last = __hip_atomic_fetch_add(gt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                    (uint32_t)(gsz - 1);
        if (last) {
            __hip_atomic_store(gt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   (uint32_t)((G + kGroupWgs - 1) / kGroupWgs - 1);
        }
        lds.last = last;
    }
    __syncthreads();
    if (!lds.last)
        return;

    const int M = a.M;
    const int n_draft = a.R * (a.T - 1);
    constexpr int kPer = kBatchMaxRows / kRThreads;
    unsigned long long key[kPer];
    int dft[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {   // every load in flight before any is used
        const int m = tid + j * kRThreads;
        key[j] = m < M ? __hip_atomic_load(&a.keys[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                       : 0ull;
        dft[j] = m < n_draft ? a.draft[m] : 0;
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int m = tid + j * kRThreads;
        if (m < M) {
            const int row = key_index(key[j]);
            const int idx = a.vmap ? a.vmap[row] : row;   // row -> token id
            a.logits_max[m] = key_value(key[j]);
            a.argmax[m] = idx;
            lds.arg[m] = idx;
            __hip_atomic_store(&a.keys[m], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (m < n_draft)
            lds.draft[m] = dft[j];
    }
    __syncthreads();
    for (int i = tid; i < a.R; i += kRThreads) {
        const int T = a.T;
        int n = 0;
        while (n < T - 1 && lds.arg[i * T + n] == lds.draft[i * (T - 1) + n])
            ++n;
        a.n_acc[i] = n;
    }
    if (tid == 0)
        __hip_atomic_store(a.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- small kernels

__global__ void fill_zero_u32(uint32_t *p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = 0u;
}

__global__ void __launch_bounds__(256) count_bad_nibbles(const u32x4 *w, size_t n_vec, int32_t *out)
{
    int cnt = 0;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_vec;
         i += (size_t)gridDim.x * blockDim.x) {
        const u32x4 q = __builtin_nontemporal_load(w + i);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // a nibble equals 0x8 iff (nib ^ 0x8) == 0
            const uint32_t x = q[j] ^ 0x88888888u;
#pragma unroll
            for (int k = 0; k < 8; ++k)
                cnt += ((x >> (4 * k)) & 0xFu) == 0u;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        cnt += __shfl_xor(cnt, off);
    if ((threadIdx.x & 63) == 0 && cnt)
        atomicAdd(out, cnt);
}

// Count positions of a row -> token map that break "strictly increasing,
// non-negative" (map[0] < 0, or map[i] <= map[i-1]).
__global__ void __launch_bounds__(256) count_bad_map(const int32_t *map, int V, int32_t *out)
{
    int cnt = 0;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < V; i += gridDim.x * blockDim.x)
        cnt += (i == 0) ? (map[0] < 0) : (map[i] <= map[i - 1]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        cnt += __shfl_xor(cnt, off);
    if ((threadIdx.x & 63) == 0 && cnt)
        atomicAdd(out, cnt);
}

// ---------------------------------------------------------------- topk_rows_kernel
// Sampled verification of calls past the weight-stream kernels' 64 rows: the
// batch kernel writes every logit of the call into the workspace, and with it
// each row's best key over every vocabulary tile of 128 rows (one work item's
// columns); one workgroup per row then takes the row's top-k (order keys:
// larger value, then lower row), the log-sum-exp of logit / tau over the
// vocabulary and p(d) of the row's draft, with the formulas of the
// weight-stream kernels' sampled epilogue.  Exact for any input, ties
// included: the kTopK-th largest of the row's tile keys, th, is at most the
// row's kTopK-th key, and a key of the row that reaches th lies in a tile
// whose best key reaches th -- kTopK tiles -- so the kernel reads only those
// tiles' logits (at most kTopK * 128) and the kTopK largest of their keys that
// reach th are the row's.  The log-sum-exp, when needed, is one read of the
// whole row (one exp2 per logit).
constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelTile = 128;        // vocabulary rows per tile key (the batch kernel's work items)
constexpr int kSelUnroll = 16;       // loads in flight per thread (the log-sum-exp's read of the row)

struct SArgs {
    const float *logits;      // [M, V] binary32, in the workspace
    const unsigned long long *item_keys;   // [M, ceil(V / 128)] the rows' best keys per tile
    const int32_t *draft;     // [R, T-1] or null
    int32_t *topk_ids;        // [M, top_k] or null
    float *topk_logits;       // [M, top_k] or null
    float *p_draft;           // [R, T-1] or null
    float *lse_out;           // [M] or null
    int R, T, V, top_k;
    float tau;
};

__device__ __forceinline__ unsigned long long key_shfl_xor(unsigned long long k, int mask)
{
    const uint32_t lo = __shfl_xor((uint32_t)k, mask);
    const uint32_t hi = __shfl_xor((uint32_t)(k >> 32), mask);
    return ((unsigned long long)hi << 32) | lo;
}

// The 64 keys of a wave (one per lane), sorted best first across the lanes:
// a bitonic network of cross-lane compare-exchanges (keys are distinct).
__device__ __forceinline__ unsigned long long wave_sort64(unsigned long long k, int lane)
{
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const unsigned long long o = key_shfl_xor(k, stride);
            // descending overall: the lower lane of a pair keeps the larger key
            // in blocks whose bit `size` is clear, the smaller one otherwise
            const bool keep_max = ((lane & stride) == 0) == ((lane & size) == 0);
            k = keep_max ? (o > k ? o : k) : (o < k ? o : k);
        }
    return k;
}

// The best 64 of two best-first lane-sorted lists, best first: the larger of
// a[j] and b[63 - j] form a bitonic sequence of exactly those 64 keys, which a
// bitonic merge sorts.
__device__ __forceinline__ unsigned long long wave_merge64(unsigned long long a, unsigned long long b, int lane)
{
    const unsigned long long br = key_shfl(b, 63 - lane);
    unsigned long long m = a > br ? a : br;
#pragma unroll
    for (int stride = 32; stride > 0; stride >>= 1) {
        const unsigned long long o = key_shfl_xor(m, stride);
        m = (lane & stride) == 0 ? (o > m ? o : m) : (o < m ? o : m);
    }
    return m;
}

// The kTopK largest of the n distinct keys buf[0, n) into out[0, kTopK), best
// first (key 0, below every real key, for ranks past n).  Each wave keeps the
// best 64 of its chunks of 64 keys (sort, merge); wave 0 merges the waves'
// best kTopK.  Called by the whole workgroup; out is complete when it
// returns.
template <int kTopK>
__device__ void wg_top_keys(const unsigned long long *buf, int n, unsigned long long *out,
                            unsigned long long (*wtop)[kTopK])
{
    static_assert(kSelWaves * kTopK <= 128, "two registers of wave 0 hold the waves' lists");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    unsigned long long r = 0ull;
    for (int c = wave * 64; c < n; c += kSelThreads) {
        const unsigned long long k = c + lane < n ? buf[c + lane] : 0ull;
        r = wave_merge64(r, wave_sort64(k, lane), lane);
    }
    if (lane < kTopK)
        wtop[wave][lane] = r;
    __syncthreads();
    if (wave == 0) {
        constexpr int kAll = kSelWaves * kTopK;
        const unsigned long long a = lane < kAll ? wtop[lane / kTopK][lane % kTopK] : 0ull;
        unsigned long long m = wave_sort64(a, lane);
        if constexpr (kAll > 64) {
            const unsigned long long b = 64 + lane < kAll ? wtop[(64 + lane) / kTopK][(64 + lane) % kTopK] : 0ull;
            m = wave_merge64(m, wave_sort64(b, lane), lane);
        }
        if (lane < kTopK)
            out[lane] = m;
    }
    __syncthreads();
}

// Grid: one workgroup per row of the call.  kTopK: 8 or 16 (top_k rounded up;
// 0 for sampling over the whole vocabulary, which needs no list: the greedy
// outputs come from the batch kernel).  kLse: the log-sum-exp is needed (top_k
// == 0, or the caller asked for it).
template <int kTopK, bool kLse>
__global__ void __launch_bounds__(kSelThreads) topk_rows_kernel(SArgs a)
{
    constexpr int kCand = kTopK * kSelTile;   // gathered keys, at most
    __shared__ unsigned long long s_cand[kCand > 0 ? kCand : 1];
    __shared__ unsigned long long s_top[kTopK > 0 ? kTopK : 1];
    __shared__ unsigned long long s_wtop[kSelWaves][kTopK > 0 ? kTopK : 1];
    __shared__ float s_lm[kSelWaves], s_ls[kSelWaves];
    __shared__ int s_qs[kTopK > 0 ? kTopK : 1];
    __shared__ int s_n, s_nq;

    const int m = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int V = a.V;
    const float *lg = a.logits + (size_t)m * V;

    if (tid == 0) {
        s_n = 0;
        s_nq = 0;
    }
    if constexpr (kLse) {
        // (max, sum) of exp2(logit * log2(e) / tau) over the row, one exp2
        // per logit, kSelUnroll loads in flight per thread
        const float zscale = 1.4426950408889634f / a.tau;   // log2(e) / tau
        float lm = -__builtin_huge_valf(), ls = 0.0f;
        int i0 = tid;
        for (; i0 + (kSelUnroll - 1) * kSelThreads < V; i0 += kSelUnroll * kSelThreads) {
            float v[kSelUnroll];
#pragma unroll
            for (int u = 0; u < kSelUnroll; ++u)
                v[u] = lg[i0 + u * kSelThreads];
#pragma unroll
            for (int u = 0; u < kSelUnroll; ++u)
                lse_add(lm, ls, v[u] * zscale);
        }
        for (; i0 < V; i0 += kSelThreads)
            lse_add(lm, ls, lg[i0] * zscale);
        row_lse16(lm, ls);
        lse_combine(lm, ls, __shfl_xor(lm, 16), __shfl_xor(ls, 16));
        lse_combine(lm, ls, __shfl_xor(lm, 32), __shfl_xor(ls, 32));
        if (lane == 0) {
            s_lm[wave] = lm;
            s_ls[wave] = ls;
        }
    }
    __syncthreads();
    if constexpr (kTopK > 0) {
        const int n_t = (V + kSelTile - 1) / kSelTile;
        const unsigned long long *tk = a.item_keys + (size_t)m * n_t;
        wg_top_keys<kTopK>(tk, n_t, s_top, s_wtop);
        // th is 0 when the row has fewer than kTopK tiles: then every tile
        // qualifies and every logit is a candidate
        const unsigned long long th = s_top[kTopK - 1];
        const float thv = th != 0ull ? key_value(th) : -__builtin_huge_valf();
        // the tiles whose best key reaches th (at most kTopK)
        for (int t = tid; t < n_t; t += kSelThreads)
            if (tk[t] >= th) {
                const int slot = atomicAdd(&s_nq, 1);
                if (slot < kTopK)
                    s_qs[slot] = t;
            }
        __syncthreads();
        // their keys that reach th (value test first; a key reaching th has a
        // value reaching th's), every load of a thread in flight at once
        const int nq = min(s_nq, kTopK);
        constexpr int kPer = kCand / kSelThreads;
        float v[kPer];
        int idx[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = tid + u * kSelThreads;            // element e % 128 of qualifying tile e / 128
            const int q = e / kSelTile;
            const int i = q < nq ? s_qs[q] * kSelTile + e % kSelTile : V;
            idx[u] = i < V ? i : -1;
            v[u] = i < V ? lg[i] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u)
            if (idx[u] >= 0 && v[u] >= thv) {
                const unsigned long long k = order_key(v[u], idx[u]);
                if (k >= th) {
                    const int slot = atomicAdd(&s_n, 1);
                    if (slot < kCand)
                        s_cand[slot] = k;
                }
            }
        __syncthreads();
        wg_top_keys<kTopK>(s_cand, min(s_n, kCand), s_top, s_wtop);
    }

    // outputs: wave 0, lane j of its first 16 lanes takes rank j
    if (wave != 0)
        return;
    const int T = a.T, req = m / T, t = m % T;
    const bool drafted = t < T - 1;
    const int di = drafted ? req * (T - 1) + t : 0;
    const int d = drafted ? a.draft[di] : -1;
    float lse = 0.0f;
    if constexpr (kLse) {
        float gm = s_lm[0], gs = s_ls[0];
#pragma unroll
        for (int w = 1; w < kSelWaves; ++w)
            lse_combine(gm, gs, s_lm[w], s_ls[w]);
        lse = (gm + __log2f(gs)) * 0.6931471805599453f;
    }
    float p = 0.0f;
    if constexpr (kTopK > 0) {
        const int j = lane & 15;
        const unsigned long long key = j < kTopK ? s_top[j] : 0ull;
        const float hv = key_value(key);
        const int hi = key_index(key);
        const float lmax = key_value(s_top[0]);
        const bool in = lane < 16 && j < a.top_k;
        const float e = in ? expf((hv - lmax) / a.tau) : 0.0f;
        const float sum = row_sum16(e);
        const float e_d = row_sum16(in && hi == d ? e : 0.0f);
        if (in) {
            a.topk_ids[(size_t)m * a.top_k + j] = hi;
            a.topk_logits[(size_t)m * a.top_k + j] = hv;
        }
        p = e_d / sum;
    } else {
        p = (d >= 0 && d < V) ? expf(lg[d] / a.tau - lse) : 0.0f;
    }
    if (lane == 0) {
        if (kLse && a.lse_out)
            a.lse_out[m] = lse;
        if (drafted)
            a.p_draft[di] = p;
    }
}

// The accepted count of each request from its rows' p(d): drafts are
// accepted while uniforms * draft_probs < p_draft (binary32, the comparison of
// the weight-stream kernels' epilogue).
__global__ void __launch_bounds__(256) accept_rows_kernel(const float *p_draft, const float *dprob, const float *unif,
                                                          int R, int T, int32_t *n_acc)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= R)
        return;
    int n = 0;
    while (n < T - 1) {
        const int di = i * (T - 1) + n;
        if (!(unif[di] * dprob[di] < p_draft[di]))
            break;
        ++n;
    }
    n_acc[i] = n;
}

// ---------------------------------------------------------------- host side

int hip_fail(hipError_t e, const char *what)
{
    return int4vh_detail::hip_fail(e, what);
}

using int4vh_detail::cu_count;
using int4vh_detail::launch_timed;

bool aligned(const void *p, size_t al)
{
    return ((uintptr_t)p % al) == 0;
}

typedef void (*KernelFn)(Args);

struct Pair {
    KernelFn stage;
    KernelFn verify;
};

// Ring depth: three tiles in flight while they fit in LDS, else two.
template <int kP, int kUnits, bool kLogits, int kTopK, bool kLse>
Pair make_pair()
{
    constexpr int kRing = kUnits <= 5 ? 3 : 2;
    return Pair{stage_kernel<kP, kUnits>, verify_kernel<kP, kUnits, kRing, kLogits, kTopK, kLse, false>};
}

// Token groups of 16 rows sharing the tile stream: the weight copies use
// the normal cache policy, so that the workgroups of a tile set that ask for
// a tile after the first find it in their XCD's L2.
template <int kUnits, bool kLogits>
Pair make_grouped()
{
    constexpr int kRing = kUnits <= 5 ? 3 : 2;
    return Pair{stage_kernel<16, kUnits>, verify_kernel<16, kUnits, kRing, kLogits, 0, false, false, 0>};
}

// Token groups with the sampled epilogue (8- or 16-entry lists, with or
// without the whole-vocabulary log-sum-exp).
template <int kUnits, int kTopK, bool kLse>
Pair make_grouped_sampled()
{
    constexpr int kRing = kUnits <= 5 ? 3 : 2;
    return Pair{stage_kernel<16, kUnits>, verify_kernel<16, kUnits, kRing, false, kTopK, kLse, false, 0>};
}

template <int kTopK, bool kLse>
Pair pick_grouped_sampled(int units)
{
    switch (units) {
    case 1: return make_grouped_sampled<1, kTopK, kLse>();
    case 2: return make_grouped_sampled<2, kTopK, kLse>();
    case 3: return make_grouped_sampled<3, kTopK, kLse>();
    case 4: return make_grouped_sampled<4, kTopK, kLse>();
    case 5: return make_grouped_sampled<5, kTopK, kLse>();
    case 6: return make_grouped_sampled<6, kTopK, kLse>();
    case 7: return make_grouped_sampled<7, kTopK, kLse>();
    default: return make_grouped_sampled<8, kTopK, kLse>();
    }
}

template <bool kLogits>
Pair pick_grouped(int units)
{
    switch (units) {
    case 1: return make_grouped<1, kLogits>();
    case 2: return make_grouped<2, kLogits>();
    case 3: return make_grouped<3, kLogits>();
    case 4: return make_grouped<4, kLogits>();
    case 5: return make_grouped<5, kLogits>();
    case 6: return make_grouped<6, kLogits>();
    case 7: return make_grouped<7, kLogits>();
    default: return make_grouped<8, kLogits>();
    }
}

// One launch, staging inside the verify kernel (up to 2 rows).
template <int kUnits, bool kLogits>
Pair make_fused()
{
    constexpr int kRing = kUnits <= 5 ? 3 : 2;
    return Pair{nullptr, verify_kernel<5, kUnits, kRing, kLogits, 0, false, true>};
}

template <bool kLogits>
Pair pick_fused(int units)
{
    switch (units) {
    case 1: return make_fused<1, kLogits>();
    case 2: return make_fused<2, kLogits>();
    case 3: return make_fused<3, kLogits>();
    case 4: return make_fused<4, kLogits>();
    case 5: return make_fused<5, kLogits>();
    case 6: return make_fused<6, kLogits>();
    case 7: return make_fused<7, kLogits>();
    default: return make_fused<8, kLogits>();
    }
}

// Whether a greedy call of M rows stages inside the verify kernel: its codes
// (3 bytes per row and padded channel) must fit the 32 KB partial-sum area.
bool fused_staging(int M, int units)
{
    return M <= 2 && (size_t)M * 3 * units * kWaves * kUnitH + 2 * kWaves * sizeof(float) <=
                         sizeof(unsigned long long) * 2 * kWaves * kTileRows * kTileRows;
}

template <int kP, bool kLogits, int kTopK, bool kLse>
Pair pick(int units)
{
    switch (units) {
    case 1: return make_pair<kP, 1, kLogits, kTopK, kLse>();
    case 2: return make_pair<kP, 2, kLogits, kTopK, kLse>();
    case 3: return make_pair<kP, 3, kLogits, kTopK, kLse>();
    case 4: return make_pair<kP, 4, kLogits, kTopK, kLse>();
    case 5: return make_pair<kP, 5, kLogits, kTopK, kLse>();
    case 6: return make_pair<kP, 6, kLogits, kTopK, kLse>();
    case 7: return make_pair<kP, 7, kLogits, kTopK, kLse>();
    default: return make_pair<kP, 8, kLogits, kTopK, kLse>();
    }
}

template <bool kLogits, int kTopK, bool kLse>
Pair pick_rows(int M, int units, int *kp)
{
    if (M <= 5) {
        *kp = 5;
        return pick<5, kLogits, kTopK, kLse>(units);
    }
    if (M <= 8) {
        *kp = 8;
        return pick<8, kLogits, kTopK, kLse>(units);
    }
    *kp = 16;
    return pick<16, kLogits, kTopK, kLse>(units);
}

// Kernel pair for a call: greedy (with or without every logit written), or
// the sampled epilogue with an 8- or 16-entry top-k list, with the running
// log-sum-exp when the call samples over the whole vocabulary or asks for it.
Pair pick_kernels(int M, int units, bool logits, bool sampled, int top_k, bool lse, int *kp)
{
    if (sampled && top_k > 8)
        return lse ? pick_rows<false, 16, true>(M, units, kp) : pick_rows<false, 16, false>(M, units, kp);
    if (sampled)
        return lse ? pick_rows<false, 8, true>(M, units, kp) : pick_rows<false, 8, false>(M, units, kp);
    return logits ? pick_rows<true, 0, false>(M, units, kp) : pick_rows<false, 0, false>(M, units, kp);
}

// K steps of the batch path (128 channels each, rounded up to even).
int rows_steps(int H)
{
    const int n = (H + kRStepH - 1) / kRStepH;
    return (n + 1) & ~1;
}

// Rows of the largest call the weight-stream kernels take (token groups of
// 16 sharing the tile stream); larger calls run the matrix-core batch path.
constexpr int kStreamMaxRows = kMaxRows * kMaxGroups;

// The sampled epilogue's area (per-workgroup and per-merge-group lists and
// pairs) follows the activation fragments of the call's token groups.
constexpr size_t kSampledArea = kWsBytes - kWsTopK;
size_t sampled_base(int n_groups)
{
    return kWsFrag + (size_t)n_groups * kFragBytes;
}

size_t workspace_need(int R, int T, int V, int H)
{
    if (R < 1 || T < 1 || T > INT4VH_MAX_T || V < 1 || H < 32 || (H % 32) != 0)
        return 0;
    const long long M = (long long)R * T;
    if (M > kBatchMaxRows)
        return 0;
    if (M <= kMaxRows)
        return kWsBytes;
    if (M <= kStreamMaxRows)   // one fragment area per token group, then the sampled epilogue's area
        return sampled_base((int)((M + kMaxRows - 1) / kMaxRows)) + kSampledArea;
    const size_t n_mt = (size_t)((M + kRTokTile - 1) / kRTokTile);
    return kWsFrag + n_mt * (size_t)kRTbPerTile * (size_t)rows_steps(H) * 2 * 3 * 64 * 16;
}

// The sampled call's workspace: past the weight-stream kernels' rows the
// call's logits (binary32 [M, V]) and the rows' best keys per vocabulary tile
// of 128 (uint64 [M, ceil(V / 128)]) follow the batch path's area.
size_t logits_offset(int R, int T, int V, int H)
{
    return (workspace_need(R, T, V, H) + 255) & ~(size_t)255;
}
size_t item_keys_offset(int R, int T, int V, int H)
{
    return (logits_offset(R, T, V, H) + (size_t)R * (size_t)T * (size_t)V * sizeof(float) + 255) & ~(size_t)255;
}
size_t sampled_need(int R, int T, int V, int H)
{
    const size_t base = workspace_need(R, T, V, H);
    if (base == 0 || (long long)R * T <= kStreamMaxRows)
        return base;
    return item_keys_offset(R, T, V, H) +
           (size_t)R * (size_t)T * (size_t)((V + kRVocTile - 1) / kRVocTile) * sizeof(unsigned long long);
}

// Every argument check except the workspace's (no GPU call).
int validate_args(const void *hidden, const uint8_t *w, const void *scales, const int32_t *draft,
                  int R, int T, int V, int H, const float *lmax, const int32_t *amax_ids,
                  const int32_t *nacc, const float *lout)
{
    if (R < 1 || T < 1 || T > INT4VH_MAX_T || V < 1 || H < 32 || (H % 32) != 0)
        return INT4VH_EINVAL;
    if ((long long)R * T > kBatchMaxRows)
        return INT4VH_EINVAL;
    if (!hidden || !w || !scales || !lmax || !amax_ids || !nacc)
        return INT4VH_EINVAL;
    if (T > 1 && !draft)
        return INT4VH_EINVAL;
    if (H > INT4VH_MAX_H)
        return INT4VH_EUNSUPPORTED;
    if ((unsigned long long)V * (unsigned long long)(H / 2) >= (1ull << 40))
        return INT4VH_EUNSUPPORTED;
    if (!aligned(hidden, 16) || !aligned(w, 16) || !aligned(scales, 16) || !aligned(lmax, 16) ||
        !aligned(amax_ids, 16) || !aligned(nacc, 4) || (draft && !aligned(draft, 4)) ||
        (lout && !aligned(lout, 16)))
        return INT4VH_EALIGN;
    return INT4VH_OK;
}

int validate(const void *hidden, const uint8_t *w, const void *scales, const int32_t *draft,
             int R, int T, int V, int H, const float *lmax, const int32_t *amax_ids,
             const int32_t *nacc, const float *lout, const void *ws, size_t ws_bytes)
{
    const int st = validate_args(hidden, w, scales, draft, R, T, V, H, lmax, amax_ids, nacc, lout);
    if (st != INT4VH_OK)
        return st;
    if (!ws)
        return INT4VH_EINVAL;
    if (!aligned(ws, 256))
        return INT4VH_EALIGN;
    if (ws_bytes < workspace_need(R, T, V, H))
        return INT4VH_EWORKSPACE;
    return INT4VH_OK;
}

// The main kernel of a call, timed by ev0 / ev1 when given (launch_timed).
template <typename A>
int launch_main(void (*kernel)(A), dim3 grid, dim3 block, hipStream_t s, void *ev0, void *ev1, const A &a,
                const char *what)
{
    const hipError_t e = launch_timed(kernel, grid, block, s, ev0, ev1, a);
    return e == hipSuccess ? INT4VH_OK : hip_fail(e, what);
}

int launch_rows(const void *hidden, const uint8_t *w, const void *scales, const int32_t *draft,
                int R, int T, int V, int H, float *lmax, int32_t *amax_ids, int32_t *nacc,
                float *lout, const int32_t *vmap, char *wsb, int dev, hipStream_t s, void *ev0,
                void *ev1, unsigned long long *item_keys = nullptr)
{
    RArgs a;
    a.vmap = vmap;
    a.item_keys = item_keys;
    a.hidden = static_cast<const uint16_t *>(hidden);
    a.w = w;
    a.scales = static_cast<const uint16_t *>(scales);
    a.draft = draft;
    a.logits_max = lmax;
    a.argmax = amax_ids;
    a.n_acc = nacc;
    a.logits_out = lout;
    a.keys = reinterpret_cast<unsigned long long *>(wsb + kWsKeys);
    a.ticket = reinterpret_cast<uint32_t *>(wsb + kWsTicket);
    a.group_ticket = reinterpret_cast<uint32_t *>(wsb + kWsGroupTk);
    a.exps = reinterpret_cast<int32_t *>(wsb + kWsExp);
    a.frag = reinterpret_cast<const u32x4 *>(wsb + kWsFrag);
    a.frag_out = reinterpret_cast<u32x4 *>(wsb + kWsFrag);
    a.R = R;
    a.T = T;
    a.M = R * T;
    a.V = V;
    a.H = H;
    a.n_steps = rows_steps(H);
    a.n_tb = (a.M + 15) / 16;
    a.n_mt = (a.M + kRTokTile - 1) / kRTokTile;
    const long long n_vt = (V + kRVocTile - 1) / kRVocTile;
    if ((long long)a.n_mt * n_vt > 0x7FFFFFFFll / 2)
        return INT4VH_EUNSUPPORTED;
    a.n_items = (int)(a.n_mt * n_vt);
    a.w_bytes = (unsigned long long)V * (unsigned long long)(H / 2);
    int grid = cu_count(dev);
    if (grid > a.n_items)
        grid = a.n_items;
    const dim3 stage_grid(a.n_mt * kRTbPerTile, (a.n_steps + kRStageSteps - 1) / kRStageSteps);
    hipLaunchKernelGGL(stage_rows_kernel, stage_grid, dim3(kRStageThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return hip_fail(e, "stage_rows kernel launch");
    return launch_main(lout ? verify_rows_kernel<true> : verify_rows_kernel<false>, dim3(grid), dim3(kRThreads), s,
                       ev0, ev1, a, "verify_rows kernel launch");
}

// Outputs and parameters of the sampled epilogue.
struct Sampled {
    int top_k;
    float tau;
    const float *dprob;
    const float *unif;
    int32_t *topk_ids;
    float *topk_logits;
    float *p_draft;
    float *lse;
};

int launch_verify(const void *hidden, const uint8_t *w, const void *scales, const int32_t *draft,
                  int R, int T, int V, int H, float *lmax, int32_t *amax_ids, int32_t *nacc,
                  float *lout, void *ws, size_t ws_bytes, void *stream, void *ev0 = nullptr,
                  void *ev1 = nullptr, const int32_t *vmap = nullptr, const Sampled *smp = nullptr)
{
    const int st = validate(hidden, w, scales, draft, R, T, V, H, lmax, amax_ids, nacc, lout, ws,
                            ws_bytes);
    if (st != INT4VH_OK)
        return st;
    if (vmap && !aligned(vmap, 4))
        return INT4VH_EALIGN;
    if (smp && R * T > kStreamMaxRows)
        return INT4VH_EUNSUPPORTED;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");

    char *wsb = static_cast<char *>(ws);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (R * T > kStreamMaxRows)
        return launch_rows(hidden, w, scales, draft, R, T, V, H, lmax, amax_ids, nacc, lout, vmap,
                           wsb, dev, s, ev0, ev1);
    Args a;
    a.vmap = vmap;
    a.group_ticket = reinterpret_cast<uint32_t *>(wsb + kWsGroupTk);
    a.top_k = smp ? smp->top_k : 0;
    a.tau = smp ? smp->tau : 1.0f;
    a.dprob = smp ? smp->dprob : nullptr;
    a.unif = smp ? smp->unif : nullptr;
    a.topk_ids = smp ? smp->topk_ids : nullptr;
    a.topk_logits = smp ? smp->topk_logits : nullptr;
    a.p_draft = smp ? smp->p_draft : nullptr;
    a.lse_out = smp ? smp->lse : nullptr;
    a.draft_seen = reinterpret_cast<int32_t *>(wsb + kWsDraftSeen);
    a.draft_logit = reinterpret_cast<float *>(wsb + kWsDraftLogit);
    a.hidden = static_cast<const uint16_t *>(hidden);
    a.w = w;
    a.scales = static_cast<const uint16_t *>(scales);
    a.draft = draft;
    a.logits_max = lmax;
    a.argmax = amax_ids;
    a.n_acc = nacc;
    a.logits_out = lout;
    a.ticket = reinterpret_cast<uint32_t *>(wsb + kWsTicket);
    a.exps = reinterpret_cast<int32_t *>(wsb + kWsExp);
    a.part = reinterpret_cast<uint64_t *>(wsb + kWsPart);
    a.frag = reinterpret_cast<const u32x4 *>(wsb + kWsFrag);
    a.frag_out = reinterpret_cast<u32x4 *>(wsb + kWsFrag);
    a.R = R;
    a.T = T;
    a.M = R * T;
    a.V = V;
    a.H = H;
    a.n_units = (H + kUnitH - 1) / kUnitH;
    a.n_tiles = (V + kTileRows - 1) / kTileRows;
    a.w_bytes = (unsigned long long)V * (unsigned long long)(H / 2);
    const int units = (a.n_units + kWaves - 1) / kWaves;
    int grid = cu_count(dev);
    if (grid > kMaxGrid)
        grid = kMaxGrid;
    // more than 16 rows: token groups of 16, one workgroup of each group per
    // tile set (whole sets of 8 when there are 8 or more, so a set shares an
    // XCD; at most 128 sets, the final merge's capacity)
    a.n_groups = (a.M + kMaxRows - 1) / kMaxRows;
    a.group_words = kFragBytes / sizeof(u32x4);
    {
        // the sampled epilogue's area follows the groups' fragments
        char *sb = wsb + sampled_base(a.n_groups);
        a.part_topk = reinterpret_cast<unsigned long long *>(sb);
        a.group_topk = reinterpret_cast<unsigned long long *>(sb + (kWsGroupTopK - kWsTopK));
        a.part_lse = reinterpret_cast<uint64_t *>(sb + (kWsLse - kWsTopK));
        a.group_lse = reinterpret_cast<uint64_t *>(sb + (kWsGroupLse - kWsTopK));
    }
    if (a.n_groups > 1) {
        int sets = grid / a.n_groups;
        if (sets > kMaxGrid / kMaxGroups)
            sets = kMaxGrid / kMaxGroups;
        if (smp && sets > kSampledMaxGrid / a.n_groups)   // the sampled area's capacity
            sets = kSampledMaxGrid / a.n_groups;
        if (sets > a.n_tiles)
            sets = a.n_tiles;
        if (sets >= 8)
            sets -= sets % 8;
        a.n_sets = sets;
        grid = sets * a.n_groups;
    } else {
        if (grid > a.n_tiles)
            grid = a.n_tiles;
        if (smp && grid > kSampledMaxGrid)
            grid = kSampledMaxGrid;
        a.n_sets = grid;
    }
    int kp = 16;
    const bool fused = !smp && a.n_groups == 1 && fused_staging(a.M, units);
    const bool smp_lse = smp && (smp->top_k == 0 || smp->lse != nullptr);
    const Pair fn = fused ? (lout ? pick_fused<true>(units) : pick_fused<false>(units))
                    : (a.n_groups > 1 && smp)
                        ? (smp->top_k > 8 ? (smp_lse ? pick_grouped_sampled<16, true>(units)
                                                     : pick_grouped_sampled<16, false>(units))
                                          : (smp_lse ? pick_grouped_sampled<8, true>(units)
                                                     : pick_grouped_sampled<8, false>(units)))
                    : a.n_groups > 1 ? (lout ? pick_grouped<true>(units) : pick_grouped<false>(units))
                                     : pick_kernels(a.M, units, lout != nullptr, smp != nullptr, smp ? smp->top_k : 0,
                                                    smp && (smp->top_k == 0 || smp->lse != nullptr), &kp);
    if (fn.stage) {
        hipLaunchKernelGGL(fn.stage, dim3(kp * a.n_groups), dim3(kStageThreads), 0, s, a);
        e = hipGetLastError();
        if (e != hipSuccess)
            return hip_fail(e, "stage kernel launch");
    }
    return launch_main(fn.verify, dim3(grid), dim3(kThreads), s, ev0, ev1, a, "verify kernel launch");
}

// Sampled call of more than 64 rows: the batch kernels with the logits
// written to the workspace, then topk_rows_kernel (one workgroup per row) and
// the acceptance count.
int launch_sampled_rows(const void *hidden, const uint8_t *w, const void *scales, const int32_t *draft,
                        int R, int T, int V, int H, float *lmax, int32_t *amax_ids, int32_t *nacc,
                        void *ws, size_t ws_bytes, void *stream, void *ev0, void *ev1, const Sampled &smp)
{
    int st = validate_args(hidden, w, scales, draft, R, T, V, H, lmax, amax_ids, nacc, nullptr);
    if (st != INT4VH_OK)
        return st;
    if (!ws)
        return INT4VH_EINVAL;
    if (!aligned(ws, 256))
        return INT4VH_EALIGN;
    if (ws_bytes < sampled_need(R, T, V, H))
        return INT4VH_EWORKSPACE;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    char *wsb = static_cast<char *>(ws);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    float *lg = reinterpret_cast<float *>(wsb + logits_offset(R, T, V, H));
    auto *tk = reinterpret_cast<unsigned long long *>(wsb + item_keys_offset(R, T, V, H));
    const bool lse = smp.top_k == 0 || smp.lse != nullptr;
    st = launch_rows(hidden, w, scales, draft, R, T, V, H, lmax, amax_ids, nacc, lg, nullptr, wsb, dev, s, ev0,
                     ev1, smp.top_k > 0 ? tk : nullptr);
    if (st != INT4VH_OK)
        return st;
    const SArgs a{lg, tk, draft, smp.topk_ids, smp.topk_logits, smp.p_draft, smp.lse, R, T, V, smp.top_k,
                  smp.tau};
    const dim3 grid(R * T), block(kSelThreads);
    if (smp.top_k == 0)
        hipLaunchKernelGGL((topk_rows_kernel<0, true>), grid, block, 0, s, a);
    else if (smp.top_k <= 8 && lse)
        hipLaunchKernelGGL((topk_rows_kernel<8, true>), grid, block, 0, s, a);
    else if (smp.top_k <= 8)
        hipLaunchKernelGGL((topk_rows_kernel<8, false>), grid, block, 0, s, a);
    else if (lse)
        hipLaunchKernelGGL((topk_rows_kernel<16, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((topk_rows_kernel<16, false>), grid, block, 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess)
        return hip_fail(e, "topk_rows kernel launch");
    if (T > 1) {
        // (the batch kernel's greedy count is replaced)
        hipLaunchKernelGGL(accept_rows_kernel, dim3((R + 255) / 256), dim3(256), 0, s, smp.p_draft, smp.dprob,
                           smp.unif, R, T, nacc);
        e = hipGetLastError();
        if (e != hipSuccess)
            return hip_fail(e, "accept_rows kernel launch");
    }
    return INT4VH_OK;
}

// ---------------------------------------------------------------- static scratch
// The workspace of verify_lm_head_int4_batch_noalloc: one array per device,
// allocated when the code object is loaded and held until the process ends.
// Host code never uses the array's name as an address (in host code it names
// a host-side stand-in); it uses the device address from hipGetSymbolAddress,
// taken once per device with that device current.
constexpr size_t kScratchBytes = INT4VH_SCRATCH_BYTES;

} // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

struct ScratchSlot {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
    std::atomic<bool> zeroed{false};   // control block zeroed by an uncaptured fill
};
ScratchSlot g_scratch[int4vh_detail::kMaxDevicesPublic];

// The device address of `scratch` on device dev (the current device), with
// its control block zeroed.  The zeroing is a fill kernel on the caller's
// stream: under stream capture it becomes part of the graph (every replay
// zeroes again), and the next uncaptured call issues it once more.  Every
// verify call leaves the control block zeroed, so this is needed once per
// device, and again after a call that failed.
int scratch_for_device(int dev, hipStream_t s, char **out)
{
    if (dev < 0 || dev >= int4vh_detail::kMaxDevicesPublic)
        return INT4VH_EUNSUPPORTED;
    ScratchSlot &sl = g_scratch[dev];
    std::call_once(sl.once, [&sl] { sl.err = hipGetSymbolAddress(&sl.ptr, HIP_SYMBOL(scratch)); });
    if (sl.err != hipSuccess)
        return hip_fail(sl.err, "hipGetSymbolAddress(scratch)");
    if (!sl.ptr || !aligned(sl.ptr, 256))
        return hip_fail(hipErrorInvalidSymbol, "scratch address");
    if (!sl.zeroed.load(std::memory_order_acquire)) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing(s, &cs);
        if (e != hipSuccess)
            return hip_fail(e, "hipStreamIsCapturing");
        const int n = (int)(kWsCtlBytes / sizeof(uint32_t));
        hipLaunchKernelGGL(fill_zero_u32, dim3((n + 255) / 256), dim3(256), 0, s, static_cast<uint32_t *>(sl.ptr),
                           n);
        e = hipGetLastError();
        if (e != hipSuccess)
            return hip_fail(e, "scratch zero launch");
        if (cs == hipStreamCaptureStatusNone)
            sl.zeroed.store(true, std::memory_order_release);
    }
    *out = static_cast<char *>(sl.ptr);
    return INT4VH_OK;
}

} // namespace

extern "C" {

size_t verify_lm_head_int4_workspace_bytes(int R, int T, int V, int H)
{
    return workspace_need(R, T, V, H);
}

size_t verify_lm_head_int4_sampled_workspace_bytes(int R, int T, int V, int H)
{
    return sampled_need(R, T, V, H);
}

int verify_lm_head_int4_workspace_init(void *ws, size_t ws_bytes, void *stream)
{
    if (!ws)
        return INT4VH_EINVAL;
    if (!aligned(ws, 256))
        return INT4VH_EALIGN;
    if (ws_bytes < kWsCtlBytes)
        return INT4VH_EWORKSPACE;
    const int n = (int)(kWsCtlBytes / sizeof(uint32_t));
    hipLaunchKernelGGL(fill_zero_u32, dim3((n + 255) / 256), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<uint32_t *>(ws), n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return hip_fail(e, "workspace init launch");
    return INT4VH_OK;
}

int verify_lm_head_int4(const void *hidden, const uint8_t *packed_w, const void *scales,
                        const int32_t *draft_ids, int T, int V, int H, float *logits_max,
                        int32_t *argmax_ids, int32_t *n_accepted, float *logits_out,
                        void *workspace, size_t workspace_bytes, void *stream)
{
    return launch_verify(hidden, packed_w, scales, draft_ids, 1, T, V, H, logits_max, argmax_ids,
                         n_accepted, logits_out, workspace, workspace_bytes, stream);
}

int verify_lm_head_int4_batch(const void *hidden, const uint8_t *packed_w, const void *scales,
                              const int32_t *draft_ids, int R, int T, int V, int H,
                              float *logits_max, int32_t *argmax_ids, int32_t *n_accepted,
                              float *logits_out, void *workspace, size_t workspace_bytes,
                              void *stream)
{
    return launch_verify(hidden, packed_w, scales, draft_ids, R, T, V, H, logits_max, argmax_ids,
                         n_accepted, logits_out, workspace, workspace_bytes, stream);
}

int verify_lm_head_int4_batch_timed(const void *hidden, const uint8_t *packed_w,
                                    const void *scales, const int32_t *draft_ids, int R, int T,
                                    int V, int H, float *logits_max, int32_t *argmax_ids,
                                    int32_t *n_accepted, float *logits_out, void *workspace,
                                    size_t workspace_bytes, void *stream, void *event_before,
                                    void *event_after)
{
    return launch_verify(hidden, packed_w, scales, draft_ids, R, T, V, H, logits_max, argmax_ids,
                         n_accepted, logits_out, workspace, workspace_bytes, stream, event_before,
                         event_after);
}

int verify_lm_head_int4_batch_noalloc(const void *hidden, const uint8_t *packed_w, const void *scales,
                                      const int32_t *draft_ids, int R, int T, int V, int H,
                                      float *logits_max, int32_t *argmax_ids, int32_t *n_accepted,
                                      float *logits_out, void *stream)
{
    int st = validate_args(hidden, packed_w, scales, draft_ids, R, T, V, H, logits_max, argmax_ids,
                           n_accepted, logits_out);
    if (st != INT4VH_OK)
        return st;
    if (workspace_need(R, T, V, H) > kScratchBytes)
        return INT4VH_ESCRATCH;
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    const hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = nullptr;
    st = scratch_for_device(dev, s, &ws);
    if (st != INT4VH_OK)
        return st;
    st = launch_verify(hidden, packed_w, scales, draft_ids, R, T, V, H, logits_max, argmax_ids,
                       n_accepted, logits_out, ws, kScratchBytes, stream);
    if (st == INT4VH_EHIP)
        g_scratch[dev].zeroed.store(false, std::memory_order_release);   // zero again next time
    return st;
}

int verify_lm_head_int4_mapped(const void *hidden, const uint8_t *packed_w, const void *scales,
                               const int32_t *vocab_ids, const int32_t *draft_ids, int R, int T,
                               int V, int H, float *logits_max, int32_t *argmax_ids,
                               int32_t *n_accepted, float *logits_out, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    if (!vocab_ids)
        return INT4VH_EINVAL;
    return launch_verify(hidden, packed_w, scales, draft_ids, R, T, V, H, logits_max, argmax_ids,
                         n_accepted, logits_out, workspace, workspace_bytes, stream, nullptr,
                         nullptr, vocab_ids);
}

int verify_lm_head_int4_sampled_timed(const void *hidden, const uint8_t *packed_w,
                                      const void *scales, const int32_t *draft_ids,
                                      const float *draft_probs, const float *uniforms, int R, int T,
                                      int V, int H, int top_k, float temperature,
                                      float *logits_max, int32_t *argmax_ids, int32_t *topk_ids,
                                      float *topk_logits, float *lse, float *p_draft,
                                      int32_t *n_accepted, void *workspace, size_t workspace_bytes,
                                      void *stream, void *event_before, void *event_after)
{
    if (top_k < 0 || top_k > kMaxTopK || top_k > V || !(temperature > 0.0f) ||
        !(temperature < __builtin_huge_valf()))
        return INT4VH_EINVAL;
    if (top_k > 0 && (!topk_ids || !topk_logits))
        return INT4VH_EINVAL;
    if (T > 1 && (!draft_probs || !uniforms || !p_draft))
        return INT4VH_EINVAL;
    if ((topk_ids && !aligned(topk_ids, 4)) || (topk_logits && !aligned(topk_logits, 4)) ||
        (lse && !aligned(lse, 4)) || (draft_probs && !aligned(draft_probs, 4)) ||
        (uniforms && !aligned(uniforms, 4)) || (p_draft && !aligned(p_draft, 4)))
        return INT4VH_EALIGN;
    const Sampled smp{top_k, temperature, draft_probs, uniforms, topk_ids, topk_logits, p_draft, lse};
    if (R >= 1 && T >= 1 && (long long)R * T > kStreamMaxRows)
        return launch_sampled_rows(hidden, packed_w, scales, draft_ids, R, T, V, H, logits_max, argmax_ids,
                                   n_accepted, workspace, workspace_bytes, stream, event_before, event_after, smp);
    return launch_verify(hidden, packed_w, scales, draft_ids, R, T, V, H, logits_max, argmax_ids,
                         n_accepted, nullptr, workspace, workspace_bytes, stream, event_before,
                         event_after, nullptr, &smp);
}

int verify_lm_head_int4_sampled(const void *hidden, const uint8_t *packed_w, const void *scales,
                                const int32_t *draft_ids, const float *draft_probs,
                                const float *uniforms, int R, int T, int V, int H, int top_k,
                                float temperature, float *logits_max, int32_t *argmax_ids,
                                int32_t *topk_ids, float *topk_logits, float *lse, float *p_draft,
                                int32_t *n_accepted, void *workspace, size_t workspace_bytes,
                                void *stream)
{
    return verify_lm_head_int4_sampled_timed(hidden, packed_w, scales, draft_ids, draft_probs,
                                             uniforms, R, T, V, H, top_k, temperature, logits_max,
                                             argmax_ids, topk_ids, topk_logits, lse, p_draft,
                                             n_accepted, workspace, workspace_bytes, stream, nullptr,
                                             nullptr);
}

int verify_lm_head_int4_check_vocab_map(const int32_t *vocab_ids, int V, int32_t *n_bad_out,
                                        void *stream)
{
    if (!vocab_ids || !n_bad_out || V < 1)
        return INT4VH_EINVAL;
    if (!aligned(vocab_ids, 4) || !aligned(n_bad_out, 4))
        return INT4VH_EALIGN;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(fill_zero_u32, dim3(1), dim3(64), 0, s, reinterpret_cast<uint32_t *>(n_bad_out), 1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return hip_fail(e, "check_vocab_map zero launch");
    int blocks = (V + 255) / 256;
    if (blocks > 1024)
        blocks = 1024;
    hipLaunchKernelGGL(count_bad_map, dim3(blocks), dim3(256), 0, s, vocab_ids, V, n_bad_out);
    e = hipGetLastError();
    if (e != hipSuccess)
        return hip_fail(e, "check_vocab_map launch");
    return INT4VH_OK;
}

int verify_lm_head_int4_check_weights(const uint8_t *packed_w, int V, int H, int32_t *n_bad_out,
                                      void *stream)
{
    if (!packed_w || !n_bad_out || V < 1 || H < 32 || (H % 32) != 0)
        return INT4VH_EINVAL;
    if (!aligned(packed_w, 16) || !aligned(n_bad_out, 4))
        return INT4VH_EALIGN;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(fill_zero_u32, dim3(1), dim3(64), 0, s, reinterpret_cast<uint32_t *>(n_bad_out), 1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return hip_fail(e, "check_weights zero launch");
    const size_t n_vec = (size_t)V * (size_t)(H / 2) / 16;
    size_t blocks = (n_vec + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    hipLaunchKernelGGL(count_bad_nibbles, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const u32x4 *>(packed_w), n_vec, n_bad_out);
    e = hipGetLastError();
    if (e != hipSuccess)
        return hip_fail(e, "check_weights launch");
    return INT4VH_OK;
}

const char *verify_lm_head_int4_status_string(int status)
{
    switch (status) {
    case INT4VH_OK: return "ok";
    case INT4VH_EINVAL: return "invalid argument";
    case INT4VH_EALIGN: return "misaligned pointer";
    case INT4VH_EWORKSPACE: return "workspace too small";
    case INT4VH_EHIP: return "HIP runtime error";
    case INT4VH_EUNSUPPORTED: return "unsupported shape";
    case INT4VH_ESCRATCH: return "shape needs more than the static scratch of the no-allocation entry point";
    default: return "unknown status";
    }
}

const char *verify_lm_head_int4_last_error(void)
{
    return int4vh_detail::g_last_error.c_str();
}

} // extern "C"
