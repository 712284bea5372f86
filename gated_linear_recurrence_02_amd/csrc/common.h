// common.h -- device helpers shared by the RG-LRU kernels (gfx950 only).
//
// Layout conventions are those of include/rglru.h.  Activation storage is
// either float or clang's native __bf16 (bf16 <-> f32 conversions compile to
// a shift and to v_cvt_pk_bf16_f32, which rounds to nearest even).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/rglru.h"
#include "internal.h"

namespace rglru {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

template <typename T> __device__ __forceinline__ float ldf(const T *p) { return to_f32(*p); }

// ------------------------------------------------------------- chunk carries
// The scan over T is split into chunks of CHUNK tokens.  Each chunk publishes
// its affine aggregate (A, X) -- the map h_in -> A h_in + X it applies to the
// state -- and, once known, its inclusive end state.  A chunk finds its start
// state by walking back over published words (decoupled look-back).  Every
// word is 64 bits: the low half holds the fp32 value, the high half a tag that
// is unique to the launch, so a word is either absent or complete and no
// memory fence is needed.  Stale words from earlier launches carry another tag.
//
// The workspace starts with a header of counters; the last workgroup of a
// launch resets the counters and advances the epoch, so a zero-filled
// workspace stays reusable.
struct WsHeader {
    uint32_t counter;   // unused
    uint32_t done;      // workgroups finished
    uint32_t epoch;     // launches completed
    uint32_t error;     // set if a look-back wait ever gave up
    uint32_t counter2;  // unused
    uint32_t done2;     // unused
    uint32_t done8[8];  // per-XCD-slot finish counters of persistent launches
    uint32_t pad[50];
};
static_assert(sizeof(WsHeader) == 256, "header is 256 bytes");
static_assert(offsetof(WsHeader, error) == WS_ERROR_OFFSET, "timeout word where the host reads it");

constexpr int CHUNK = 32;               // tokens per chunk (one 32-row MFMA tile)
constexpr uint32_t SPIN_LIMIT = 1u << 22;

__device__ __forceinline__ uint32_t tag_of_epoch(uint32_t e) { return (e & 0x7FFFFFFFu) | 0x80000000u; }

__device__ __forceinline__ void put_word(uint64_t *p, float v, uint32_t tag)
{
    const uint64_t w = ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool get_word(const uint64_t *p, uint32_t tag, float &v)
{
    const uint64_t w = __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    v = __uint_as_float((uint32_t)w);
    return (uint32_t)(w >> 32) == tag;
}

// Workgroup barrier that orders LDS only: the fences are restricted to the
// local address space, so the barrier waits for this wave's LDS operations
// (lgkmcnt) but not for its global stores and loads in flight (a plain
// __syncthreads() also drains vmcnt, i.e. waits for every outstanding store
// to reach memory and for every prefetch to land).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup barrier for LDS written by ds_* instructions only.  In a kernel
// that also fills LDS through global_load_lds, the compiler's local-memory
// fences wait for every vector memory operation (such a fill completes with
// vmcnt), and __syncthreads() does as well; both would stall on stores and
// requests meant to stay in flight.  This form waits for the wave's LDS
// operations and keeps the compiler from moving memory accesses across it;
// LDS that a global_load_lds fills may be read after it only once every
// wave has waited for that fill (s_waitcnt vmcnt) before the barrier.
__device__ __forceinline__ void ds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8): every LDS operation done and at most N vector memory
// operations outstanding
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// Every atomic here is relaxed on purpose: no data is published through the
// counters (each carry word holds its own tag, outputs are read only after
// the kernel ends), and acquire/release at agent scope would write back and
// invalidate the whole L2 on every call.

// Walk back from chunk `k` (the chunk just before the caller's) to the newest
// chunk j <= k whose inclusive (end) state is published, passing over chunks
// whose aggregate is published; chunk -1's end state is `h_before_first`.
// Words are indexed base + k * stride; chunks are numbered in the order the
// scan runs (a reverse scan numbers them from the end of the sequence).
// Returns the state at the end of chunk k.
//
// The result is the same whatever the walk finds, bit for bit: every
// inclusive state is the serial recurrence over chunk aggregates,
//     e(-1) = h_before_first,   e(m) = fma(A_m, e(m-1), X_m),
// and the aggregates of chunks j+1 .. k are folded onto e(j) forward, in chunk
// order, with the same fma, so the same operations run on the same values
// however far back the walk had to go (a look-back that composed the
// aggregates backward would group the products differently from run to run).
//
// The words of LB_BATCH predecessors are loaded together.  When the walk ends
// inside the first round, the aggregates are already in registers; later
// rounds take LB_WIDE chunks and load only the tag halves of their
// aggregates, and a longer walk then loads the aggregates' values for the
// fold, eight chunks per round trip (they are published, so these loads
// return the published values).  The walk only waits on chunks that were handed out before the
// caller's chunk, so it ends once their aggregates are published; a wait
// that exceeds SPIN_LIMIT flags the header and returns NaN rather than
// hanging.  Two chunks per round: the words of one round stay in registers
// across the wait, and at 4 chunks (24 registers) the fused forward measured
// 3% slower at 2B width and 2% at 32k tokens (1 chunk: 1% slower than 2); by
// the time a chunk's back half runs, its predecessor has usually published
// its inclusive state.
constexpr int LB_BATCH = 2;
constexpr int LB_WIDE = 3;   // chunks per later round (tag halves of the aggregates only)

__device__ __forceinline__ uint64_t load_word(const uint64_t *p)
{
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// the tag half of a word (the high 32 bits)
__device__ __forceinline__ uint32_t load_tag(const uint64_t *p)
{
    return __hip_atomic_load((uint32_t *)const_cast<uint64_t *>(p) + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// the value half of a word already known to be published
__device__ __forceinline__ float load_value(const uint64_t *p)
{
    return __uint_as_float(__hip_atomic_load((uint32_t *)const_cast<uint64_t *>(p), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT));
}

__device__ __forceinline__ bool tagged(uint64_t w, uint32_t tag) { return (uint32_t)(w >> 32) == tag; }
__device__ __forceinline__ float word_val(uint64_t w) { return __uint_as_float((uint32_t)w); }

__device__ __forceinline__ float look_back(const uint64_t *aggA, const uint64_t *aggX,
                                           const uint64_t *incl, long k, long stride,
                                           float h_before_first, uint32_t tag, WsHeader *hdr)
{
    uint32_t spins = 0;
    // chunk indices and the stride fit 32 bits: one 32x32->64 multiply-add
    // per chunk word offset instead of a full 64-bit product
    const uint32_t st = (uint32_t)stride;
    long j = k;                  // newest chunk not yet walked over
    long jf = -1;                // chunk whose inclusive state starts the fold
    float base = h_before_first;
    while (j >= 0) {
        int passed = 0;          // chunks of this round walked over
        bool done = false;
        if (j == k) {
            // a round at the caller's predecessor: whole words, so that a
            // walk ending here folds the aggregates in hand
            uint64_t wi[LB_BATCH], wa[LB_BATCH], wx[LB_BATCH];
#pragma unroll
            for (int q = 0; q < LB_BATCH; ++q) {
                const int kk = max((int)j - q, 0);
                const uint64_t o = (uint64_t)(uint32_t)kk * st;
                wi[q] = load_word(incl + o);
                wa[q] = load_word(aggA + o);
                wx[q] = load_word(aggX + o);
            }
#pragma unroll
            for (int q = 0; q < LB_BATCH; ++q) {
                if (done || passed != q) continue;   // an earlier slot ended the round
                if (j - q < 0) {
                    done = true;                     // reached the start: fold onto h_before_first
                } else if (tagged(wi[q], tag)) {
                    done = true;
                    jf = j - q;
                    base = word_val(wi[q]);
                } else if (tagged(wa[q], tag) && tagged(wx[q], tag)) {
                    ++passed;
                }
            }
            if (!done && j - passed < 0) done = true;   // passed chunk 0
            if (done) {   // short walk: the aggregates to fold are in hand
                float s = base;
#pragma unroll
                for (int q = LB_BATCH - 1; q >= 0; --q)   // chunks k - q, oldest first
                    if (q < passed) s = fmaf(word_val(wa[q]), s, word_val(wx[q]));
                return s;
            }
        } else {
            // later rounds: LB_WIDE chunks, of the aggregates only the tag
            // halves (their values are loaded by the fold below)
            uint64_t wi[LB_WIDE];
            uint32_t ta[LB_WIDE], tx[LB_WIDE];
#pragma unroll
            for (int q = 0; q < LB_WIDE; ++q) {
                const int kk = max((int)j - q, 0);
                const uint64_t o = (uint64_t)(uint32_t)kk * st;
                wi[q] = load_word(incl + o);
                ta[q] = load_tag(aggA + o);
                tx[q] = load_tag(aggX + o);
            }
#pragma unroll
            for (int q = 0; q < LB_WIDE; ++q) {
                if (done || passed != q) continue;
                if (j - q < 0) {
                    done = true;
                } else if (tagged(wi[q], tag)) {
                    done = true;
                    jf = j - q;
                    base = word_val(wi[q]);
                } else if (ta[q] == tag && tx[q] == tag) {
                    ++passed;
                }
            }
            if (!done && j - passed < 0) done = true;
            if (done) break;
        }
        j -= passed;
        if (passed == 0) {
            // chunk j has not published yet: every chunk publishes its aggregate
            // before its inclusive state, so poll that one word before reloading
            while (!tagged(load_word(aggX + (uint64_t)(uint32_t)j * st), tag)) {
                if (++spins > SPIN_LIMIT) {
                    __hip_atomic_store(&hdr->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    return __builtin_nanf("");
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
    }
    // a walk longer than the first round: fold chunks jf+1 .. k, 8 at a time.
    // Their words are published and never change again within the launch,
    // so only the value halves (the low 32 bits) are loaded
    float s = base;
    for (long m = jf + 1; m <= k; m += 8) {
        float a8[8], x8[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint64_t o = (uint64_t)(uint32_t)min(m + q, k) * st;
            a8[q] = load_value(aggA + o);
            x8[q] = load_value(aggX + o);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (m + q <= k) s = fmaf(a8[q], s, x8[q]);
    }
    return s;
}

// Finish of a persistent launch: workgroups count themselves in one of 8
// counters (blockIdx % 8), the last of each group in the top counter, and the
// very last one resets them and advances the epoch.  Spreading the count over
// 8 addresses keeps the end-of-launch atomics from queueing on one address.
__device__ __forceinline__ void finish_persistent(WsHeader *hdr)
{
    if (threadIdx.x == 0) {
        const uint32_t nwg = gridDim.x, grp = blockIdx.x & 7u;
        const uint32_t in_grp = (nwg - grp + 7u) / 8u;
        const uint32_t prev = __hip_atomic_fetch_add(&hdr->done8[grp], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (prev == in_grp - 1u) {
            __hip_atomic_store(&hdr->done8[grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t ngrp = nwg < 8u ? nwg : 8u;
            const uint32_t p2 = __hip_atomic_fetch_add(&hdr->done, 1u, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
            if (p2 == ngrp - 1u) {
                __hip_atomic_store(&hdr->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_fetch_add(&hdr->epoch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// Work claimed at run time.  Kernels launched without a co-residency
// guarantee take their work units from per-group counters (relaxed
// fetch-add, one thread per workgroup) and process them in claim order; a
// unit only ever waits on units claimed before it, by workgroups that are
// already running, so every wait ends whatever the number of resident
// workgroups.  The counters live in the workspace after the header.
__device__ __forceinline__ uint32_t claim_next(uint32_t *ctr)
{
    return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The same claim with the counter's address passed through a vector
// register.  LLVM's atomic optimizer rewrites atomics on a uniform address
// into one wave-wide operation whose result is read at once, and that read
// waits for every vector memory operation the wave issued before the atomic
// (its stores included).  With the address in a VGPR the rewrite does not
// apply and the result is waited for only where it is used.
__device__ __forceinline__ uint32_t claim_next_late(uint32_t *ctr)
{
    uintptr_t a = (uintptr_t)ctr;
    asm volatile("" : "+v"(a));
    // a global (not flat) atomic: a flat one would also count against lgkmcnt
    // and hold up the wave's LDS waits until it returns
    typedef __attribute__((address_space(1))) uint32_t global_u32;
    return __hip_atomic_fetch_add((global_u32 *)a, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// End of a launch whose work was claimed from `nclaims` counters: called by
// every thread after a __syncthreads.  Workgroups count themselves as in
// finish_persistent; the last one zeroes the claim counters (all threads of
// it) and advances the epoch.  `s_flag` is one word of LDS.
__device__ __forceinline__ void finish_claimed(WsHeader *hdr, uint32_t *claims, int nclaims,
                                               uint32_t *s_flag)
{
    if (threadIdx.x == 0) {
        uint32_t last = 0;
        const uint32_t nwg = gridDim.x, grp = blockIdx.x & 7u;
        const uint32_t in_grp = (nwg - grp + 7u) / 8u;
        const uint32_t prev = __hip_atomic_fetch_add(&hdr->done8[grp], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (prev == in_grp - 1u) {
            __hip_atomic_store(&hdr->done8[grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t ngrp = nwg < 8u ? nwg : 8u;
            const uint32_t p2 = __hip_atomic_fetch_add(&hdr->done, 1u, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
            last = p2 == ngrp - 1u;
        }
        *s_flag = last;
    }
    __syncthreads();
    if (*s_flag) {
        for (int i = threadIdx.x; i < nclaims; i += blockDim.x)
            __hip_atomic_store(&claims[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (threadIdx.x == 0) {
            __hip_atomic_store(&hdr->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(&hdr->epoch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// The claim counters sit in a region of fixed size right after the header,
// one 32-bit counter per group, for up to MAX_CLAIM_GROUPS groups.  Its size
// does not depend on the shape, so the carry words of one call can never
// land where a later call of another shape keeps its counters: a forward
// workspace serves calls of any shape.
constexpr size_t CLAIM_REGION_BYTES = (size_t)MAX_CLAIM_GROUPS * 4;

// Element `e` of an array whose base is the same for the whole wave: the
// 32-bit byte offset lets the compiler use scalar-base addressing.
template <typename T> __device__ __forceinline__ T *at(T *base, uint32_t e)
{
    return (T *)((char *)base + e * (uint32_t)sizeof(T));
}

__device__ __forceinline__ uint32_t launch_tag(WsHeader *hdr)
{
    return tag_of_epoch(__hip_atomic_load(&hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// ---------------------------------------------------------------------- math
// Fast forms on the hardware transcendentals (v_exp_f32 = 2^x, v_rcp_f32,
// v_sqrt_f32, each within about 1 ulp) for bf16 I/O, where the output rounding
// (2^-9) dominates; accurate device-library calls for fp32 I/O.
constexpr float LOG2E = 1.4426950408889634f;
__device__ __forceinline__ float hw_exp2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float hw_rcp(float v) { return __builtin_amdgcn_rcpf(v); }
__device__ __forceinline__ float hw_sqrt(float v) { return __builtin_amdgcn_sqrtf(v); }

// Accurate fp32 helpers (device-library calls).
__device__ __forceinline__ float sigmoid_acc(float z) { return 1.0f / (1.0f + expf(-z)); }
__device__ __forceinline__ float softplus_acc(float v)
{
    return v > 0.0f ? v + log1pf(expf(-v)) : log1pf(expf(v));
}

// Gate values r and i that the backward's state pass keeps for every token.
// r is stored in fp16 for bf16 I/O (it lies in (0, 1), where fp16 resolves
// 2^-11 relative), i always in fp32: the gradient of u is sensitive enough
// to i that fp16 i doubles its error.  Per 32-token unit (stream b, chunk c)
// and 256-channel block g: [(b NC + c) G + g] { r block, i block }.  Inside a
// block (element type E, V = 16 / sizeof(E) values per 16-byte piece),
// token t of channel ch sits in piece (t / 16, (t % 16) / V) of channel ch:
// pieces are ordered (half, piece, channel), so the lanes of a wave, which
// hold consecutive channels, touch consecutive 16-byte pieces.
template <typename T> struct GateStore {
    using rtype = float;
    static constexpr size_t R_BYTES = 256 * 32 * sizeof(rtype);    // r block of a unit
    static constexpr size_t UNIT_BYTES = R_BYTES + 256 * 32 * 4;   // r and i blocks
};
template <> struct GateStore<bf16> {
    using rtype = _Float16;
    static constexpr size_t R_BYTES = 256 * 32 * sizeof(rtype);
    static constexpr size_t UNIT_BYTES = R_BYTES + 256 * 32 * 4;
};
// start of unit (b, c), block g
template <typename T>
__device__ __forceinline__ char *gate_store_unit(void *base, int b, int c, int NC, int G, int g)
{
    return (char *)base + ((size_t)((long)b * NC + c) * G + g) * GateStore<T>::UNIT_BYTES;
}
// element offset of token t (0..31) of channel ch inside a block of type E
template <typename E> __device__ __forceinline__ uint32_t gate_off(int ch, int t)
{
    constexpr int V = 16 / sizeof(E);
    return (uint32_t)((((t >> 4) * (16 / V) + ((t & 15) / V)) * 256 + ch) * V + (t % V));
}

// GeLU(v) = v Phi(v) = 0.5 v (1 + erf(v / sqrt 2)), the exact form, with erfc
// from Abramowitz & Stegun, Handbook of Mathematical Functions (1964), eq.
// 7.1.26 (|error| <= 1.5e-7): for x >= 0, erfc(x) = p(s) s e^(-x^2),
// s = 1 / (1 + 0.3275911 x), p of degree 4.  With h = erfc(|v| / sqrt 2) / 2,
// v Phi(v) = max(v, 0) - |v| h on both sides of zero (Phi(-w) = erfc(w / sqrt 2) / 2),
// so the left tail has no cancellation; h's polynomial carries the 1/2.
__device__ __forceinline__ float gelu_exact(float v)
{
    const float a = fabsf(v);
    const float s = hw_rcp(fmaf(0.2316418883f, a, 1.0f));   // 0.3275911 / sqrt 2
    float p = fmaf(0.5307027145f, s, -0.7265760135f);
    p = fmaf(p, s, 0.7107068705f);
    p = fmaf(p, s, -0.142248368f);
    p = fmaf(p, s, 0.127414796f);
    const float h = p * s * hw_exp2((v * v) * -0.72134752044448170f);   // e^(-v^2 / 2)
    return fmaf(-a, h, fmaxf(v, 0.0f));
}

// Token held by row `r` of a 32-row MFMA tile.  The 32x32 output tile gives
// lane l the column l%32 and the rows 8j + 4(l/32) + i (register 4j + i);
// mapping row 8j + 4h + i to token 16h + 4j + i makes register k of lane l
// hold token 16(l/32) + k, so every lane owns 16 consecutive tokens.
__device__ __forceinline__ int tile_row_token(int r) { return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }

}  // namespace rglru
