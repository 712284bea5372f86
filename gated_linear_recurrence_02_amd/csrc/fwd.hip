// fwd.hip -- a3..a5: decay, normalisation and the forward scan, with the conv
// and the gates optionally fused in front (modes A, B, C of rglru_scan_fwd).
//
// Page "Griffin Guide: RecurrentGemma, RG-LRU & Hybrid Attention",
// "Formulation of the RG-LRU Gating Mechanism": gates r, i; decay in log
// space, log a_t = -c r_t softplus(-Lambda); state update
// h_t = a_t h_{t-1} + sqrt(1 - a_t^2) (i_t x_t); output y_t = h_t.  The same
// page's "Custom Linear Scan Kernels" section describes fusing conv, gating,
// log-decay and the sequential state update into one kernel that keeps h on
// chip; mode A is that fusion written for CDNA4.
//
// Persistent kernel, one workgroup (8 waves) per CU.  Workgroup w serves the
// 256-channel block g = w % G; for bf16 the block's gate weights stay in
// registers for the whole launch (wave w holds W_a and W_x rows 32w..32w+31:
// 128 VGPRs).  Work units are chunks of 32 tokens of one stream, numbered
// chunk-major inside the block (unit q = c*B + b) and claimed at run time from
// the block's counter, one unit ahead, so the launch needs no co-residency
// guarantee and no cooperative launch.
//
// Per unit, lane l = 32*half + n of wave w owns channel d = 256g + 32w + n and
// the 16 consecutive tokens 32c + 16*half .. +15:
//   front  1. inputs: the conv over a 19-token window (mode A; interior bf16
//             chunks read a tile that global_load_lds brought into LDS one
//             unit ahead), x (mode B), or x, r, i (mode C, requested into
//             registers one unit ahead);
//          2. modes A/B: x goes to an LDS tile; the gate products come back in
//             the MFMA output layout, which hands the lane its 16 tokens of
//             channel d;
//          3. gates, decay, normalisation; local scan from h = 0 keeping the
//             running state and running decay product per token;
//          4. the halves combine across lanes l, l^32 into the unit's affine
//             aggregate (A, X), published right after the look-back of step
//             5 for the previous unit (at once if there is none);
//   back   5. one unit later: the unit's start state from the decoupled
//             look-back over earlier chunks of the same (b, g), its end state
//             published, and y_t = local state + running product * start
//             state stored.  In bf16 mode A the words that look-back reads
//             first were requested into LDS before the unit's gate products
//             (lb_prefetch), so a short walk usually finds them there.
// The running state and product of the unit waiting for its back half sit in
// LDS, so the look-back of unit j overlaps the front of the next unit.
//
// Forward progress: a workgroup processes its units in claim order, every
// wait is a look-back for a unit's start state, and it waits only for units
// of the same block with a smaller index, which were claimed earlier by
// running workgroups.  Take the smallest unit whose look-back has not ended:
// each unit it waits for has either published its end state already, or sits
// in a workgroup that is not waiting (any wait there would be for a still
// smaller unit), which goes on to publish that unit's aggregate and end state.
// So the smallest waiting look-back always ends, and by induction every one.
#include <stdlib.h>

#include <mutex>
#include <type_traits>

#include "common.h"
#include "gatemath.h"
#include "internal.h"

namespace rglru {

namespace {

constexpr int PSTRIDE = 36;   // floats per lane in the pending slot (b128, conflict-free)

// Staged input tile (bf16, mode A, interior chunks): tokens 32c-4 .. 32c+31 of
// the 256 channels of block g, written straight from global memory into LDS
// by global_load_lds_dwordx4 one chunk ahead.  One wave instruction moves two
// 512-byte rows (64 lanes x 16 bytes); blocks of two rows are padded to 1040
// bytes so that rows 16 apart fall in different LDS banks.
constexpr int ST_BLOCKS = 18, ST_BLK = 1040, ST_BYTES = ST_BLOCKS * ST_BLK;
// Mode 4: the branch-2 tile of a full chunk (tokens 32c .. 32c+31), same row
// layout, brought in while the chunk's front runs and read by its back half
constexpr int GT_BLOCKS = 16, GT_BYTES = GT_BLOCKS * ST_BLK;

__device__ __forceinline__ bool stageable(int c, int T) { return c > 0 && (c + 1) * CHUNK <= T; }

// OPQ: the lane's part of the address is rebuilt at every call instead of
// being computed once and kept live (as a 64-bit value) across the caller's
// loop, where it was spilled and its reload, waited for with every request in
// flight, stalled the issue of the next tile.  OPQ 1 hides the offset from
// the compiler, OPQ 2 the lane index it is computed from (modes 3 and 4,
// where the offset itself was still hoisted and spilled; there the block
// index also starts at the wave index taken as a scalar, so that the LDS
// addresses are scalar).
template <int NBLK = ST_BLOCKS, int OPQ = 0>
__device__ __forceinline__ void stage_issue(const bf16 *in, long row0, int D, int g, char *dst,
                                            int wave, int lane)
{
    int ln = lane;
    if constexpr (OPQ == 2) asm volatile("" : "+v"(ln));
    int loff = (ln >> 5) * D + (ln & 31) * 8;
    if constexpr (OPQ == 1) asm volatile("" : "+v"(loff));
    for (int i = OPQ == 2 ? __builtin_amdgcn_readfirstlane(wave) : wave; i < NBLK; i += 8) {
        const bf16 *src = OPQ != 0 ? in + (row0 + 2 * i) * D + g * 256 + loff
                              : in + (row0 + 2 * i + (lane >> 5)) * D + g * 256 + (lane & 31) * 8;
        __builtin_amdgcn_global_load_lds((const void *)src,
                                         (__attribute__((address_space(3))) void *)(dst + i * ST_BLK),
                                         16, 0, 0);
    }
}

// value of channel ch at staged row r (token 32c - 4 + r)
__device__ __forceinline__ float stage_read(const char *buf, int r, int ch)
{
    return (float)*(const bf16 *)(buf + (r >> 1) * ST_BLK + (r & 1) * 512 + ch * 2);
}

struct FwdParams {
    int B, T, D, NC, G, units;
    int lbp;   // mode A: prefetch the look-back words (walks expected to be short)
    float c;
    const void *in, *r, *i;
    const float *cw, *cb;
    const void *hist_in;
    const void *Wa, *Wx;
    const float *ba, *bx, *Lambda, *h0;
    void *y;
    float *h_last;
    void *hist_out;
    float *hstart_out;   // nullable: state before each chunk, [B][NC][D]
    void *ri_out;        // mode 3: r and i of every token in the backward's unit layout
    const void *gate_in; // mode 4: branch-2 pre-activation g; y becomes y * GeLU(g)
    WsHeader *hdr;
    uint32_t *claim;
    uint64_t *aggA, *aggX, *incl;
};

// Look-back prefetch (bf16 mode A).  Before a unit's gate products the
// wave asks the LDS-DMA path for the words the pending chunk's look-back reads
// first, for the wave's 32 channels: the inclusive states of chunks c-1, c-2
// and c-3 and both aggregate halves of c-1 and c-2.  They land in the wave's
// 2 KB slot while the products and the elementwise work run, so that the back
// half usually finds the start state there instead of paying a round trip to
// memory; a word not yet published when it was copied sends the lane to
// look_back.  Slot layout: array k at k * 256 bytes, channel n of the wave at
// n * 8 within it; k = 0..3 the inclusive states of chunks c-1 .. c-4 (c-4
// unused), k = 4, 5 the aggregate halves A, X of chunk c-1, k = 6, 7 those of
// chunk c-2.
constexpr int LBP_BYTES = 2048;

// Two DMA instructions of 16 bytes per lane (two channels' words): lanes
// 16q .. 16q+15 fill array q of the instruction's half of the slot.  The
// three word arrays sit one after another in the workspace (aggA, aggX,
// incl; see run_fwd), so both instructions read at one scalar base (stream b, the wave's channels) plus a
// 32-bit lane offset that is affine in q: q chunks back in the inclusive
// array, and aggregate half q & 1 of chunk c-1-(q >> 1).  The host enables
// the prefetch only when the three arrays span less than 2^31 bytes.  Chunks
// before the first read chunk 0 (in bounds; never used).  The words are read
// at agent coherence (sc1), as look_back reads them.
__device__ __forceinline__ void lb_prefetch(const FwdParams &p, int b, int c, int g, int wave, int lane,
                                            char *slot)
{
    // the lane's part is rebuilt at every call rather than kept live across
    // the caller's loop, where registers are short
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int q = ln >> 4;
    const uint32_t Db = (uint32_t)p.D * 8u;             // bytes per chunk row of one array
    const uint32_t nwb = (uint32_t)p.NC * (uint32_t)p.B * Db;   // bytes per array (aggA, aggX, incl)
    const uint32_t lo = (uint32_t)(ln & 15) * 16u;
    const uint32_t v1 = 2u * nwb + (uint32_t)max(c - 1 - q, 0) * Db + lo;
    const uint32_t v2 = (uint32_t)(q & 1) * nwb + (uint32_t)max(c - 1 - (q >> 1), 0) * Db + lo;
    const char *base = (const char *)(p.aggA + (long)b * p.NC * p.D + g * 256 + wave * 32);
    __builtin_amdgcn_global_load_lds((const void *)(base + v1), (__attribute__((address_space(3))) void *)slot, 16,
                                     0, 16);
    __builtin_amdgcn_global_load_lds((const void *)(base + v2),
                                     (__attribute__((address_space(3))) void *)(slot + 1024), 16, 0, 16);
}

// The state before the chunk after chunk k (k >= 0) from the prefetched
// words of channel n, when they reach back to a published inclusive state or
// to the sequence start; false sends the caller to look_back.  The fold is
// look_back's, term for term (aggregates applied oldest first with fmaf), so
// either way the result is the serial recurrence over chunk aggregates.
__device__ __forceinline__ bool lb_from_slot(const char *slot, int n, int k, float h_before_first,
                                             uint32_t tag, float &out)
{
    auto word = [&](int arr) { return *(const uint64_t *)(slot + arr * 256 + n * 8); };
    const uint64_t i1 = word(0);
    if (tagged(i1, tag)) {
        out = word_val(i1);
        return true;
    }
    const uint64_t a1 = word(4), x1 = word(5);
    if (!tagged(a1, tag) || !tagged(x1, tag)) return false;
    float s;
    if (k == 0) {
        s = h_before_first;
    } else {
        const uint64_t i2 = word(1);
        if (tagged(i2, tag)) {
            s = word_val(i2);
        } else {
            const uint64_t a2 = word(6), x2 = word(7);
            if (!tagged(a2, tag) || !tagged(x2, tag)) return false;
            float s2;
            if (k == 1) {
                s2 = h_before_first;
            } else {
                const uint64_t i3 = word(2);
                if (!tagged(i3, tag)) return false;
                s2 = word_val(i3);
            }
            s = fmaf(word_val(a2), s2, word_val(x2));
        }
    }
    out = fmaf(word_val(a1), s, word_val(x1));
    return true;
}

// Mode C: the x, r and i values of a lane's 16 tokens of unit q, as stored
// (requested one unit ahead and kept in registers until used); tokens past the
// end and channels past D read element 0 and are masked where used
template <typename T>
struct ScanIn {
    T x[16], r[16], i[16];
};

template <typename T>
__device__ __forceinline__ void scan_in_load(ScanIn<T> &v, const FwdParams &p, uint32_t q, int d, int half)
{
    const T *x = (const T *)p.in, *r = (const T *)p.r, *i = (const T *)p.i;
    const int c = (int)(q / p.B), b = (int)(q % p.B);
    const bool ok_unit = q < (uint32_t)p.units && d < p.D;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int t = c * CHUNK + 16 * half + k;
        const long e = (ok_unit && t < p.T) ? ((long)b * p.T + t) * p.D + d : 0;
        v.x[k] = x[e];
        v.r[k] = r[e];
        v.i[k] = i[e];
    }
}

// scalars of a chunk whose back half is pending
struct Pend {
    int b, c;
    float A0, X0;      // first half's product and local end state (as seen by half 1)
    float Ach, Xch;    // chunk aggregate (half 1 lanes)
};

template <typename T, int MODE>
__global__ __launch_bounds__(512) void fwd_kernel(FwdParams p)
{
    constexpr int S = XTile<T>::STRIDE;
    constexpr bool CONV = MODE == 0 || MODE == 3 || MODE == 4;   // conv fused in front
    constexpr bool RI = MODE == 3;                          // gate values stored
    constexpr bool MERGE = MODE == 4;                       // y * GeLU(g) stored instead of y
    constexpr bool WREG = (sizeof(T) == 2) && MODE != 2;   // weights held in registers
    constexpr bool STAGE = (sizeof(T) == 2) && CONV;        // input tile prefetched into LDS
    constexpr bool GTILE = STAGE && MERGE;                   // branch-2 tile staged too
    constexpr bool LBP = STAGE && MODE == 0;                 // look-back words prefetched
    extern __shared__ __attribute__((aligned(16))) char smem[];
    T *Xs = (T *)smem;
    float *pslot_base = (float *)(smem + (MODE == 2 ? 0 : 32 * S * sizeof(T)));
    char *stage_base = (char *)pslot_base + 512 * PSTRIDE * sizeof(float);

    // mode A takes the wave index as a scalar: wave-derived addresses then
    // live in scalar registers (fewer vector registers held across the loop)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = LBP ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
    const int n = lane & 31, half = lane >> 5;
    const int g = blockIdx.x % p.G;
    char *gt_base = stage_base + (STAGE ? 2 * ST_BYTES : 0);   // mode 4: two branch-2 tiles
    char *lbp_base = gt_base + (GTILE ? 2 * GT_BYTES : 0);   // look-back prefetch slots
    uint32_t *s_unit = (uint32_t *)(lbp_base + (LBP ? 8 * LBP_BYTES : 0));   // 2 claim slots, flag
    uint32_t *claim = p.claim + g;
    if (tid == 0) {
        s_unit[0] = claim_next(claim);
        s_unit[1] = claim_next(claim);
    }
    const int ch = wave * 32 + n;
    const int d = g * 256 + ch;
    const bool dv = d < p.D;
    const uint32_t tag = launch_tag(p.hdr);
    const T *in = (const T *)p.in;
    float *pslot = pslot_base + (wave * 64 + lane) * PSTRIDE;

    // per-channel constants
    float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 0.f, bias = 0.f;
    if (CONV && dv) {
        w0 = p.cw[4 * (long)d + 0];
        w1 = p.cw[4 * (long)d + 1];
        w2 = p.cw[4 * (long)d + 2];
        w3 = p.cw[4 * (long)d + 3];
        bias = p.cb ? p.cb[d] : 0.0f;
    }
    const float ncs = dv ? -p.c * softplus_acc(-p.Lambda[d]) : 0.0f;   // log a_t = ncs r_t
    const float bav = (MODE != 2 && dv && p.ba) ? p.ba[d] : 0.0f;
    const float bxv = (MODE != 2 && dv && p.bx) ? p.bx[d] : 0.0f;
    // fast-path forms: 2^(-log2e (z + b)) and 2^(log2e ncs r)
    const float kba = -LOG2E * bav, kbx = -LOG2E * bxv, kdec = LOG2E * ncs;
    // a_t = 2^(kdec r_t) with r_t = 1 / (1 + e_t) is 2^(1 / ((1 + e_t) / kdec)):
    // with 1 / kdec precomputed that is one FMA, no product.  A zero or tiny
    // kdec takes +-FLT_MAX, which still gives a_t = 1 (never 0 * inf)
    const float ikdec = kdec != 0.0f ? fminf(fmaxf(1.0f / kdec, -3.4e38f), 3.4e38f) : -3.4e38f;

    // gate weights of rows 32*wave .. +31 of block g, as MFMA B operands
    bf16x8 wa[WREG ? 16 : 1], wx[WREG ? 16 : 1];
    if constexpr (WREG) {
        const int r = lane & 31, kg = lane >> 5;
        const bf16 *pa = (const bf16 *)p.Wa + (size_t)g * 65536 + (size_t)(32 * wave + r) * 256 + 8 * kg;
        const bf16 *px = (const bf16 *)p.Wx + (size_t)g * 65536 + (size_t)(32 * wave + r) * 256 + 8 * kg;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            wa[s] = *(const bf16x8 *)(pa + 16 * s);
            wx[s] = *(const bf16x8 *)(px + 16 * s);
        }
    }

    const uint32_t units = (uint32_t)p.units;
    Pend pd = {0, 0, 0.f, 0.f, 0.f, 0.f};
    bool have_pend = false;
    // wave-uniform: some half-1 lane of this wave has a channel, so the wave
    // runs the back half's branch (and its wait for the tile requests)
    const bool half1_live = g * 256 + wave * 32 < p.D;
    // wave-uniform: the wave's 32 channels exist and their words are 16-byte
    // aligned, so the look-back words can be prefetched
    const bool lbp_ok = LBP && p.lbp && (p.D & 1) == 0 && g * 256 + wave * 32 + 32 <= p.D;
    char *lbp_slot = lbp_base + wave * LBP_BYTES;
    bool tile_waited = false;
    // Unit u_m of this workgroup travels through claim slot m & 1: thread 0
    // claims u_{n+2} at the start of iteration n and stores it later in the
    // iteration; every thread reads u_{n+1} after the first barrier of
    // iteration n.  The parity of n also selects the stage buffer.
    __syncthreads();
    uint32_t j = s_unit[0];
    uint32_t my_claim = 0xFFFFFFFFu;   // thread 0 only: the unit claimed this iteration
    int it = 0;
    ScanIn<T> sin;   // mode C: inputs of unit j
    if constexpr (MODE == 2) scan_in_load(sin, p, j, d, half);
    if constexpr (STAGE) {
        if (j < units) {
            const int c0 = (int)(j / p.B), b0 = (int)(j % p.B);
            if (stageable(c0, p.T))
                stage_issue<ST_BLOCKS, LBP ? 1 : 2>((const bf16 *)in, (long)b0 * p.T + (long)c0 * CHUNK - 4, p.D,
                                              g, stage_base, wave, lane);
        }
    }

    for (;;) {
        const bool have = j < units;
        if (!have && !have_pend) break;
        // thread 0 claims every iteration (a unit number past the last one
        // means no unit); only thread 0 writes the register, so no other wave
        // waits for the claim's return before reusing it
        if (tid == 0) my_claim = claim_next_late(claim);
        auto publish_claim = [&]() {   // u_{n+2}, read after the first barrier of the next iteration
            // every thread takes the value (only thread 0's is used) through an
            // empty asm, which keeps the wait for the claim's return here
            uint32_t v = my_claim;
            asm volatile("" : "+v"(v));
            if (tid == 0) s_unit[it & 1] = v;
        };

        float hl[16], P[16];
        Pend cur = {0, 0, 0.f, 0.f, 0.f, 0.f};
        bool lbp_pend = false;   // the pending chunk's look-back words were requested
        auto publish_agg = [&](const Pend &u) {   // half-1 lanes with a channel
            const long widx = ((long)u.b * p.NC + u.c) * p.D + d;
            put_word(p.aggA + widx, u.Ach, tag);
            put_word(p.aggX + widx, u.Xch, tag);
        };
        if constexpr (STAGE) {
            // this wave's tile requests have landed (waited for in the last
            // back half where one ran), and every wave's; the other stage
            // buffer, the x tile and the claim slot read last time are free
            // again.  The last back half's stores stay in flight.
            if (!tile_waited) __builtin_amdgcn_s_waitcnt(0);
            ds_barrier();
        } else {
            __syncthreads();
        }
        const uint32_t jn = s_unit[(it + 1) & 1];   // u_{n+1}
        ScanIn<T> sin_next;   // mode C: inputs of the next unit, requested now
        if constexpr (MODE == 2) scan_in_load(sin_next, p, jn, d, half);
        if (have) {
            // ------------------------------------------------ front of chunk j
            const int c = (int)(j / p.B), b = (int)(j % p.B);
            cur.b = b;
            cur.c = c;
            const long row_b = (long)b * p.T;
            const int tb = c * CHUNK + 16 * half;
            const bool full = (c + 1) * CHUNK <= p.T;
            float x[16];
            if (CONV) {
                float win[19];
                bool staged = false;
                if constexpr (STAGE) {
                    staged = stageable(c, p.T);
                    if (jn < units) {   // prefetch the next unit's tile
                        const int cn = (int)(jn / p.B), bn = (int)(jn % p.B);
                        if (stageable(cn, p.T))
                            stage_issue<ST_BLOCKS, LBP ? 1 : 2>((const bf16 *)in, (long)bn * p.T + (long)cn * CHUNK - 4,
                                                          p.D, g, stage_base + ((it + 1) & 1) * ST_BYTES, wave,
                                                          lane);
                    }
                    // this unit's branch-2 tile, read by its back half in the next iteration
                    if (GTILE && full)
                        stage_issue<GT_BLOCKS, 2>((const bf16 *)p.gate_in, row_b + (long)c * CHUNK, p.D, g,
                                                     gt_base + (it & 1) * GT_BYTES, wave, lane);
                }
                if (staged) {
                    const char *buf = stage_base + (it & 1) * ST_BYTES;
#pragma unroll
                    for (int m = 0; m < 19; ++m) win[m] = stage_read(buf, 16 * half + 1 + m, ch);
                } else if (full && c > 0 && dv) {
                    const T *src = in + (row_b + tb - 3) * p.D + d;
#pragma unroll
                    for (int m = 0; m < 19; ++m) win[m] = ldf(src + (long)m * p.D);
                } else {
#pragma unroll
                    for (int m = 0; m < 19; ++m) {
                        const int tau = tb - 3 + m;
                        float v = 0.0f;
                        if (dv && tau < p.T) {
                            if (tau >= 0) v = ldf(in + (row_b + tau) * p.D + d);
                            else if (p.hist_in)
                                v = ldf((const T *)p.hist_in + ((long)b * 3 + 3 + tau) * p.D + d);
                        }
                        win[m] = v;
                    }
                }
#pragma unroll
                for (int k = 0; k < 16; ++k)
                    x[k] = fmaf(w3, win[k + 3], fmaf(w2, win[k + 2], fmaf(w1, win[k + 1], fmaf(w0, win[k], bias))));
            } else if (MODE == 2) {
#pragma unroll
                for (int k = 0; k < 16; ++k) x[k] = (dv && tb + k < p.T) ? to_f32(sin.x[k]) : 0.0f;
            } else {
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const int t = tb + k;
                    x[k] = (dv && t < p.T) ? ldf(in + (row_b + t) * p.D + d) : 0.0f;
                }
            }

            float za[16], zx[16];
            if constexpr (MODE != 2) {
                if constexpr (sizeof(T) == 2) {   // two tokens per conversion
                    typedef __attribute__((ext_vector_type(2))) float f32x2v;
                    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v;
#pragma unroll
                    for (int k = 0; k < 16; k += 2) {
                        const bf16x2v pr = __builtin_convertvector(f32x2v{x[k], x[k + 1]}, bf16x2v);
                        Xs[(16 * half + k) * S + ch] = pr.x;
                        Xs[(16 * half + k + 1) * S + ch] = pr.y;
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < 16; ++k) Xs[(16 * half + k) * S + ch] = from_f32<T>(x[k]);
                }
                // orders the x tile only; the next unit's tile requests (into
                // the other stage buffer) and the last back half's stores stay
                // in flight
                ds_barrier();
                if constexpr (LBP) {
                    lbp_pend = lbp_ok && have_pend && pd.c > 0;
                    if (lbp_pend) lb_prefetch(p, pd.b, pd.c, g, wave, lane, lbp_slot);
                }
                if constexpr (WREG) {
                    const int r = lane & 31, kg = lane >> 5;
                    const bf16 *xrow = (const bf16 *)Xs + tile_row_token(r) * S + 8 * kg;
                    f32x16 A = {}, X = {};
#pragma unroll
                    for (int s = 0; s < 16; ++s) {
                        const bf16x8 av = *(const bf16x8 *)(xrow + 16 * s);
                        A = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, wa[s], A, 0, 0, 0);
                        X = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, wx[s], X, 0, 0, 0);
                    }
#pragma unroll
                    for (int k = 0; k < 16; ++k) {
                        za[k] = A[k];
                        zx[k] = X[k];
                    }
                } else {
                    gate_tile(Xs, (const T *)p.Wa + (size_t)g * 65536, (const T *)p.Wx + (size_t)g * 65536,
                              wave, lane, za, zx);
                }
            } else {
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const bool ok = dv && tb + k < p.T;
                    za[k] = ok ? to_f32(sin.r[k]) : 0.0f;
                    zx[k] = ok ? to_f32(sin.i[k]) : 0.0f;
                }
            }

            // u_{n+2} into its claim slot (read after the next iteration's
            // first barrier) now, while the wave has few memory operations in
            // flight: waiting for the claim's return later would also wait for
            // the stores issued after it
            if constexpr (STAGE) publish_claim();

            // gates, decay, normalisation, local scan from zero; interior
            // chunks take a copy of the loop without the end-of-sequence test
            using RT = typename GateStore<T>::rtype;
            RT rs[4];   // mode 3: r and i of 4 tokens, stored as they complete
            f32x4 is4;
            RT *r_dst = nullptr;
            float *i_dst = nullptr;
            if constexpr (RI) {   // d < D always holds here (D = 256 G)
                char *u0 = gate_store_unit<T>(p.ri_out, b, c, p.NC, p.G, g);
                r_dst = (RT *)u0;
                i_dst = (float *)(u0 + GateStore<T>::R_BYTES);
            }
            auto put_ri = [&](int k, float rr, float ii) {
                rs[k & 3] = (RT)rr;
                is4[k & 3] = ii;
                if ((k & 3) == 3) {
                    typedef __attribute__((__vector_size__(4 * sizeof(RT)))) RT rt4;
                    *(rt4 *)(r_dst + gate_off<RT>(ch, 16 * half + k - 3)) = rt4{rs[0], rs[1], rs[2], rs[3]};
                    *(f32x4 *)(i_dst + gate_off<float>(ch, 16 * half + k - 3)) = is4;
                }
            };
            auto scan16 = [&](auto edge_tag) {
                constexpr bool EDGE = decltype(edge_tag)::value;
                float h = 0.0f, pr = 1.0f;
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    float a, bb;
                    if constexpr (sizeof(T) == 2) {
                        float rr, ii;
                        if (MODE == 2) {
                            rr = za[k];
                            ii = zx[k];
                        } else if (RI) {
                            rr = hw_rcp(1.0f + hw_exp2(fmaf(za[k], -LOG2E, kba)));
                            ii = hw_rcp(1.0f + hw_exp2(fmaf(zx[k], -LOG2E, kbx)));
                        } else {   // r_t itself is not needed, only a_t
                            rr = 0.0f;
                            ii = hw_rcp(1.0f + hw_exp2(fmaf(zx[k], -LOG2E, kbx)));
                        }
                        if constexpr (RI) put_ri(k, rr, ii);
                        if (MODE == 2 || RI) a = hw_exp2(rr * kdec);
                        else {
                            const float er = hw_exp2(fmaf(za[k], -LOG2E, kba));
                            a = hw_exp2(hw_rcp(fmaf(er, ikdec, ikdec)));
                        }
                        bb = hw_sqrt(fmaf(-a, a, 1.0f)) * ii * x[k];
                    } else {
                        float rr, ii;
                        if (MODE == 2) {
                            rr = za[k];
                            ii = zx[k];
                        } else {
                            rr = sigmoid_acc(za[k] + bav);
                            ii = sigmoid_acc(zx[k] + bxv);
                        }
                        if constexpr (RI) put_ri(k, rr, ii);
                        const float l = ncs * rr;
                        a = expf(l);
                        bb = sqrtf(-expm1f(2.0f * l)) * ii * x[k];
                    }
                    if (EDGE && !(dv && tb + k < p.T)) {   // past the end: identity step
                        a = 1.0f;
                        bb = 0.0f;
                    }
                    h = fmaf(a, h, bb);
                    pr *= a;
                    hl[k] = h;
                    P[k] = pr;
                }
            };
            if (full && dv) scan16(std::false_type{});
            else scan16(std::true_type{});

            // chunk aggregate; published here only when no back half follows
            cur.A0 = __shfl_xor(P[15], 32);
            cur.X0 = __shfl_xor(hl[15], 32);
            cur.Ach = P[15] * cur.A0;
            cur.Xch = fmaf(P[15], cur.X0, hl[15]);
            if (!have_pend && half == 1 && dv) publish_agg(cur);
        }

        if (have_pend) {
            // ------------------------------------------- back of the pending chunk
            const int b = pd.b, c = pd.c;
            const long row_b = (long)b * p.T;
            const int tb = c * CHUNK + 16 * half;
            float hchunk = 0.0f;   // state before the chunk (half 1 lanes)
            if (half == 1 && dv) {
                const long base = (long)b * p.NC * p.D + d;
                const long widx = base + (long)c * p.D;
                const float hbefore = p.h0 ? p.h0[(long)b * p.D + d] : 0.0f;
                bool got = c == 0;
                hchunk = hbefore;
                if constexpr (LBP) {
                    if (!got && lbp_pend) {
                        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));   // the slot has landed
                        got = lb_from_slot(lbp_slot, n, c - 1, hbefore, tag, hchunk);
                    }
                }
                if (!got)
                    hchunk = look_back(p.aggA + base, p.aggX + base, p.incl + base, c - 1, p.D, hbefore, tag,
                                       p.hdr);
                // the tile requests of this iteration's front were issued before
                // the look-back's loads, so this wait costs little
                if constexpr (STAGE) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
                // the current unit's aggregate goes out after the look-back's
                // loads: issued before them, these stores would have had to
                // complete before the loads could be waited for
                if (have) publish_agg(cur);
                put_word(p.incl + widx, fmaf(pd.Ach, hchunk, pd.Xch), tag);
                if (p.hstart_out) p.hstart_out[widx] = hchunk;
            }
            const float hother = __shfl_xor(hchunk, 32);
            const float hstart = half == 0 ? hother : fmaf(pd.A0, hchunk, pd.X0);
            float yl[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 vh = *(const f32x4 *)(pslot + 4 * q);
                const f32x4 vp = *(const f32x4 *)(pslot + 16 + 4 * q);
#pragma unroll
                for (int e = 0; e < 4; ++e) yl[4 * q + e] = fmaf(vp[e], hstart, vh[e]);
            }
            float zl[16];   // what is stored: y, or y * GeLU(g) in mode 4
            if constexpr (MERGE) {
                float gv[16];
                if (GTILE && (c + 1) * CHUNK <= p.T) {   // staged during the chunk's front
                    // the lane's offset is rebuilt here rather than kept live
                    // across the loop, where registers are short
                    int off = ((it + 1) & 1) * GT_BYTES + half * 8 * ST_BLK + ch * 2;
                    asm volatile("" : "+v"(off));
                    const char *buf = gt_base + off;
#pragma unroll
                    for (int k = 0; k < 16; ++k)
                        gv[k] = (float)*(const bf16 *)(buf + (k >> 1) * ST_BLK + (k & 1) * 512);
                } else {
                    const T *gp = (const T *)p.gate_in + (row_b + tb) * p.D + d;
#pragma unroll
                    for (int k = 0; k < 16; ++k) gv[k] = (dv && tb + k < p.T) ? ldf(gp + (long)k * p.D) : 0.0f;
                }
#pragma unroll
                for (int k = 0; k < 16; ++k) zl[k] = yl[k] * gelu_exact(gv[k]);
            } else {
#pragma unroll
                for (int k = 0; k < 16; ++k) zl[k] = yl[k];
            }
            T *y = (T *)p.y;
            if (y && dv) {
                T *dst = y + (row_b + tb) * p.D + d;
                if ((c + 1) * CHUNK <= p.T) {
                    if constexpr (sizeof(T) == 2) {
                        // two tokens per conversion (the pair's halves go to two rows)
                        typedef __attribute__((ext_vector_type(2))) float f32x2v;
                        typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v;
#pragma unroll
                        for (int k = 0; k < 16; k += 2) {
                            const bf16x2v pr = __builtin_convertvector(f32x2v{zl[k], zl[k + 1]}, bf16x2v);
                            dst[(long)k * p.D] = pr.x;
                            dst[(long)(k + 1) * p.D] = pr.y;
                        }
                    } else {
#pragma unroll
                        for (int k = 0; k < 16; ++k) dst[(long)k * p.D] = from_f32<T>(zl[k]);
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < 16; ++k)
                        if (tb + k < p.T) dst[(long)k * p.D] = from_f32<T>(zl[k]);
                }
            }
            if (c == p.NC - 1 && dv) {
                if (half == 1 && p.h_last) p.h_last[(long)b * p.D + d] = yl[15];
                if (CONV && half == 0 && p.hist_out) {
                    for (int jj = 0; jj < 3; ++jj) {
                        const int pos = p.T - 3 + jj;
                        T v = from_f32<T>(0.0f);
                        if (pos >= 0) v = in[(row_b + pos) * p.D + d];
                        else if (p.hist_in) v = ((const T *)p.hist_in)[((long)b * 3 + 3 + pos) * p.D + d];
                        ((T *)p.hist_out)[((long)b * 3 + jj) * p.D + d] = v;
                    }
                }
            }
        }

        if (have) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                *(f32x4 *)(pslot + 4 * q) = f32x4{hl[4 * q], hl[4 * q + 1], hl[4 * q + 2], hl[4 * q + 3]};
                *(f32x4 *)(pslot + 16 + 4 * q) = f32x4{P[4 * q], P[4 * q + 1], P[4 * q + 2], P[4 * q + 3]};
            }
            pd = cur;
        }
        tile_waited = have_pend && half1_live;
        have_pend = have;
        if constexpr (MODE == 2) sin = sin_next;
        if (!STAGE || !have) publish_claim();
        j = jn;
        ++it;
    }
    __syncthreads();
    finish_claimed(p.hdr, p.claim, p.G, s_unit + 2);
}

template <typename T, int MODE>
size_t fwd_lds_bytes()
{
    const bool stage = sizeof(T) == 2 && (MODE == 0 || MODE == 3 || MODE == 4);
    const bool gtile = sizeof(T) == 2 && MODE == 4;
    const bool lbp = stage && MODE == 0;
    return (MODE == 2 ? 0 : 32 * XTile<T>::STRIDE * sizeof(T)) + 512 * PSTRIDE * sizeof(float) +
           (stage ? 2 * ST_BYTES : 0) + (gtile ? 2 * GT_BYTES : 0) + (lbp ? 8 * LBP_BYTES : 0) + 16;
}

// Per device: CU count and resident workgroups per CU of one kernel, looked
// up once (the attribute call and the occupancy query cost host time).
struct LaunchShape {
    int ncu = 0, occ = 0;
};

template <typename T, int MODE>
LaunchShape fwd_shape()
{
    static std::mutex mu;
    static LaunchShape cache[64];
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev < 0 || dev >= 64) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    LaunchShape &ls = cache[dev];
    if (ls.ncu == 0) {
        const void *fn = (const void *)&fwd_kernel<T, MODE>;
        const size_t shmem = fwd_lds_bytes<T, MODE>();
        int ncu = 0, occ = 0;
        // failures here surface through the launch and hipGetLastError
        (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
        (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, 512, shmem);
        ls.ncu = ncu < 1 ? 1 : ncu;
        ls.occ = occ < 1 ? 1 : occ;
    }
    return ls;
}

template <typename T, int MODE>
void launch_mode(FwdParams p, hipStream_t s)
{
    static_assert(32 * 260 * 4 + 512 * PSTRIDE * 4 + 16 <= 160 * 1024, "LDS budget (fp32)");
    static_assert(32 * 264 * 2 + 512 * PSTRIDE * 4 + 2 * ST_BYTES + 2 * GT_BYTES + 16 <= 160 * 1024,
                  "LDS budget (bf16, mode 4)");
    static_assert(32 * 264 * 2 + 512 * PSTRIDE * 4 + 2 * ST_BYTES + 8 * LBP_BYTES + 16 <= 160 * 1024,
                  "LDS budget (bf16, mode A)");
    const LaunchShape ls = fwd_shape<T, MODE>();
    // workgroups per block: fill the resident slots, never more than the units;
    // RGLRU_FWD_GROUP_WORKGROUPS (a positive integer) caps the count, which
    // changes nothing in the results (work is claimed in order at run time)
    long wpg = ((long)ls.ncu * ls.occ) / p.G;
    if (const char *cap = getenv("RGLRU_FWD_GROUP_WORKGROUPS")) {
        const long c = atol(cap);
        if (c > 0 && c < wpg) wpg = c;
    }
    if (wpg < 1) wpg = 1;
    if (wpg > p.units) wpg = p.units;
    const long grid = (long)p.G * wpg;
    const size_t shmem = fwd_lds_bytes<T, MODE>();
    // A block's workgroups hold about wpg consecutive units, wpg / B chunks of
    // each stream; the prefetch reaches 3 chunks back, so it pays only when
    // few chunks of a stream are in flight together (a lone 32k-token stream
    // has ~25 in flight and its walks are long); it addresses the three word
    // arrays by 32-bit offsets, so they must span less than 2^31 bytes
    p.lbp = wpg <= 4L * p.B && 3 * (size_t)p.B * p.NC * p.D * sizeof(uint64_t) < ((size_t)1 << 31);
    fwd_kernel<T, MODE><<<dim3((unsigned)grid), dim3(512), shmem, s>>>(p);
}

template <typename T>
void launch_t(const FwdParams &p, int mode, hipStream_t s)
{
    if (mode == 0) launch_mode<T, 0>(p, s);
    else if (mode == 1) launch_mode<T, 1>(p, s);
    else if (mode == 2) launch_mode<T, 2>(p, s);
    else if (mode == 3) launch_mode<T, 3>(p, s);
    else launch_mode<T, 4>(p, s);
}

void run_fwd(const rglru_desc &d, const rglru_weights &w, int mode, const void *in, const void *r,
             const void *i, const void *hist_in, const float *h0, void *y, float *h_last,
             void *hist_out, float *hstart_out, void *ri_out, const void *gate_in, void *ws,
             hipStream_t s)
{
    FwdParams p;
    p.B = (int)d.B;
    p.T = (int)d.T;
    p.D = (int)d.D;
    p.NC = (int)((d.T + CHUNK - 1) / CHUNK);
    p.G = (int)((d.D + 255) / 256);
    p.units = p.B * p.NC;
    p.c = d.c;
    p.in = in;
    p.r = r;
    p.i = i;
    p.cw = w.conv_w;
    p.cb = w.conv_b;
    p.hist_in = hist_in;
    p.Wa = w.W_a;
    p.Wx = w.W_x;
    p.ba = w.b_a;
    p.bx = w.b_x;
    p.Lambda = w.Lambda;
    p.h0 = h0;
    p.y = y;
    p.h_last = h_last;
    p.hist_out = hist_out;
    p.hstart_out = hstart_out;
    p.ri_out = ri_out;
    p.gate_in = gate_in;
    p.hdr = (WsHeader *)ws;
    p.claim = (uint32_t *)((char *)ws + sizeof(WsHeader));
    const size_t nw = (size_t)d.B * p.NC * d.D;
    p.aggA = (uint64_t *)((char *)ws + sizeof(WsHeader) + CLAIM_REGION_BYTES);
    p.aggX = p.aggA + nw;
    p.incl = p.aggX + nw;
    if (d.io == RGLRU_BF16) launch_t<bf16>(p, mode, s);
    else launch_t<float>(p, mode, s);
}

}  // namespace

size_t fwd_workspace_bytes(int64_t B, int64_t T, int64_t D)
{
    const int64_t NC = (T + CHUNK - 1) / CHUNK, G = (D + 255) / 256;
    (void)G;
    return sizeof(WsHeader) + CLAIM_REGION_BYTES + 3 * (size_t)B * NC * D * sizeof(uint64_t);
}

void launch_scan_fwd(const rglru_desc &d, const rglru_weights &w, int mode, const void *in,
                     const void *r, const void *i, const void *hist_in, const float *h0, void *y,
                     float *h_last, void *hist_out, void *ws, hipStream_t s)
{
    if (mode == 0 && fused_fwd_applies(d)) {
        launch_fused_fwd(d, w, in, hist_in, h0, y, h_last, hist_out, ws, s);
        return;
    }
    run_fwd(d, w, mode, in, r, i, hist_in, h0, y, h_last, hist_out, nullptr, nullptr, nullptr, ws, s);
}

void launch_fwd_states(const rglru_desc &d, const rglru_weights &w, const void *u,
                       const void *hist_in, const float *h0, float *hstart_out, void *ri_out,
                       void *ws, hipStream_t s)
{
    run_fwd(d, w, 3, u, nullptr, nullptr, hist_in, h0, nullptr, nullptr, nullptr, hstart_out, ri_out, nullptr,
            ws, s);
}

void launch_scan_fwd_merge(const rglru_desc &d, const rglru_weights &w, const void *u, const void *g,
                           const void *hist_in, const float *h0, void *z, float *h_last, void *hist_out,
                           void *ws, hipStream_t s)
{
    run_fwd(d, w, 4, u, nullptr, nullptr, hist_in, h0, z, h_last, hist_out, nullptr, nullptr, g, ws, s);
}

}  // namespace rglru
