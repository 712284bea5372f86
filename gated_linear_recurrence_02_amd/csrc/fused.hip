// fused.hip -- the fused forward of rglru_scan_fwd mode A for bf16 I/O
// (conv + block-diagonal gates + log-space decay + chunked scan, u -> y in one
// kernel), written so that one wave per SIMD keeps its matrix cores and its
// vector ALU busy at the same time.
//
// Page "Griffin Guide: RecurrentGemma, RG-LRU & Hybrid Attention": the
// causal depthwise conv of width 4 ("Temporal Filtering via Separable 1D
// Convolutions"), the gates r_t = sigma(W_a x_t + b_a), i_t = sigma(W_x x_t +
// b_x) with block-diagonal W ("Block-Diagonal Sharding for Zero-Communication
// Tensor Parallelism"), log a_t = -c r_t softplus(-Lambda) and
// h_t = a_t h_{t-1} + sqrt(1 - a_t^2) i_t x_t, y_t = h_t ("Formulation of the
// RG-LRU Gating Mechanism"), fused in one kernel that keeps h on chip ("Custom
// Linear Scan Kernels (Pallas and Triton)").
//
// Layout of the work.  One workgroup of 4 waves per CU, one wave per SIMD;
// workgroup w serves the 256-channel block g = w % G.  Wave v owns the 64
// output channels 64v .. 64v+63 of the block and holds their rows of W_a and
// W_x as MFMA B operands for the whole launch (256 registers, which the
// compiler keeps in the accumulation registers).  Lane l = 32 half + n owns
// channels 64v + n and 64v + 32 + n (q = 0, 1) and the 16 tokens
// 16 half .. 16 half + 15 of the current 32-token chunk.  Work units are
// chunks of one stream, numbered chunk-major inside the block (unit
// m = c B + b) and claimed at run time from the block's counter.
//
// Pipeline.  Iteration n handles four consecutive units of the workgroup:
//   F = u_n      gate products (v_mfma_f32_32x32x16_bf16, 16 K steps x 2
//                gates x 2 channel tiles) and the elementwise work (gates,
//                decay, normalisation, local scan from h = 0 keeping the
//                running state and decay product), its chunk aggregate
//                published once the back half's look-back has resolved;
//   C = u_{n+1}  the conv from the staged input tile, into the x tile of the
//                next iteration's gate products (bf16) and into registers
//                (fp32, for the next iteration's b = beta i x);
//   P = u_{n+2}  input tile requested into LDS (global_load_lds);
//   u_{n-1}      back half: the start state from the look-back (its first
//                loads issued after the conv, consumed after the elementwise
//                work), y = local state + product * start state,
//                stored with buffer stores whose row offsets are scalars.
// The products of F are issued between the conv's and the elementwise
// work's vector instructions; a wave's own MFMAs then run while its vector
// ALU works (measured: together about 1.1x the vector work alone, against
// 1.3x for MFMA and FMA waves sharing a SIMD).  One barrier per iteration:
// x tiles, stage tiles and claim slots are double or quadruple buffered.
//
// Forward progress: every wait is for a unit of the same block with a
// smaller index than the unit being resolved, claimed earlier by a running
// workgroup (one workgroup per CU, all resident), and before a workgroup
// publishes a unit's aggregate it waits only on units with smaller indices
// still.  The unpublished unit of smallest index therefore always gets its
// aggregate out.
//
// Opt-in (RGLRU_FWD_FUSED=1): measured slower than the 8-wave kernel of
// fwd.hip at the prefill shapes (the vector work of one wave per SIMD leaves
// the look-back latency exposed), kept as a second, independently written
// implementation of mode A.
#include <stdlib.h>

#include <mutex>

#include "common.h"
#include "internal.h"

namespace rglru {

namespace {

constexpr int FX_STRIDE = 256 + 8;                      // x tile row (bf16): 528 bytes
constexpr int FX_BYTES = 32 * FX_STRIDE * 2;            // one x tile
// Staged input tile, one slab per wave and a single buffer: tokens 32c-4 ..
// 32c+31 (36 rows) of the wave's 64 channels, 128 bytes per row.  Each
// global_load_lds moves 8 rows (64 lanes x 16 bytes) into a 1 KB block;
// blocks are 1088 bytes apart, so the rows 16 apart that the two lane halves
// of the conv read together lie 32 banks apart.  5 blocks; rows 36..39 of the
// last one repeat row 35.  A wave reads only its own slab, so it refills it
// right after its conv with no barrier.
constexpr int FSB_STRIDE = 1088, FSB_BLOCKS = 5;
constexpr int FS_WAVE = FSB_STRIDE * FSB_BLOCKS;
constexpr int FS_BYTES = 4 * FS_WAVE;
// Pending slot of a lane: per channel the local states of its 16 tokens in
// fp32 (64 bytes) then their decay products in fp16 (32 bytes), 208-byte
// stride so that the 16-byte accesses of 16 lanes cover the 64 banks once;
// two buffers, one written by the current unit while the other is read
constexpr int F_PBYTES = 208;
constexpr int F_PSLOTS = 256 * F_PBYTES;
constexpr size_t F_LDS = 2 * FX_BYTES + FS_BYTES + 2 * F_PSLOTS + 32;
static_assert(F_LDS <= 160 * 1024, "LDS budget");
constexpr uint32_t RSRC_WORD3 = 0x00020000;             // raw buffer, 32-bit words (gfx9)
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

struct FusedParams {
    int B, T, D, NC, G, units;
    const bf16 *u;
    const float *cw, *cb;
    const bf16 *hist_in;
    const bf16 *Wa, *Wx;
    const float *ba, *bx, *Lambda, *h0;
    bf16 *y;
    float *h_last;
    bf16 *hist_out;
    float c;
    uint32_t y_bytes;   // B T D 2 (below 2^31)
    WsHeader *hdr;
    uint32_t *claim;
    uint64_t *aggA, *aggX, *incl;
};

__device__ __forceinline__ bool fstageable(int c, int T) { return c > 0 && (c + 1) * CHUNK <= T; }

// Input tile of unit (b, c) into the wave's slab: lane l loads 16 bytes of
// row 8 i + l / 8, channels 64 wave + 8 (l % 8) .. +7
__device__ __forceinline__ void fstage_issue(const bf16 *u, long row0, int D, int g, char *slab, int wave,
                                             int lane)
{
    const int r = lane >> 3, col = 64 * wave + 8 * (lane & 7);
#pragma unroll
    for (int i = 0; i < FSB_BLOCKS; ++i) {
        const int row = min(8 * i + r, 35);
        const bf16 *src = u + (row0 + row) * D + g * 256 + col;
        __builtin_amdgcn_global_load_lds((const void *)src,
                                         (__attribute__((address_space(3))) void *)(slab + i * FSB_STRIDE), 16, 0, 0);
    }
}

// value of the wave's channel chw (0..63) at staged row r (token 32c - 4 + r)
__device__ __forceinline__ float fstage_read(const char *slab, int r, int chw)
{
    return (float)*(const bf16 *)(slab + (r >> 3) * FSB_STRIDE + (r & 7) * 128 + chw * 2);
}

// Gate products with the weight operand in accumulation registers.  The
// compiler's MFMA builtin takes its B operand from ordinary VGPRs only, which
// would copy 4 registers per product out of the AGPRs every time; written out,
// the instruction reads B from AGPRs directly and accumulates in VGPRs.
// The compiler does not see the matrix-core hazards of these statements, so
// they carry their own wait states: 2 before each product (for a vector-ALU
// write of an operand just before it) and 20 after the last product of a chain,
// more than the 18 a 16-pass MFMA result needs before a vector-ALU read.
// Every call site accumulates into a chain of its own.
__device__ __forceinline__ void mfma_first(f32x16 &c, const bf16x8 &a, const bf16x8 &w)
{
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(c) : "v"(a), "a"(w));
}
__device__ __forceinline__ void mfma_next(f32x16 &c, const bf16x8 &a, const bf16x8 &w)
{
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(w));
}
__device__ __forceinline__ void mfma_last(f32x16 &c, const bf16x8 &a, const bf16x8 &w)
{
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 3"
        : "+v"(c) : "v"(a), "a"(w));
}
// one channel tile of both gates: 16 K steps, the A operand (16 bytes of one
// x tile row per lane) read from LDS once per step and used by both gates
__device__ __forceinline__ void tile_products(f32x16 &ca, f32x16 &cx, const bf16 *xf, const bf16x8 (&wA)[16],
                                              const bf16x8 (&wX)[16])
{
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        const bf16x8 av = *(const bf16x8 *)(xf + 16 * s);
        if (s == 0) {
            mfma_first(ca, av, wA[s]);
            mfma_first(cx, av, wX[s]);
        } else if (s == 15) {
            mfma_last(ca, av, wA[s]);
            mfma_last(cx, av, wX[s]);
        } else {
            mfma_next(ca, av, wA[s]);
            mfma_next(cx, av, wX[s]);
        }
    }
}

struct FPend {
    int b, c;
    float Ach, Xch;     // aggregate of the lane's look-back channel (q = half)
    float A0[2], X0[2]; // first-half aggregates of both channels (used by half-1 lanes)
};

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void fused_fwd_kernel(FusedParams p)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    bf16 *xtiles = (bf16 *)smem;
    char *stages = smem + 2 * FX_BYTES;
    char *pslots = stages + FS_BYTES;
    uint32_t *s_unit = (uint32_t *)(pslots + 2 * F_PSLOTS);   // 4 claim slots, 1 flag

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    char *slab = stages + wave * FS_WAVE;   // this wave's staged input tile
    const int n = lane & 31, half = lane >> 5;
    const int g = blockIdx.x % p.G;
    const int B = p.B, T = p.T, D = p.D;
    const uint32_t units = (uint32_t)p.units;
    uint32_t *claim = p.claim + g;

    if (tid == 0) {
        s_unit[0] = claim_next(claim);
        s_unit[1] = claim_next(claim);
    }

    // per-channel constants of the lane's two channels
    int cbk[2], dd[2];
    float w0[2], w1[2], w2[2], w3[2], bias[2], kba[2], kbx[2], ikdec[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        cbk[q] = 64 * wave + 32 * q + n;
        dd[q] = g * 256 + cbk[q];
        const f32x4 t4 = *(const f32x4 *)(p.cw + 4 * (long)dd[q]);
        w0[q] = t4[0];
        w1[q] = t4[1];
        w2[q] = t4[2];
        w3[q] = t4[3];
        bias[q] = p.cb ? p.cb[dd[q]] : 0.0f;
        // fast forms: i = 1 / (1 + 2^(-log2e (z + b_x))); a = 2^(kdec r) with
        // r = 1 / (1 + e) is 2^(1 / ((1 + e) / kdec)), one FMA with 1/kdec
        kba[q] = -LOG2E * (p.ba ? p.ba[dd[q]] : 0.0f);
        kbx[q] = -LOG2E * (p.bx ? p.bx[dd[q]] : 0.0f);
        const float kdec = LOG2E * (-p.c * softplus_acc(-p.Lambda[dd[q]]));
        // a zero or tiny kdec takes +-FLT_MAX, which still gives a = 1
        ikdec[q] = kdec != 0.0f ? fminf(fmaxf(1.0f / kdec, -3.4e38f), 3.4e38f) : -3.4e38f;
    }
    // gate weights: tile t (channels 64 wave + 32 t + n), K step s
    bf16x8 wa[2][16], wx[2][16];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const size_t row = (size_t)g * 65536 + (size_t)(64 * wave + 32 * t + n) * 256 + 8 * half;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            wa[t][s] = *(const bf16x8 *)(p.Wa + row + 16 * s);
            wx[t][s] = *(const bf16x8 *)(p.Wx + row + 16 * s);
            asm volatile("" : "+a"(wa[t][s]));   // kept in accumulation registers
            asm volatile("" : "+a"(wx[t][s]));
        }
    }
    const uint32_t tag = launch_tag(p.hdr);
    const __amdgpu_buffer_rsrc_t yres = __builtin_amdgcn_make_buffer_rsrc(p.y, 0, (int)p.y_bytes, RSRC_WORD3);
    // byte offset of the lane's first token row and channel, per channel
    const int yv[2] = {2 * (16 * half * D + dd[0]), 2 * (16 * half * D + dd[1])};
    const int xr = tile_row_token(n) * FX_STRIDE + 8 * half;   // A-operand row of the lane

    __syncthreads();
    uint32_t uF = 0xFFFFFFFFu, uC = s_unit[0], uP = s_unit[1];
    // the first tile, read by the first iteration's conv
    if (uC < units) {
        const int c0 = (int)(uC / B), b0 = (int)(uC % B);
        if (fstageable(c0, T))
            fstage_issue(p.u, (long)b0 * T + (long)c0 * CHUNK - 4, D, g, slab, wave, lane);
    }
    float xcur[2][16];   // fp32 conv output of F
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int k = 0; k < 16; ++k) xcur[q][k] = 0.0f;
    FPend pd = {0, 0, 0.f, 0.f, {0.f, 0.f}, {0.f, 0.f}};
    bool have_pend = false, stored = false;

    for (int it = 0;; ++it) {   // iteration n = it - 1
        const bool fv = uF < units, cv = uC < units;
        if (!fv && !cv && !have_pend) break;
        // This wave's tile loads for C (issued last iteration) must have
        // landed.  Vector memory operations complete in issue order; after a
        // full back half the last 32 of them are that chunk's y stores, so
        // waiting until at most 32 are outstanding covers the tile while the
        // stores drain.  Otherwise wait for everything.
        if (stored) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(32));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
        lds_barrier();
        uint32_t my_claim;   // u_{n+3}, written to its slot at the end of the iteration
        if (tid == 0) my_claim = claim_next(claim);
        if (it > 0) uP = s_unit[(it + 1) & 3];
        const int fb = it & 1, cb = (it + 1) & 1;   // x tile buffers of F and C
        // ----------------------------------------- gate products of F, conv of C
        // Two blocks without branches interleave the 64 products of F with
        // vector work: tile 0 with the conv of C (when C's tile is staged),
        // tile 1 with the elementwise work of F's channel 0 (when F is a full
        // chunk).  Other cases take the plain order below.
        f32x16 accA[2], accX[2];
        const bf16 *xf = xtiles + fb * (FX_BYTES / 2) + xr;
        float xnext[2][16];
        const int cC = (int)(uC / B), bC = (int)(uC % B);
        bf16 *xc = xtiles + cb * (FX_BYTES / 2) + (16 * half) * FX_STRIDE;
        auto conv_pair = [&](int q, const float (&win)[19], int kp) {
            const int k = 2 * kp;
            const float x0 = fmaf(w3[q], win[k + 3], fmaf(w2[q], win[k + 2], fmaf(w1[q], win[k + 1], fmaf(w0[q], win[k], bias[q]))));
            const float x1 = fmaf(w3[q], win[k + 4], fmaf(w2[q], win[k + 3], fmaf(w1[q], win[k + 2], fmaf(w0[q], win[k + 1], bias[q]))));
            xnext[q][k] = x0;
            xnext[q][k + 1] = x1;
            typedef __attribute__((ext_vector_type(2))) float f32x2v;
            typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v;
            const bf16x2v pr = __builtin_convertvector(f32x2v{x0, x1}, bf16x2v);
            xc[k * FX_STRIDE + cbk[q]] = pr.x;
            xc[(k + 1) * FX_STRIDE + cbk[q]] = pr.y;
        };
        auto conv_window_staged = [&](int q, float (&win)[19]) {
#pragma unroll
            for (int m = 0; m < 19; ++m) win[m] = fstage_read(slab, 16 * half + 1 + m, 32 * q + n);
        };
        if (fv && cv && fstageable(cC, T)) {
            float win0[19], win1[19];
            conv_window_staged(0, win0);
            bf16x8 avb[3];
            avb[0] = *(const bf16x8 *)xf;
#pragma unroll
            for (int s2 = 0; s2 < 16; ++s2) {
                if (s2 + 1 < 16) avb[(s2 + 1) % 3] = *(const bf16x8 *)(xf + 16 * (s2 + 1));
                if (s2 == 0) {
                    mfma_first(accA[0], avb[0], wa[0][0]);
                    mfma_first(accX[0], avb[0], wx[0][0]);
                } else if (s2 == 15) {
                    mfma_last(accA[0], avb[s2 % 3], wa[0][s2]);
                    mfma_last(accX[0], avb[s2 % 3], wx[0][s2]);
                } else {
                    mfma_next(accA[0], avb[s2 % 3], wa[0][s2]);
                    mfma_next(accX[0], avb[s2 % 3], wx[0][s2]);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (s2 == 4) conv_window_staged(1, win1);
                if (s2 < 8) conv_pair(0, win0, s2);
                else conv_pair(1, win1, s2 - 8);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            if (fv) tile_products(accA[0], accX[0], xf, wa[0], wx[0]);
            if (cv) {
                const int tb = cC * CHUNK + 16 * half;
                const long row_b = (long)bC * T;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    float win[19];
                    if (fstageable(cC, T)) {
                        conv_window_staged(q, win);
                    } else {
#pragma unroll
                        for (int m = 0; m < 19; ++m) {
                            const int tau = tb - 3 + m;
                            float v = 0.0f;
                            if (tau < T) {
                                if (tau >= 0) v = (float)p.u[(row_b + tau) * D + dd[q]];
                                else if (p.hist_in) v = (float)p.hist_in[((long)bC * 3 + 3 + tau) * D + dd[q]];
                            }
                            win[m] = v;
                        }
                    }
#pragma unroll
                    for (int kp = 0; kp < 8; ++kp) conv_pair(q, win, kp);
                }
            }
        }

        // The conv has read the slab (every read consumed); refill it with P's
        // tile, read by the next iteration's conv
        if (uP < units) {
            const int cp = (int)(uP / B), bp = (int)(uP % B);
            if (fstageable(cp, T)) {
                __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
                fstage_issue(p.u, (long)bp * T + (long)cp * CHUNK - 4, D, g, slab, wave, lane);
            }
        }

        // First round of the pending unit's look-back, for the lane's look-back
        // channel (q = half): end states and aggregates of chunks c-1 and c-2
        // and the end state of chunk c-3, requested once the products of F
        // are under way and used by the back half, after F's elementwise work.
        // (not initialised: writing the registers would first wait for the
        // previous iteration's loads into them; they are read only on the
        // route that loads them)
        uint64_t lw_i[3], lw_a[2], lw_x[2];
        const long lbase = have_pend ? ((long)pd.b * p.NC) * D + dd[half] : 0;
        if (have_pend && pd.c > 0) {
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const uint64_t o = lbase + (uint64_t)(uint32_t)max(pd.c - 1 - j, 0) * (uint32_t)D;
                lw_i[j] = load_word(p.incl + o);
                if (j < 2) {
                    lw_a[j] = load_word(p.aggA + o);
                    lw_x[j] = load_word(p.aggX + o);
                }
            }
        }

        // -------------------------------------------- elementwise work of F
        FPend cur = {0, 0, 0.f, 0.f, {0.f, 0.f}, {0.f, 0.f}};
        float hend[2] = {0.f, 0.f}, pend[2] = {1.f, 1.f};   // the lane's local end state and product
        if (fv) {
            const int cF = (int)(uF / B), bF = (int)(uF % B);
            cur.b = bF;
            cur.c = cF;
            const int nv = min(max(T - (cF * CHUNK + 16 * half), 0), 16);   // valid tokens of the lane
            char *pw = pslots + (it & 1) * F_PSLOTS + tid * F_PBYTES;
            float th[8], tp[8];   // states and products of the current 8-token group
            // gates, decay, normalisation and the local scan of token k of channel q;
            // every 8 tokens the group goes to the pending slot (fp16, toward zero)
            auto token = [&](int q, int k, float zak, float zxk, bool edge) {
                const float er = hw_exp2(fmaf(zak, -LOG2E, kba[q]));
                float a = hw_exp2(hw_rcp(fmaf(er, ikdec[q], ikdec[q])));
                const float ii = hw_rcp(1.0f + hw_exp2(fmaf(zxk, -LOG2E, kbx[q])));
                float bb = hw_sqrt(fmaf(-a, a, 1.0f)) * ii * xcur[q][k];
                if (edge && k >= nv) {   // past the end of the sequence: identity step
                    a = 1.0f;
                    bb = 0.0f;
                }
                hend[q] = fmaf(a, hend[q], bb);
                pend[q] *= a;
                th[k & 7] = hend[q];
                tp[k & 7] = pend[q];
                if ((k & 7) == 7) {
                    typedef __attribute__((ext_vector_type(2))) float f32x2v;
                    typedef __attribute__((ext_vector_type(2))) _Float16 f16x2v;
                    u32x4 pv;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        pv[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{tp[2 * e], tp[2 * e + 1]}, f16x2v));
                    char *pq = pw + 96 * q;
                    *(f32x4 *)(pq + 32 * (k >> 3)) = f32x4{th[0], th[1], th[2], th[3]};
                    *(f32x4 *)(pq + 32 * (k >> 3) + 16) = f32x4{th[4], th[5], th[6], th[7]};
                    *(u32x4 *)(pq + 64 + 16 * (k >> 3)) = pv;
                }
            };
            if ((cF + 1) * CHUNK <= T) {
                bf16x8 avb[3];
                avb[0] = *(const bf16x8 *)xf;
#pragma unroll
                for (int s2 = 0; s2 < 16; ++s2) {
                    if (s2 + 1 < 16) avb[(s2 + 1) % 3] = *(const bf16x8 *)(xf + 16 * (s2 + 1));
                    if (s2 == 0) {
                        mfma_first(accA[1], avb[0], wa[1][0]);
                        mfma_first(accX[1], avb[0], wx[1][0]);
                    } else if (s2 == 15) {
                        mfma_last(accA[1], avb[s2 % 3], wa[1][s2]);
                        mfma_last(accX[1], avb[s2 % 3], wx[1][s2]);
                    } else {
                        mfma_next(accA[1], avb[s2 % 3], wa[1][s2]);
                        mfma_next(accX[1], avb[s2 % 3], wx[1][s2]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    token(0, s2, accA[0][s2], accX[0][s2], false);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int k = 0; k < 16; ++k) token(1, k, accA[1][k], accX[1][k], false);
            } else {
                tile_products(accA[1], accX[1], xf, wa[1], wx[1]);
#pragma unroll
                for (int k = 0; k < 16; ++k) token(0, k, accA[0][k], accX[0][k], true);
#pragma unroll
                for (int k = 0; k < 16; ++k) token(1, k, accA[1][k], accX[1][k], true);
            }
            // chunk aggregates: the halves combine across lanes l, l ^ 32
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const float oA = __shfl_xor(pend[q], 32), oX = __shfl_xor(hend[q], 32);
                const float fA = half ? oA : pend[q], fX = half ? oX : hend[q];
                const float sA = half ? pend[q] : oA, sX = half ? hend[q] : oX;
                cur.A0[q] = fA;
                cur.X0[q] = fX;
                if (q == half) {
                    cur.Ach = sA * fA;
                    cur.Xch = fmaf(sA, fX, sX);
                }
            }
        }
        // F's aggregate is published after the pending unit's look-back has
        // used its words: the words were requested before these stores, but
        // using them would otherwise wait for the stores too (vector memory
        // operations complete in order).  Waiting first is safe: the look-back
        // waits only on units with smaller indices than the pending unit, whose
        // index is smaller than F's.
        auto publish_f = [&]() {
            if (fv) {
                const long widx = ((long)cur.b * p.NC + cur.c) * D + dd[half];
                put_word(p.aggA + widx, cur.Ach, tag);
                put_word(p.aggX + widx, cur.Xch, tag);
            }
        };

        // ----------------------------------------- back half of u_{n-1}
        stored = false;
        if (!have_pend) publish_f();   // otherwise right after the look-back below
        if (have_pend) {
            const int b = pd.b, c = pd.c;
            float hchunk;
            // the state before the first chunk, loaded only on the routes that use it
            auto h_before = [&]() { return p.h0 ? p.h0[(long)b * D + dd[half]] : 0.0f; };
            if (c == 0) {
                hchunk = h_before();
            } else {
                // the first round's words, then the full walk if needed; every
                // route is the serial fold over chunk aggregates (look_back)
                const int k = c - 1;
                bool ok = false;
                hchunk = 0.0f;
                // newest published end state among chunks k, k-1, k-2 (or the
                // state before chunk 0), then the aggregates after it folded on
                // in chunk order
                const bool a0 = tagged(lw_a[0], tag) && tagged(lw_x[0], tag);
                const bool a1 = tagged(lw_a[1], tag) && tagged(lw_x[1], tag);
                if (tagged(lw_i[0], tag)) {
                    hchunk = word_val(lw_i[0]);
                    ok = true;
                } else if (a0 && (k == 0 || tagged(lw_i[1], tag))) {
                    const float s = k == 0 ? h_before() : word_val(lw_i[1]);
                    hchunk = fmaf(word_val(lw_a[0]), s, word_val(lw_x[0]));
                    ok = true;
                } else if (a0 && a1 && k >= 1 && (k == 1 || tagged(lw_i[2], tag))) {
                    const float s = k == 1 ? h_before() : word_val(lw_i[2]);
                    hchunk = fmaf(word_val(lw_a[0]), fmaf(word_val(lw_a[1]), s, word_val(lw_x[1])), word_val(lw_x[0]));
                    ok = true;
                }
                if (!ok)
                    hchunk = look_back(p.aggA + lbase, p.aggX + lbase, p.incl + lbase, k, D, h_before(), tag, p.hdr);
            }
            const float hend_lb = fmaf(pd.Ach, hchunk, pd.Xch);   // state at the chunk's end
            put_word(p.incl + lbase + (long)c * D, hend_lb, tag);
            publish_f();
            const float hother = __shfl_xor(hchunk, 32);
            float hst[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const float hc = q == half ? hchunk : hother;
                hst[q] = half ? fmaf(pd.A0[q], hc, pd.X0[q]) : hc;
            }
            const char *prd = pslots + ((it + 1) & 1) * F_PSLOTS + tid * F_PBYTES;
            float yl[2][16];
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int k8 = 0; k8 < 2; ++k8) {
                    const char *pq = prd + 96 * q;
                    const f32x4 h0v = *(const f32x4 *)(pq + 32 * k8), h1v = *(const f32x4 *)(pq + 32 * k8 + 16);
                    const u32x4 vp = *(const u32x4 *)(pq + 64 + 16 * k8);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        // products of tokens 8 k8 + 2e (low half) and + 1 (high half)
                        const uint32_t pw2 = vp[e];
                        const float plo = (float)__builtin_bit_cast(_Float16, (uint16_t)(pw2 & 0xFFFFu));
                        const float phi = (float)__builtin_bit_cast(_Float16, (uint16_t)(pw2 >> 16));
                        const float hlo = e < 2 ? h0v[2 * e] : h1v[2 * e - 4];
                        const float hhi = e < 2 ? h0v[2 * e + 1] : h1v[2 * e - 3];
                        yl[q][8 * k8 + 2 * e] = fmaf(plo, hst[q], hlo);
                        yl[q][8 * k8 + 2 * e + 1] = fmaf(phi, hst[q], hhi);
                    }
                }
            const int soff0 = 2 * (((b * T) + c * CHUNK) * D);   // row 32c of stream b, in bytes
            typedef __attribute__((ext_vector_type(2))) float f32x2v;
            typedef __attribute__((ext_vector_type(2))) unsigned short u16x2v;
            if ((c + 1) * CHUNK <= T) {
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int k = 0; k < 16; k += 2) {
                        const u16x2v pr = __builtin_bit_cast(
                            u16x2v, __builtin_convertvector(f32x2v{yl[q][k], yl[q][k + 1]},
                                                            __attribute__((ext_vector_type(2))) __bf16));
                        __builtin_amdgcn_raw_buffer_store_b16(pr.x, yres, yv[q], soff0 + 2 * k * D, 0);
                        __builtin_amdgcn_raw_buffer_store_b16(pr.y, yres, yv[q], soff0 + 2 * (k + 1) * D, 0);
                    }
                stored = true;
            } else {
                const int nv = min(max(T - (c * CHUNK + 16 * half), 0), 16);
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int k = 0; k < 16; ++k)
                        if (k < nv)
                            __builtin_amdgcn_raw_buffer_store_b16(
                                __builtin_bit_cast(unsigned short, (bf16)yl[q][k]), yres, yv[q], soff0 + 2 * k * D, 0);
            }
            if (c == p.NC - 1) {
                // the carried state in fp32: the end state of the look-back channel
                if (p.h_last) p.h_last[(long)b * D + dd[half]] = hend_lb;
                if (half == 0 && p.hist_out) {
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        for (int jj = 0; jj < 3; ++jj) {
                            const int pos = T - 3 + jj;
                            bf16 v = (bf16)0.0f;
                            if (pos >= 0) v = p.u[((long)b * T + pos) * D + dd[q]];
                            else if (p.hist_in) v = p.hist_in[((long)b * 3 + 3 + pos) * D + dd[q]];
                            p.hist_out[((long)b * 3 + jj) * D + dd[q]] = v;
                        }
                }
            }
        }

        // ------------------------------------------------ hand over
        if (fv) pd = cur;
        have_pend = fv;
        if (cv) {
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int k = 0; k < 16; ++k) xcur[q][k] = xnext[q][k];
        }
        if (tid == 0) s_unit[(it + 2) & 3] = my_claim;   // u_{n+3}
        uF = uC;
        uC = uP;
    }
    __syncthreads();
    finish_claimed(p.hdr, p.claim, p.G, s_unit + 4);
}

struct FShape {
    int ncu = 0;
};

FShape fused_shape()
{
    static std::mutex mu;
    static FShape cache[64];
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev < 0 || dev >= 64) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    FShape &fs = cache[dev];
    if (fs.ncu == 0) {
        int ncu = 0;
        // failures here surface through the launch and hipGetLastError
        (void)hipFuncSetAttribute((const void *)&fused_fwd_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)F_LDS);
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
        fs.ncu = ncu < 1 ? 1 : ncu;
    }
    return fs;
}

}  // namespace

bool fused_fwd_applies(const rglru_desc &d)
{
    if (d.io != RGLRU_BF16 || d.D % 256 != 0 || d.D / d.H != 256) return false;
    if ((double)d.B * d.T * d.D * 2.0 >= 2147483648.0) return false;   // 32-bit buffer offsets
    const char *on = getenv("RGLRU_FWD_FUSED");
    return on && on[0] == '1';
}

void launch_fused_fwd(const rglru_desc &d, const rglru_weights &w, const void *u, const void *hist_in,
                      const float *h0, void *y, float *h_last, void *hist_out, void *ws, hipStream_t s)
{
    FusedParams p;
    p.B = (int)d.B;
    p.T = (int)d.T;
    p.D = (int)d.D;
    p.NC = (int)((d.T + CHUNK - 1) / CHUNK);
    p.G = (int)(d.D / 256);
    p.units = p.B * p.NC;
    p.u = (const bf16 *)u;
    p.cw = w.conv_w;
    p.cb = w.conv_b;
    p.hist_in = (const bf16 *)hist_in;
    p.Wa = (const bf16 *)w.W_a;
    p.Wx = (const bf16 *)w.W_x;
    p.ba = w.b_a;
    p.bx = w.b_x;
    p.Lambda = w.Lambda;
    p.h0 = h0;
    p.y = (bf16 *)y;
    p.h_last = h_last;
    p.hist_out = (bf16 *)hist_out;
    p.c = d.c;
    p.y_bytes = (uint32_t)(d.B * d.T * d.D * 2);
    p.hdr = (WsHeader *)ws;
    p.claim = (uint32_t *)((char *)ws + sizeof(WsHeader));
    const size_t nw = (size_t)d.B * p.NC * d.D;
    p.aggA = (uint64_t *)((char *)ws + sizeof(WsHeader) + CLAIM_REGION_BYTES);
    p.aggX = p.aggA + nw;
    p.incl = p.aggX + nw;
    const FShape fs = fused_shape();
    // one workgroup per CU; RGLRU_FWD_GROUP_WORKGROUPS (a positive integer)
    // caps the workgroups per block, which changes nothing in the results
    long wpg = (long)fs.ncu / p.G;
    if (const char *cap = getenv("RGLRU_FWD_GROUP_WORKGROUPS")) {
        const long c = atol(cap);
        if (c > 0 && c < wpg) wpg = c;
    }
    if (wpg < 1) wpg = 1;
    if (wpg > p.units) wpg = p.units;
    fused_fwd_kernel<<<dim3((unsigned)(p.G * wpg)), dim3(256), F_LDS, s>>>(p);
}

}  // namespace rglru
