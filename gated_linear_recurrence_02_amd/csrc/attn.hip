// attn.hip -- local sliding-window multi-query attention, the other temporal
// mixer of Griffin (wiki note "Griffin", section "Local Attention Path": token t
// attends to the window t-W+1 .. t with softmax weights; page "Griffin Guide:
// RecurrentGemma, RG-LRU & Hybrid Attention", "Local Sliding-Window Multi-Query
// Attention (MQA)": all query heads share one key head and one value head, and
// "Bounding the Key-Value Cache Footprint": the decode cache keeps the last W
// positions, evicted ring-buffer fashion -- position p lives in slot p mod W).
//
// Layouts (row-major): q, o [B][T][Hq][dh]; k, v [B][T][dh]; caches
// [B][W][dh]; decode q_t, o_t [B][Hq][dh], k_t, v_t [B][dh], pos [B] int32.
// Scores are scale * q.k; softmax and sums in fp32.
//
// Kernels
//   attn_prefill_mfma  bf16, dh = 256.  A workgroup (8 waves of 16 rows)
//       takes 128 consecutive rows of the flattened (token, head) index of
//       one stream -- for MQA, rows of neighbouring tokens share their keys --
//       and walks the union of their windows in tiles of 64 keys,
//       double-buffered in LDS, the next tile's loads issued a tile ahead.
//       Per tile and wave: S^T = K Q^T (32 v_mfma_f32_16x16x32_bf16; K rows
//       read in the order that gives each lane 8 consecutive keys of one
//       query), an online softmax per query (the 4 lanes of a query hold the
//       tile's 64 scores), and O^T += V^T P^T (32 MFMAs; the lane's own
//       probabilities are the B operand, V^T -- staged transposed through
//       registers -- the A operand).
//   attn_step_mfma     bf16, dh = 256, Hq <= 16.  Decode, split over the ring:
//       a workgroup scores 256 slots for all heads with
//       v_mfma_f32_16x16x32_bf16 (K rows straight from HBM, heads padded to
//       16), keeps the exp-weights in LDS as bf16 and forms O^T = V^T P^T with
//       the same MFMA, V staged transposed in 64-slot chunks; attn_combine
//       merges the splits and writes the new key and value into their slot.
//   attn_*_generic     any io, dh <= 256: one wave per query row, the
//       reference-shaped loop (fp32 I/O and shapes the fast kernels exclude).
#include <math.h>

#include "common.h"
#include "internal.h"

namespace rglru {

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

template <typename T> __device__ __forceinline__ float ld1(const T *p) { return (float)*p; }

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// ------------------------------------------------------------------ generic
// One wave per (stream, token, head): lanes split dh; per key a wave-wide dot
// product, then the online softmax update.  Accurate exp for fp32 I/O.
template <typename T>
__global__ __launch_bounds__(256) void attn_prefill_generic(int B, int T_, int Hq, int dh, int W, float scale,
                                                           const T *q, const T *k, const T *v, T *o)
{
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= (long)B * T_ * Hq) return;
    const int b = (int)(row / ((long)T_ * Hq));
    const int t = (int)((row / Hq) % T_);
    float qv[4], acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        qv[i] = e < dh ? ld1(q + row * dh + e) : 0.0f;
    }
    float m = -INFINITY, l = 0.0f;
    const int lo = t - W + 1 < 0 ? 0 : t - W + 1;
    for (int j = lo; j <= t; ++j) {
        const T *kr = k + ((long)b * T_ + j) * dh, *vr = v + ((long)b * T_ + j) * dh;
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            if (e < dh) part = fmaf(qv[i], ld1(kr + e), part);
        }
        const float s = wave_sum(part) * scale;
        const float mn = fmaxf(m, s);
        const float alpha = expf(m - mn), p = expf(s - mn);
        l = fmaf(l, alpha, p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            acc[i] = fmaf(acc[i], alpha, e < dh ? p * ld1(vr + e) : 0.0f);
        }
        m = mn;
    }
    const float inv = 1.0f / l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        if (e < dh) o[row * dh + e] = from_f32<T>(acc[i] * inv);
    }
}

// Decode, one wave per (stream, head): positions max(0, pos-W+1) .. pos, the
// newest from k_t / v_t, the rest from their ring slots.  The wave of head 0
// writes k_t, v_t into slot pos mod W afterwards; that slot holds position
// pos - W, which no wave reads.
template <typename T>
__global__ __launch_bounds__(256) void attn_step_generic(int B, int Hq, int dh, int W, float scale, const T *q_t,
                                                        const T *k_t, const T *v_t, T *kc, T *vc,
                                                        const int32_t *pos, T *o_t)
{
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= (long)B * Hq) return;
    const int b = (int)(row / Hq), h = (int)(row % Hq);
    const long p = pos[b];
    float qv[4], acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        qv[i] = e < dh ? ld1(q_t + row * dh + e) : 0.0f;
    }
    float m = -INFINITY, l = 0.0f;
    const long lo = p - W + 1 < 0 ? 0 : p - W + 1;
    for (long j = lo; j <= p; ++j) {
        const T *kr = j == p ? k_t + (long)b * dh : kc + ((long)b * W + j % W) * dh;
        const T *vr = j == p ? v_t + (long)b * dh : vc + ((long)b * W + j % W) * dh;
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            if (e < dh) part = fmaf(qv[i], ld1(kr + e), part);
        }
        const float s = wave_sum(part) * scale;
        const float mn = fmaxf(m, s);
        const float alpha = expf(m - mn), pr = expf(s - mn);
        l = fmaf(l, alpha, pr);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            acc[i] = fmaf(acc[i], alpha, e < dh ? pr * ld1(vr + e) : 0.0f);
        }
        m = mn;
    }
    const float inv = 1.0f / l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        if (e < dh) o_t[row * dh + e] = from_f32<T>(acc[i] * inv);
    }
    if (h == 0) {
        const long slot = ((long)b * W + p % W) * dh;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            if (e < dh) {
                kc[slot + e] = k_t[(long)b * dh + e];
                vc[slot + e] = v_t[(long)b * dh + e];
            }
        }
    }
}

// Prefill's ring fill: positions max(0, T-W) .. T-1 into slots p mod W.
// One thread per 16-byte piece (dh * esz is a multiple of 16).
__global__ __launch_bounds__(256) void attn_fill_cache(int B, int T_, int W, int pieces_per_row, const uint4 *k,
                                                      const uint4 *v, uint4 *kc, uint4 *vc)
{
    const int n = T_ < W ? T_ : W;
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)B * n * pieces_per_row) return;
    const int c = (int)(idx % pieces_per_row);
    const long r = idx / pieces_per_row;
    const int b = (int)(r / n);
    const int p = T_ - n + (int)(r % n);
    const long src = ((long)b * T_ + p) * pieces_per_row + c;
    const long dst = ((long)b * W + p % W) * pieces_per_row + c;
    kc[dst] = k[src];
    vc[dst] = v[src];
}

// ------------------------------------------------------------ MFMA prefill
// A workgroup of NW waves owns 16 NW flattened (token, head) rows and walks its
// windows' keys in tiles of KT (32 or 64).
constexpr int PF_KSTRIDE = 264;   // bf16 per K row in LDS (528 B, conflict-free b128 reads)
template <int KT> struct PfTile {
    static constexpr int VSTRIDE = KT + 8;                 // bf16 per V^T row
    __device__ static int vrow(int r) { return r * VSTRIDE * 2; }   // byte offset of V^T row r
    static constexpr int KBYTES = KT * PF_KSTRIDE * 2;
    static constexpr int VBYTES = 256 * VSTRIDE * 2;
    static constexpr int STAGE = KBYTES + VBYTES;
    static constexpr int LDS = 2 * STAGE;
};

// The staged pieces of one key tile.  The first half of the threads carry 8
// pieces (128 B) of one K row each, the second half a block of 8 keys x 8 dh
// of V, transposed in registers before the LDS write so that V^T rows hold
// consecutive keys.
// (one array for both halves: separate ones would meet at the branch join
// as copies that wait for the loads)
struct PfStage {
    u32x4 r[8];
};

// K row and 64-dh segment carried by staging thread t (t < 4 KT): each
// aligned group of 8 threads takes rows {0-3, 8-11} + offset of one segment,
// whose LDS rows (permuted below) fall in 8 different bank groups
template <int KT> __device__ __forceinline__ int pf_krow(int t)
{
    return (t & 3) | (((t >> 3) & 1) << 2) | (((t >> 2) & 1) << 3) | (t & (KT - 16));
}
template <int KT> __device__ __forceinline__ int pf_kseg(int t) { return t / KT; }

template <int NW, int KT>
__device__ __forceinline__ void pf_load(PfStage &st, const bf16 *k, const bf16 *v, long kv0, int key0, int T_,
                                        int tid)
{
    constexpr int HALF = 32 * NW;
    // the split is by whole waves; a scalar branch keeps each wave on one side
    // (with both sides under an exec mask the two register sets alias and
    // every load would be waited for at once)
    if (__builtin_amdgcn_readfirstlane(tid >> 6) < NW / 2) {
        // keys past the end read the last row instead: real, finite values
        // whose weights the mask makes 0 (loads stay unconditional, so no
        // branch makes the wave wait for them here)
        const int row = pf_krow<KT>(tid), seg = pf_kseg<KT>(tid);   // 64 dh per thread
        const int key = key0 + row;
        const u32x4 *src = (const u32x4 *)(k + (kv0 + (key < T_ ? key : T_ - 1)) * 256 + 64 * seg);
#pragma unroll
        for (int i = 0; i < 8; ++i) st.r[i] = src[i];
    } else {
        const int t2 = tid - HALF, kg = t2 % (KT / 8), dg = t2 / (KT / 8);   // keys 8kg.., dh 8dg..
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int key = key0 + 8 * kg + i;
            st.r[i] = *(const u32x4 *)(v + (kv0 + (key < T_ ? key : T_ - 1)) * 256 + 8 * dg);
        }
    }
}

template <int NW, int KT>
__device__ __forceinline__ void pf_store(const PfStage &st, char *stage, int tid)
{
    constexpr int HALF = 32 * NW;
    if (__builtin_amdgcn_readfirstlane(tid >> 6) < NW / 2) {
        const int row = pf_krow<KT>(tid), seg = pf_kseg<KT>(tid);
        // key 32j + 8a + 4u + i goes to LDS row 32j + 16u + 4a + i, so that the
        // 16 keys one score tile reads together sit in 16 consecutive rows
        const int lrow = (row & 0x23) | ((row & 0x4) << 2) | ((row & 0x18) >> 1);
        u32x4 *dst = (u32x4 *)(stage + (lrow * PF_KSTRIDE + 64 * seg) * 2);
#pragma unroll
        for (int i = 0; i < 8; ++i) dst[i] = st.r[i];
    } else {
        const int t2 = tid - HALF, kg = t2 % (KT / 8), dg = t2 / (KT / 8);
        // r[i] holds key 8kg+i, dh 8dg..8dg+7 (dword c = dh pair 2c, 2c+1);
        // V^T row 8dg + j receives keys 8kg..8kg+7 of dh 8dg + j
        char *vt = stage + PfTile<KT>::KBYTES;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;   // high or low halves
            const int c = j >> 1;
            u32x4 o;
            o[0] = __builtin_amdgcn_perm(st.r[1][c], st.r[0][c], sel);
            o[1] = __builtin_amdgcn_perm(st.r[3][c], st.r[2][c], sel);
            o[2] = __builtin_amdgcn_perm(st.r[5][c], st.r[4][c], sel);
            o[3] = __builtin_amdgcn_perm(st.r[7][c], st.r[6][c], sel);
            *(u32x4 *)(vt + PfTile<KT>::vrow(8 * dg + j) + 16 * kg) = o;
        }
    }
}

// 16 query rows per wave on v_mfma_f32_16x16x32_bf16.  In the score tiles
// (keys x queries, KT/16 of 16 keys per tile) A row r of tile st is key
// 32(st/2) + 8(r/4) + 4(st%2) + r%4, so that lane (n, g) -- query n = lane%16,
// g = lane/16 -- ends up with keys 32j + 8g .. +7 of each 32-key step j:
// exactly the k-slots it supplies as the B operand of step j of
// O^T += V^T P^T, whose A operand then reads 8 consecutive keys of a V^T row.
template <int NW, int KT>
__global__ __launch_bounds__(64 * NW, 2) void attn_prefill_mfma(int T_, int Hq, int W, float scale_log2e,
                                                             const bf16 *q, const bf16 *k, const bf16 *v, bf16 *o)
{
    constexpr int ROWS = 16 * NW, NST = KT / 16, NJ = KT / 32;
    using TL = PfTile<KT>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, g = lane >> 4;
    const long rows_per_b = (long)T_ * Hq;
    const long tiles_per_b = (rows_per_b + ROWS - 1) / ROWS;
    const int b = (int)(blockIdx.x / tiles_per_b);
    const long f0 = (blockIdx.x % tiles_per_b) * ROWS;   // first flattened row of the workgroup
    const long kv0 = (long)b * T_;                       // first key row of stream b

    // this lane's query row
    const long f = f0 + 16 * wave + n;
    const bool row_ok = f < rows_per_b;
    const int t = row_ok ? (int)(f / Hq) : -1;
    bf16x8 qb[8];
    {
        const bf16 *qr = q + ((long)b * rows_per_b + (row_ok ? f : 0)) * 256 + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qb[ks] = row_ok ? *(const bf16x8 *)(qr + 32 * ks) : bf16x8{};
    }

    // keys of the union of the workgroup's windows
    const long f_last = (f0 + ROWS - 1 < rows_per_b ? f0 + ROWS - 1 : rows_per_b - 1);
    const int t_first = (int)(f0 / Hq), t_last = (int)(f_last / Hq);
    const int k_lo = t_first - W + 1 < 0 ? 0 : t_first - W + 1;
    const int tile0 = k_lo / KT, tile1 = t_last / KT;

    f32x4_t acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = f32x4_t{};
    float m = -INFINITY, l = 0.0f;

    // tile i is computed from LDS while tile i+1 is on its way from memory
    PfStage st;
    pf_load<NW, KT>(st, k, v, kv0, tile0 * KT, T_, tid);
    pf_store<NW, KT>(st, smem + (tile0 & 1) * TL::STAGE, tid);
    __syncthreads();

    for (int tile = tile0; tile <= tile1; ++tile) {
        if (tile < tile1) pf_load<NW, KT>(st, k, v, kv0, (tile + 1) * KT, T_, tid);
        const char *stage = smem + (tile & 1) * TL::STAGE;

        // S^T = K Q^T over dh = 256, NST tiles of 16 keys (A row of this lane
        // in tile st: LDS row 32(st/2) + 16(st%2) + n)
        f32x4_t sa[NST] = {};
        {
            const bf16 *kr = (const bf16 *)stage + n * PF_KSTRIDE + 8 * g;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                for (int s4 = 0; s4 < NST; ++s4) {
                    const int off = (32 * (s4 >> 1) + 16 * (s4 & 1)) * PF_KSTRIDE;
                    const bf16x8 a = *(const bf16x8 *)(kr + off + 32 * ks);
                    sa[s4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[ks], sa[s4], 0, 0, 0);
                }
        }
        // this lane's keys: 32j + 8g + e, e = 4(st%2) + i, j = st/2
        float sv[4 * NST];
#pragma unroll
        for (int s4 = 0; s4 < NST; ++s4)
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[8 * (s4 >> 1) + 4 * (s4 & 1) + i] = sa[s4][i];
        float mt = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4 * NST; ++e) {
            const int key = tile * KT + 32 * (e >> 3) + 8 * g + (e & 7);
            const bool ok = key <= t && key > t - W;
            sv[e] = ok ? sv[e] * scale_log2e : -INFINITY;
            mt = fmaxf(mt, sv[e]);
        }
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        // the reference maximum moves only when the tile's maximum passes it
        // by more than 8 (log2 units): the weights then stay below 2^8 and
        // the accumulators are rescaled rarely
        const float mn = mt > m + 8.0f ? mt : m;
        const float mu = mn == -INFINITY ? 0.0f : mn;
        const float alpha = hw_exp2(m - mu);   // 0 while m is -inf
        float ls = 0.0f;
        bf16x8 pb[NJ];
#pragma unroll
        for (int e = 0; e < 4 * NST; ++e) {
            const float pr = hw_exp2(sv[e] - mu);
            ls += pr;
            pb[e >> 3][e & 7] = (bf16)pr;
        }
        ls += __shfl_xor(ls, 16);
        ls += __shfl_xor(ls, 32);
        l = fmaf(l, alpha, ls);
        m = mn;
        if (__any(alpha != 1.0f)) {   // rescale only when some query's maximum moved
#pragma unroll
            for (int i = 0; i < 16; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][r] *= alpha;
        }
        // O^T += V^T P^T: 16 dh tiles, NJ 32-key steps each
        {
            const char *vt = stage + TL::KBYTES + 16 * g;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int dt = 0; dt < 16; ++dt) {
                    const bf16x8 a = *(const bf16x8 *)(vt + TL::vrow(16 * dt + n) + 64 * j);
                    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[j], acc[dt], 0, 0, 0);
                }
        }
        if (tile < tile1) pf_store<NW, KT>(st, smem + ((tile + 1) & 1) * TL::STAGE, tid);
        __syncthreads();
    }

    if (row_ok) {
        const float inv = 1.0f / l;
        bf16 *orow = o + ((long)b * rows_per_b + f) * 256;
        typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) {
            bf16x4 w4;
#pragma unroll
            for (int i = 0; i < 4; ++i) w4[i] = (bf16)(acc[dt][i] * inv);
            *(bf16x4 *)(orow + 16 * dt + 4 * g) = w4;   // lane holds dh 16 dt + 4 g + i
        }
    }
}

// the launch shape: workgroups of 4 waves (64 rows) and 32-key tiles, 75 KB of
// LDS, so that two workgroups share a CU and drift out of phase
constexpr int PF_NW = 4, PF_KT = 32;

// -------------------------------------------------------------- MFMA decode
constexpr int DS_SLOTS = 256;   // ring slots per workgroup

// Partial results per (stream, split, head): dh sums of exp-weighted values,
// the split's maximum score (log2 units) and its exp-weight sum.
struct StepWs {
    float *o;   // [B][NS][16][256]
    float *m;   // [B][NS][16]
    float *l;   // [B][NS][16]
};

__global__ __launch_bounds__(256) void attn_step_mfma(int Hq, int W, int NS, float scale_log2e, const bf16 *q_t,
                                                     const bf16 *k_t, const bf16 *v_t, const bf16 *kc,
                                                     const bf16 *vc, const int32_t *pos, StepWs ws)
{
    constexpr int PT = DS_SLOTS + 8;   // bf16 per row of P^T (16-byte pieces, rows apart in banks)
    constexpr int VS = 72;             // bf16 per V^T row of a 64-slot chunk (144 B)
    __shared__ __attribute__((aligned(16))) bf16 Pt[16][PT];    // exp-weights [head][slot]
    __shared__ __attribute__((aligned(16))) bf16 Vt[256][VS];   // one chunk of V, transposed
    __shared__ float wmax[4][16];
    __shared__ float wsum[4][16];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int b = blockIdx.x / NS, sp = blockIdx.x % NS;
    const int p = pos[b];
    const int cur = p % W;
    const int n16 = lane & 15, kg = lane >> 4;
    // a slot s < W holds a position of the window iff it has been written,
    // i.e. s <= p (the slot's position is p - ((p - s) mod W), which is >= 0
    // exactly then)

    // q^T as B operand: lane holds head n16, dh 32*ks + 8*kg .. +8
    bf16x8 qb[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
        qb[ks] = n16 < Hq ? *(const bf16x8 *)(q_t + ((long)b * Hq + (n16 < Hq ? n16 : 0)) * 256 + 32 * ks + 8 * kg)
                          : bf16x8{};

    // scores of this wave's 64 slots, 16 at a time
    float sc[4][4];
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const int slot_a = sp * DS_SLOTS + 64 * wave + 16 * st + n16;   // A-operand row of this lane
        const bool a_ok = slot_a < W;
        // rows past the ring read its last slot: whatever it holds only enters
        // scores that the mask below replaces, and the loads need no branch
        const bf16 *kr = slot_a == cur ? k_t + (long)b * 256 : kc + ((long)b * W + (a_ok ? slot_a : W - 1)) * 256;
        f32x4_t acc = {};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const bf16x8 a = *(const bf16x8 *)(kr + 32 * ks + 8 * kg);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[ks], acc, 0, 0, 0);
        }
        // lane holds head n16 for slots 4*kg + i of the 16
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int slot = sp * DS_SLOTS + 64 * wave + 16 * st + 4 * kg + i;
            const bool ok = slot < W && slot <= p && n16 < Hq;
            sc[st][i] = ok ? acc[i] * scale_log2e : -INFINITY;
            mx = fmaxf(mx, sc[st][i]);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (kg == 0) wmax[wave][n16] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(wmax[0][n16], wmax[1][n16]), fmaxf(wmax[2][n16], wmax[3][n16]));
    const float mu = M == -INFINITY ? 0.0f : M;
    float ls = 0.0f;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
        bf16x4 w4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float pr = hw_exp2(sc[st][i] - mu);
            ls += pr;
            w4[i] = (bf16)pr;
        }
        *(bf16x4 *)&Pt[n16][64 * wave + 16 * st + 4 * kg] = w4;
    }
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    if (kg == 0) wsum[wave][n16] = ls;

    // O^T = V^T P^T on the matrix cores, 64 slots at a time: V is staged
    // transposed (thread = 8 slots x 8 dh, transposed in registers); slots
    // never written (position < 0) and slots past W enter as zeros, so that
    // whatever they hold cannot reach the sums.  Wave w owns dh 64w .. 64w+63.
    f32x4_t o4[4] = {};
    const int sg = tid >> 5, dg = tid & 31;
    for (int ch = 0; ch < DS_SLOTS / 64; ++ch) {
        u32x4 r[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int slot = sp * DS_SLOTS + 64 * ch + 8 * sg + i;
            const bool ok = slot < W && slot <= p;
            const bf16 *vr = slot == cur ? v_t + (long)b * 256 : vc + ((long)b * W + (slot < W ? slot : W - 1)) * 256;
            const u32x4 val = *(const u32x4 *)(vr + 8 * dg);   // unconditional; zeroed below if unused
            r[i] = ok ? val : u32x4{0, 0, 0, 0};
        }
        __syncthreads();   // the previous chunk's V^T has been read (first pass: P^T is complete)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
            const int c = j >> 1;
            u32x4 o;
            o[0] = __builtin_amdgcn_perm(r[1][c], r[0][c], sel);
            o[1] = __builtin_amdgcn_perm(r[3][c], r[2][c], sel);
            o[2] = __builtin_amdgcn_perm(r[5][c], r[4][c], sel);
            o[3] = __builtin_amdgcn_perm(r[7][c], r[6][c], sel);
            *(u32x4 *)&Vt[8 * dg + j][8 * sg] = o;
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 pb = *(const bf16x8 *)&Pt[n16][64 * ch + 32 * ks + 8 * kg];
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const bf16x8 a = *(const bf16x8 *)&Vt[64 * wave + 16 * dt + n16][32 * ks + 8 * kg];
                o4[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, o4[dt], 0, 0, 0);
            }
        }
    }
    // lane holds head n16 and dh 64*wave + 16*dt + 4*kg + i
    const long base = ((long)b * NS + sp) * 16;
    if (n16 < Hq) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
            *(f32x4_t *)(ws.o + (base + n16) * 256 + 64 * wave + 16 * dt + 4 * kg) = o4[dt];
    }
    if (tid < 16) {
        ws.m[base + tid] = fmaxf(fmaxf(wmax[0][tid], wmax[1][tid]), fmaxf(wmax[2][tid], wmax[3][tid]));
        ws.l[base + tid] = wsum[0][tid] + wsum[1][tid] + wsum[2][tid] + wsum[3][tid];
    }
}

// One workgroup per (stream, head): merge the splits; the head-0 workgroup
// then writes the new key and value into slot pos mod W (no workgroup of
// this launch reads the cache).
__global__ __launch_bounds__(256) void attn_combine(int Hq, int W, int NS, StepWs ws, const bf16 *k_t,
                                                   const bf16 *v_t, bf16 *kc, bf16 *vc, const int32_t *pos,
                                                   bf16 *o_t)
{
    const int b = blockIdx.x / Hq, h = blockIdx.x % Hq, d = threadIdx.x;   // 256 threads = dh
    float M = -INFINITY;
    for (int s = 0; s < NS; ++s) M = fmaxf(M, ws.m[((long)b * NS + s) * 16 + h]);
    float num = 0.0f, den = 0.0f;
    for (int s = 0; s < NS; ++s) {
        const long base = ((long)b * NS + s) * 16 + h;
        const float wgt = hw_exp2(ws.m[base] - M);   // 0 for an empty split
        den = fmaf(wgt, ws.l[base], den);
        num = fmaf(wgt, ws.o[base * 256 + d], num);
    }
    o_t[((long)b * Hq + h) * 256 + d] = (bf16)(num / den);
    if (h == 0) {
        const long slot = ((long)b * W + pos[b] % W) * 256 + d;
        kc[slot] = k_t[(long)b * 256 + d];
        vc[slot] = v_t[(long)b * 256 + d];
    }
}

}  // namespace

bool attn_fast_prefill(const rglru_attn_desc &d) { return d.io == RGLRU_BF16 && d.dh == 256; }
bool attn_fast_step(const rglru_attn_desc &d) { return d.io == RGLRU_BF16 && d.dh == 256 && d.Hq <= 16; }

size_t attn_workspace_bytes(const rglru_attn_desc &d)
{
    if (!attn_fast_step(d)) return 256;
    const int64_t NS = (d.W + DS_SLOTS - 1) / DS_SLOTS;
    return (size_t)d.B * NS * 16 * (256 + 2) * 4 + 512;
}

void launch_attn_fwd(const rglru_attn_desc &d, const void *q, const void *k, const void *v, void *o, void *kc,
                     void *vc, hipStream_t s)
{
    const float scale = d.scale;
    if (attn_fast_prefill(d)) {
        constexpr int lds = PfTile<PF_KT>::LDS;
        static bool attr = false;
        if (!attr) {
            (void)hipFuncSetAttribute((const void *)&attn_prefill_mfma<PF_NW, PF_KT>,
                                      hipFuncAttributeMaxDynamicSharedMemorySize, lds);
            attr = true;
        }
        const long tiles = (d.T * d.Hq + 16 * PF_NW - 1) / (16 * PF_NW);
        attn_prefill_mfma<PF_NW, PF_KT><<<dim3((unsigned)(d.B * tiles)), dim3(64 * PF_NW), lds, s>>>(
            (int)d.T, (int)d.Hq, (int)d.W, scale * 1.4426950408889634f, (const bf16 *)q, (const bf16 *)k,
            (const bf16 *)v, (bf16 *)o);
    } else {
        const long rows = d.B * d.T * d.Hq;
        const unsigned grid = (unsigned)((rows + 3) / 4);
        if (d.io == RGLRU_BF16)
            attn_prefill_generic<bf16><<<grid, 256, 0, s>>>((int)d.B, (int)d.T, (int)d.Hq, (int)d.dh, (int)d.W,
                                                            scale, (const bf16 *)q, (const bf16 *)k,
                                                            (const bf16 *)v, (bf16 *)o);
        else
            attn_prefill_generic<float><<<grid, 256, 0, s>>>((int)d.B, (int)d.T, (int)d.Hq, (int)d.dh,
                                                             (int)d.W, scale, (const float *)q, (const float *)k,
                                                             (const float *)v, (float *)o);
    }
    if (kc) {
        const int esz = d.io == RGLRU_BF16 ? 2 : 4;
        const int ppr = (int)(d.dh * esz / 16);
        const long n = d.T < d.W ? d.T : d.W;
        const long total = d.B * n * ppr;
        attn_fill_cache<<<dim3((unsigned)((total + 255) / 256)), 256, 0, s>>>(
            (int)d.B, (int)d.T, (int)d.W, ppr, (const uint4 *)k, (const uint4 *)v, (uint4 *)kc, (uint4 *)vc);
    }
}

void launch_attn_step(const rglru_attn_desc &d, const void *q_t, const void *k_t, const void *v_t, void *kc,
                      void *vc, const int32_t *pos, void *o_t, void *ws, hipStream_t s)
{
    const float scale = d.scale;
    if (attn_fast_step(d)) {
        const int NS = (int)((d.W + DS_SLOTS - 1) / DS_SLOTS);
        StepWs w;
        w.o = (float *)ws;
        w.m = w.o + (size_t)d.B * NS * 16 * 256;
        w.l = w.m + (size_t)d.B * NS * 16;
        attn_step_mfma<<<dim3((unsigned)(d.B * NS)), 256, 0, s>>>(
            (int)d.Hq, (int)d.W, NS, scale * 1.4426950408889634f, (const bf16 *)q_t, (const bf16 *)k_t,
            (const bf16 *)v_t, (const bf16 *)kc, (const bf16 *)vc, pos, w);
        attn_combine<<<dim3((unsigned)(d.B * d.Hq)), 256, 0, s>>>((int)d.Hq, (int)d.W, NS, w, (const bf16 *)k_t,
                                                         (const bf16 *)v_t, (bf16 *)kc, (bf16 *)vc, pos,
                                                         (bf16 *)o_t);
    } else {
        const long rows = d.B * d.Hq;
        const unsigned grid = (unsigned)((rows + 3) / 4);
        if (d.io == RGLRU_BF16)
            attn_step_generic<bf16><<<grid, 256, 0, s>>>((int)d.B, (int)d.Hq, (int)d.dh, (int)d.W, scale,
                                                         (const bf16 *)q_t, (const bf16 *)k_t, (const bf16 *)v_t,
                                                         (bf16 *)kc, (bf16 *)vc, pos, (bf16 *)o_t);
        else
            attn_step_generic<float><<<grid, 256, 0, s>>>((int)d.B, (int)d.Hq, (int)d.dh, (int)d.W, scale,
                                                          (const float *)q_t, (const float *)k_t,
                                                          (const float *)v_t, (float *)kc, (float *)vc, pos,
                                                          (float *)o_t);
    }
}

}  // namespace rglru
