// bwd.hip -- a7: backward of the fused forward (conv + block-diagonal gates +
// log-space decay + scan), i.e. the vector-Jacobian product of
// L = <dy, y> + <dh_last, h_last>.
//
// The pages give the forward only (page "Griffin Guide: RecurrentGemma, RG-LRU
// & Hybrid Attention", "Formulation of the RG-LRU Gating Mechanism" and
// "Temporal Filtering via Separable 1D Convolutions"); this is its exact
// derivative.  With delta_t = dL/dh_t (total) and eps_t = a_t delta_t:
//     delta_t = dy_t + eps_{t+1},  eps_T = dh_last,  dh0 = eps_0
//     eps_t   = a_t eps_{t+1} + a_t dy_t            (reverse affine scan)
//     dl_t    = delta_t (a_t h_{t-1} - (a_t^2 / beta_t) i_t x_t)
//     dz^a    = -c s dl r (1 - r),   dz^x = delta beta x i (1 - i)
//     dx_t    = delta beta i + W_a^T dz^a + W_x^T dz^x
//     dLambda = sum c r sigma(-Lambda) dl,   db = sum dz,   dW = sum dz x^T
//     du_t    = sum_k cw[k] dx_{t+3-k},   dcw[k] = sum dx_t u_{t-3+k},   dcb = sum dx
//
// Passes (all on the caller's stream):
//   1. forward states: the mode-A forward kernel keeps only the state before
//      each 32-token chunk;
//   2. transposed gate weights Wt[h][j][o'] (o' < 256: W_a, else W_x);
//   3. the chunk kernel: persistent like the forward, workgroup w serves
//      block g = w % G and claims the (stream, chunk) units of that block at
//      run time, starting from the END of the sequence (unit j = cr*B + b
//      with cr the chunk index counted from the end): recompute
//      conv, gates (MFMA), decay and the states inside the chunk; reverse
//      scan whose chunk carries eps go through the same decoupled look-back
//      as the forward; local gradients; dx through the gates on the matrix
//      cores; conv backward, whose last 3 tokens need the first 3 dx of the
//      next chunk (published as tagged words); per-chunk partial sums; dz and
//      x written channel-major in fp32 for pass 4;
//   4. dW = sum over rows of dz x^T on the matrix cores, split over row
//      ranges into partials;
//   5. deterministic reductions of the partials (fixed order, no atomics;
//      the per-chunk sums in two steps, over unit splits then splits).
// Precision (bf16 I/O): products whose operands are computed values (dz, x)
// use a two-term split v = hi + lo with hi = bf16(v), lo = bf16(v - hi):
// dx = W^T dz_hi + W^T dz_lo (W is exactly bf16), dW = dz_hi x_hi^T +
// dz_hi x_lo^T + dz_lo x_hi^T; the bf16 rounding of dz or x alone would
// cost up to 4e-2 relative on dW for short sequences.
#include <mutex>

#include "common.h"
#include "gatemath.h"
#include "internal.h"

namespace rglru {

namespace {

constexpr int NSUM = 8;   // per-chunk partial sums: dcw[4], dcb, db_a, db_x, dLambda
constexpr int PS_SPLITS = 16;   // unit splits of the first reduction step

struct BwdLayout {
    size_t fwd_words, claims, bwd_words, hstart, Wt, dZt, Xt, psum, ppart, dWpart, total;
    int S;   // row-range splits of the dW products
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

BwdLayout bwd_layout(int64_t B, int64_t T, int64_t D, int64_t H, size_t esz)
{
    BwdLayout L;
    const int64_t NC = (T + CHUNK - 1) / CHUNK;
    const size_t NW = (size_t)B * NC * D;
    int S = (int)((256 + 2 * H - 1) / (2 * H));
    if (S < 1) S = 1;
    if ((int64_t)S > B * NC) S = (int)(B * NC);
    L.S = S;
    size_t off = sizeof(WsHeader);
    L.fwd_words = off;  off = align256(fwd_workspace_bytes(B, T, D));   // claims + carry words
    L.claims = off;     off = align256(off + claim_bytes(H));
    L.bwd_words = off;  off = align256(off + 6 * NW * 8);
    L.hstart = off;     off = align256(off + NW * 4);
    L.Wt = off;         off = align256(off + (size_t)H * 256 * 512 * esz);
    L.dZt = off;        off = align256(off + NW * 64 * 4);
    L.Xt = off;         off = align256(off + NW * 32 * 4);
    L.psum = off;       off = align256(off + NW * NSUM * 4);
    L.ppart = off;      off = align256(off + (size_t)PS_SPLITS * D * NSUM * 4);
    L.dWpart = off;     off = align256(off + (size_t)S * H * 2 * 65536 * 4);
    L.total = off;
    return L;
}

// ------------------------------------------------------------------ pass 2
template <typename T>
__global__ __launch_bounds__(256) void transpose_w_kernel(const T *Wa, const T *Wx, T *Wt)
{
    // tile of 32 (o) x 32 (j); grid (256/32 j-tiles, 512/32 o'-tiles, H)
    __shared__ T tile[32][33];
    const int h = blockIdx.z, j0 = blockIdx.x * 32, o0 = blockIdx.y * 32;
    const T *src = (o0 < 256 ? Wa : Wx) + (size_t)h * 65536;
    const int ob = o0 & 255;
    for (int e = threadIdx.x; e < 1024; e += 256) {
        const int oo = e >> 5, jj = e & 31;
        tile[oo][jj] = src[(size_t)(ob + oo) * 256 + j0 + jj];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 1024; e += 256) {
        const int jj = e >> 5, oo = e & 31;
        Wt[(size_t)h * 131072 + (size_t)(j0 + jj) * 512 + o0 + oo] = tile[oo][jj];
    }
}

// dx[k] += sum_o Z[16h+k][o] * Wt_part[j][o] for the lane's channel j = 32w + n,
// with Z = Zh + Zl (two LDS tiles, 32 x 256 in the XTile layout; Wt_part rows
// have stride 512)
__device__ __forceinline__ void dx_tile(const bf16 *Zh, const bf16 *Zl, const bf16 *Wt_part, int wave,
                                        int lane, float dx[16])
{
    constexpr int S = XTile<bf16>::STRIDE;
    const int r = lane & 31, kg = lane >> 5;
    const int off = tile_row_token(r) * S + 8 * kg;
    const bf16 *wrow = Wt_part + (size_t)(32 * wave + r) * 512 + 8 * kg;
    f32x16 C = {};
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        const bf16x8 bv = *(const bf16x8 *)(wrow + 16 * s);
        const bf16x8 ah = *(const bf16x8 *)(Zh + off + 16 * s);
        const bf16x8 al = *(const bf16x8 *)(Zl + off + 16 * s);
        C = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bv, C, 0, 0, 0);
        C = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bv, C, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) dx[k] += C[k];
}

__device__ __forceinline__ void dx_tile(const float *Zs, const float *, const float *Wt_part, int wave,
                                        int lane, float dx[16])
{
    constexpr int S = XTile<float>::STRIDE;
    const int n = lane & 31, half = lane >> 5;
    const float *wrow = Wt_part + (size_t)(32 * wave + n) * 512;
    const float *zs = Zs + 16 * half * S;
    for (int o = 0; o < 256; ++o) {
        const float wv = wrow[o];
#pragma unroll
        for (int k = 0; k < 16; ++k) dx[k] = fmaf(zs[k * S + o], wv, dx[k]);
    }
}

// write v into the A-operand tiles: hi part (or the value itself for fp32) and lo part
__device__ __forceinline__ void put_split(bf16 *Zh, bf16 *Zl, int idx, float v)
{
    const bf16 hi = (bf16)v;
    Zh[idx] = hi;
    Zl[idx] = (bf16)(v - (float)hi);
}
__device__ __forceinline__ void put_split(float *Zh, float *, int idx, float v) { Zh[idx] = v; }

__device__ __forceinline__ float wait_word(const uint64_t *p, uint32_t tag, WsHeader *hdr)
{
    float v;
    uint32_t spins = 0;
    while (!get_word(p, tag, v)) {
        if (++spins > SPIN_LIMIT) {
            __hip_atomic_store(&hdr->error, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return __builtin_nanf("");
        }
        __builtin_amdgcn_s_sleep(4);
    }
    return v;
}

struct BwdParams {
    int B, T, D, NC, G;
    float c;
    const void *u, *hist_in, *dy;
    const float *h0, *dh_last;
    const float *cw, *cb, *ba, *bx, *Lambda;
    const void *Wa, *Wx, *Wt;
    const float *hstart;
    void *du;
    float *dh0;
    float *dZt, *Xt;
    float *psum;
    int units;          // B * NC per block
    WsHeader *hdr;
    uint32_t *claim;    // [G] unit counters
    uint64_t *aggA, *aggX, *incl, *halo;   // halo: 3 consecutive arrays of [B][NC][D]
};

// ------------------------------------------------------------------ pass 3
template <typename T>
__global__ __launch_bounds__(512) void bwd_chunk_kernel(BwdParams p)
{
    constexpr int S = XTile<T>::STRIDE;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    T *Xs = (T *)smem;             // x tile, then dz (hi part)
    T *Zl = Xs + 32 * S;           // dz lo part (bf16 only)
    uint32_t *s_unit = (uint32_t *)(smem + 2 * 32 * S * sizeof(T));   // [2] + flag
    const uint32_t tag = launch_tag(p.hdr);
    const int g = blockIdx.x % p.G;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 31, half = lane >> 5;
    const int ch = wave * 32 + n;          // channel inside the block
    const int d = g * 256 + ch;
    const T *u = (const T *)p.u;
    const uint32_t units = (uint32_t)p.units;
    uint32_t *claim = p.claim + g;

    // Unit u_m of this workgroup travels through claim slot m & 1: thread 0
    // claims u_{n+1} at the start of iteration n and stores it at the end.
    if (tid == 0) s_unit[0] = claim_next(claim);
    for (int it = 0;; ++it) {
    __syncthreads();   // the claim slot and the LDS tiles of the previous unit are free
    const uint32_t j = s_unit[it & 1];
    if (j >= units) break;
    uint32_t my_claim = 0;
    if (tid == 0) my_claim = claim_next(claim);
    const int b = (int)(j % p.B);
    const int cr = (int)(j / p.B);         // chunk index counted from the end
    const int c = p.NC - 1 - cr;
    const int tb = c * CHUNK + 16 * half;
    const long row_b = (long)b * p.T;
    const long cidx = ((long)b * p.NC + c) * p.D + d;   // [B][NC][D] index of this chunk

    // conv recompute (window kept for dcw)
    const float w0 = p.cw[4 * (long)d + 0], w1 = p.cw[4 * (long)d + 1];
    const float w2 = p.cw[4 * (long)d + 2], w3 = p.cw[4 * (long)d + 3];
    const float bias = p.cb ? p.cb[d] : 0.0f;
    // the 19 loads go out together: addresses are selected, not branched on
    // (positions past the end or before a missing history read element 0 and
    // are zeroed afterwards)
    float win[19];
    {
        T raw[19];
#pragma unroll
        for (int m = 0; m < 19; ++m) {
            const int tau = tb - 3 + m;
            const T *src = u;
            if (tau >= 0 && tau < p.T) src = u + (row_b + tau) * p.D + d;
            else if (tau < 0 && p.hist_in) src = (const T *)p.hist_in + ((long)b * 3 + 3 + tau) * p.D + d;
            raw[m] = *src;
        }
#pragma unroll
        for (int m = 0; m < 19; ++m) {
            const int tau = tb - 3 + m;
            const bool ok = tau < p.T && (tau >= 0 || p.hist_in);
            win[m] = ok ? to_f32(raw[m]) : 0.0f;
        }
    }
    float x[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
        x[k] = fmaf(w3, win[k + 3], fmaf(w2, win[k + 2], fmaf(w1, win[k + 1], fmaf(w0, win[k], bias))));

    // gates
#pragma unroll
    for (int k = 0; k < 16; ++k) Xs[(16 * half + k) * S + ch] = from_f32<T>(x[k]);
    {   // x, channel-major per chunk, for the dW products
        float *xt = p.Xt + ((((long)b * p.NC + c) * p.G + g) * 256 + ch) * 32 + 16 * half;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *(f32x4 *)(xt + 4 * q) = f32x4{x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
    }
    __syncthreads();
    float za[16], zx[16];
    gate_tile(Xs, (const T *)p.Wa + (size_t)g * 65536, (const T *)p.Wx + (size_t)g * 65536, wave, lane,
              za, zx);

    // decay, normalisation and the forward states inside the chunk
    const float lam = p.Lambda[d];
    const float ncs = -p.c * softplus_acc(-lam);
    const float sgm = sigmoid_acc(-lam);
    const float bav = p.ba ? p.ba[d] : 0.0f, bxv = p.bx ? p.bx[d] : 0.0f;
    float a[16], hl[16], P[16];
    float h = 0.0f, pr = 1.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        za[k] = sigmoid_acc(za[k] + bav);   // r
        zx[k] = sigmoid_acc(zx[k] + bxv);   // i
        float ak = expf(ncs * za[k]);
        float bb = sqrtf(-expm1f(2.0f * ncs * za[k])) * zx[k] * x[k];
        if (tb + k >= p.T) {
            ak = 1.0f;
            bb = 0.0f;
        }
        a[k] = ak;
        h = fmaf(ak, h, bb);
        pr *= ak;
        hl[k] = h;
        P[k] = pr;
    }
    const float A0 = __shfl_xor(P[15], 32), X0 = __shfl_xor(hl[15], 32);
    const float hs_chunk = p.hstart[cidx];
    const float hs_lane = half == 0 ? hs_chunk : fmaf(A0, hs_chunk, X0);

    // reverse scan inside the lane (eps entering the lane's last token = 0)
    const T *dyp = (const T *)p.dy;
    float gdy[16];
    {
        T raw[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) raw[k] = dyp[tb + k < p.T ? (row_b + tb + k) * p.D + d : 0];
#pragma unroll
        for (int k = 0; k < 16; ++k) gdy[k] = tb + k < p.T ? to_f32(raw[k]) : 0.0f;
    }
    float dl[16], R[16];
    float e = 0.0f, Rrun = 1.0f;
#pragma unroll
    for (int k = 15; k >= 0; --k) {
        const float gk = gdy[k];
        dl[k] = gk + e;
        R[k] = Rrun;
        e = a[k] * dl[k];
        Rrun *= a[k];
    }
    // chunk carry: half 1 is first in reverse order
    const float A1 = __shfl_xor(Rrun, 32), X1 = __shfl_xor(e, 32);
    float ein_chunk = 0.0f;
    if (half == 0) {
        const float Ach = Rrun * A1;
        const float Xch = fmaf(Rrun, X1, e);
        const long base = (long)b * p.NC * p.D + d;
        const long widx = base + (long)cr * p.D;
        const float ebefore = p.dh_last ? p.dh_last[(long)b * p.D + d] : 0.0f;
        put_word(p.aggA + widx, Ach, tag);
        put_word(p.aggX + widx, Xch, tag);
        if (cr == 0) {
            ein_chunk = ebefore;
        } else {
            ein_chunk = look_back(p.aggA + base, p.aggX + base, p.incl + base, cr - 1, p.D, ebefore,
                                  tag, p.hdr);
        }
        const float eout = fmaf(Ach, ein_chunk, Xch);
        put_word(p.incl + widx, eout, tag);
        if (c == 0 && p.dh0) p.dh0[(long)b * p.D + d] = eout;
    }
    const float eother = __shfl_xor(ein_chunk, 32);
    const float ein_lane = half == 1 ? eother : fmaf(A1, ein_chunk, X1);

    // local gradients
    float dxv[16];
    float s_ba = 0.0f, s_bx = 0.0f, s_rl = 0.0f;
    float hprev = hs_lane;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const float delta = fmaf(R[k], ein_lane, dl[k]);
        const float hk = fmaf(P[k], hs_lane, hl[k]);
        const float r = za[k], ii = zx[k];
        float dza = 0.0f, dzx = 0.0f, dxd = 0.0f;
        if (tb + k < p.T) {
            const float l = ncs * r;
            const float beta = sqrtf(-expm1f(2.0f * l));
            const float dlk = delta * (a[k] * hprev - (a[k] * a[k] / beta) * ii * x[k]);
            const float di = delta * beta * x[k];
            dxd = delta * beta * ii;
            dza = ncs * dlk * r * (1.0f - r);
            dzx = di * ii * (1.0f - ii);
            s_rl = fmaf(r, dlk, s_rl);
        }
        s_ba += dza;
        s_bx += dzx;
        dxv[k] = dxd;
        za[k] = dza;   // reuse: dz^a
        zx[k] = dzx;   // reuse: dz^x
        hprev = hk;
    }
    {   // dz, channel-major per chunk, for the dW products
        float *zt = p.dZt + (((((long)b * p.NC + c) * p.G + g) * 2) * 256 + ch) * 32 + 16 * half;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            *(f32x4 *)(zt + 4 * q) = f32x4{za[4 * q], za[4 * q + 1], za[4 * q + 2], za[4 * q + 3]};
            *(f32x4 *)(zt + 256 * 32 + 4 * q) = f32x4{zx[4 * q], zx[4 * q + 1], zx[4 * q + 2], zx[4 * q + 3]};
        }
    }

    // dx through the gates: two passes over the LDS tiles (dz^a, then dz^x)
    const T *Wt_h = (const T *)p.Wt + (size_t)g * 131072;
    __syncthreads();   // every wave is done with the x tile
#pragma unroll
    for (int k = 0; k < 16; ++k) put_split(Xs, Zl, (16 * half + k) * S + ch, za[k]);
    __syncthreads();
    dx_tile(Xs, Zl, Wt_h, wave, lane, dxv);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) put_split(Xs, Zl, (16 * half + k) * S + ch, zx[k]);
    __syncthreads();
    dx_tile(Xs, Zl, Wt_h + 256, wave, lane, dxv);
#pragma unroll
    for (int k = 0; k < 16; ++k)
        if (tb + k >= p.T) dxv[k] = 0.0f;

    // conv backward: publish this chunk's first 3 dx before waiting for the next chunk's
    const long NW = (long)p.B * p.NC * p.D;
    if (half == 0) {
        put_word(p.halo + cidx, dxv[0], tag);
        put_word(p.halo + NW + cidx, dxv[1], tag);
        put_word(p.halo + 2 * NW + cidx, dxv[2], tag);
    }
    const float o0 = __shfl_xor(dxv[0], 32), o1 = __shfl_xor(dxv[1], 32), o2 = __shfl_xor(dxv[2], 32);
    float n0 = 0.0f, n1 = 0.0f, n2 = 0.0f;   // dx of the 3 tokens after the lane's 16
    if (half == 0) {
        n0 = o0;
        n1 = o1;
        n2 = o2;
    } else if (c + 1 < p.NC) {
        const long nidx = cidx + p.D;        // chunk c+1
        n0 = wait_word(p.halo + nidx, tag, p.hdr);
        n1 = wait_word(p.halo + NW + nidx, tag, p.hdr);
        n2 = wait_word(p.halo + 2 * NW + nidx, tag, p.hdr);
    }
    float ext[19];
#pragma unroll
    for (int k = 0; k < 16; ++k) ext[k] = dxv[k];
    ext[16] = n0;
    ext[17] = n1;
    ext[18] = n2;
    T *du = (T *)p.du;
    float s_cb = 0.0f, s_w0 = 0.0f, s_w1 = 0.0f, s_w2 = 0.0f, s_w3 = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        if (tb + k < p.T) {
            const float duk = fmaf(w0, ext[k + 3], fmaf(w1, ext[k + 2], fmaf(w2, ext[k + 1], w3 * ext[k])));
            du[(row_b + tb + k) * p.D + d] = from_f32<T>(duk);
        }
        s_cb += ext[k];
        s_w0 = fmaf(ext[k], win[k + 0], s_w0);
        s_w1 = fmaf(ext[k], win[k + 1], s_w1);
        s_w2 = fmaf(ext[k], win[k + 2], s_w2);
        s_w3 = fmaf(ext[k], win[k + 3], s_w3);
    }

    // per-chunk partial sums (half 0 + half 1), written by half 0
    float v[NSUM] = {s_w0, s_w1, s_w2, s_w3, s_cb, s_ba, s_bx, s_rl};
#pragma unroll
    for (int q = 0; q < NSUM; ++q) v[q] += __shfl_xor(v[q], 32);
    if (half == 0) {
        v[7] *= p.c * sgm;
        float4 *dst = (float4 *)(p.psum + cidx * NSUM);
        dst[0] = make_float4(v[0], v[1], v[2], v[3]);
        dst[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
    if (tid == 0) s_unit[(it + 1) & 1] = my_claim;   // read after the next barrier
    }   // units
    __syncthreads();
    finish_claimed(p.hdr, p.claim, p.G, s_unit + 2);
}

// ------------------------------------------------------------------ pass 4
// dW[q][o][j] over the row range of split s: sum_{units, t} dz_q[o][t] x[j][t].
// bf16 I/O: wave w owns rows o = 32w..32w+31 and all 256 columns (8 MFMA
// tiles); both operands are split into bf16 hi + lo and three products are
// accumulated (hi*hi + hi*lo + lo*hi).  Each unit's x tile is split once and
// staged in LDS for all 8 waves; the next unit's x and dz are requested while
// the current one is on the matrix cores.
constexpr int DW_XS = 40;   // LDS row stride (bf16) of a staged x tile: 32 tokens + 8 pad

__global__ __launch_bounds__(512) void dw_kernel_bf16(int units, int G, int S, const float *dZt,
                                                      const float *Xt, float *dWpart)
{
    // x of the current unit, split into bf16 hi and lo, [256 j][32 t] each
    __shared__ __attribute__((aligned(16))) bf16 Xh[256 * DW_XS], Xl[256 * DW_XS];
    const int g = blockIdx.x / 2, q = blockIdx.x % 2, s = blockIdx.y;
    const int u0 = (int)((long)units * s / S), u1 = (int)((long)units * (s + 1) / S);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 31, kg = lane >> 5;
    // staging: thread t splits x[j = t/2][16 (t&1) .. +15]
    const int sj = tid >> 1, st = 16 * (tid & 1);
    f32x16 acc[8];
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) acc[jt] = f32x16{};
    f32x4 xv[4], zv[2][2];
    auto fetch = [&](int un) {
        const float *xt = Xt + ((long)un * G + g) * 256 * 32 + sj * 32 + st;
#pragma unroll
        for (int e = 0; e < 4; ++e) xv[e] = *(const f32x4 *)(xt + 4 * e);
        const float *zt = dZt + (((long)un * G + g) * 2 + q) * 256 * 32 + (32 * wave + r) * 32 + 8 * kg;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            zv[ks][0] = *(const f32x4 *)(zt + 16 * ks);
            zv[ks][1] = *(const f32x4 *)(zt + 16 * ks + 4);
        }
    };
    if (u0 < u1) fetch(u0);
    for (int un = u0; un < u1; ++un) {
        // stage this unit's x (split) and take its dz operands
        bf16x8 hx[2], lx[2];
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float v = xv[e][c];
                const bf16 h = (bf16)v;
                hx[e >> 1][4 * (e & 1) + c] = h;
                lx[e >> 1][4 * (e & 1) + c] = (bf16)(v - (float)h);
            }
        bf16x8 ah[2], al[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = zv[ks][e >> 2][e & 3];
                const bf16 h = (bf16)v;
                ah[ks][e] = h;
                al[ks][e] = (bf16)(v - (float)h);
            }
        __syncthreads();   // every wave is done with the previous unit's tile
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            *(bf16x8 *)(Xh + sj * DW_XS + st + 8 * h2) = hx[h2];
            *(bf16x8 *)(Xl + sj * DW_XS + st + 8 * h2) = lx[h2];
        }
        __syncthreads();
        if (un + 1 < u1) fetch(un + 1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int jt = 0; jt < 8; ++jt) {
                const int off = (32 * jt + r) * DW_XS + 8 * kg + 16 * ks;
                const bf16x8 bh = *(const bf16x8 *)(Xh + off);
                const bf16x8 bl = *(const bf16x8 *)(Xl + off);
                acc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[ks], bh, acc[jt], 0, 0, 0);
                acc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[ks], bl, acc[jt], 0, 0, 0);
                acc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[ks], bh, acc[jt], 0, 0, 0);
            }
        }
    }
    float *dst = dWpart + (((long)s * G + g) * 2 + q) * 65536;
#pragma unroll
    for (int jt = 0; jt < 8; ++jt)
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int o = 32 * wave + 8 * (k >> 2) + 4 * kg + (k & 3);
            dst[o * 256 + jt * 32 + r] = acc[jt][k];
        }
}

// fp32: one thread per (o, j), rows in order
__global__ __launch_bounds__(256) void dw_kernel_f32(int units, int G, int S, const float *dZt,
                                                     const float *Xt, float *dWpart)
{
    const int gq = blockIdx.x / 256, o = blockIdx.x % 256, s = blockIdx.y;
    const int g = gq / 2, q = gq % 2, j = threadIdx.x;
    const int u0 = (int)((long)units * s / S), u1 = (int)((long)units * (s + 1) / S);
    float acc = 0.0f;
    for (int un = u0; un < u1; ++un) {
        const float *zt = dZt + (((long)un * G + g) * 2 + q) * 256 * 32 + o * 32;
        const float *xt = Xt + ((long)un * G + g) * 256 * 32 + j * 32;
        for (int t = 0; t < 32; ++t) acc = fmaf(zt[t], xt[t], acc);
    }
    dWpart[(((long)s * G + g) * 2 + q) * 65536 + o * 256 + j] = acc;
}

// ------------------------------------------------------------------ pass 5
__global__ __launch_bounds__(256) void dw_reduce_kernel(int G, int S, const float *dWpart, float *dWa,
                                                        float *dWx)
{
    const long e = (long)blockIdx.x * 256 + threadIdx.x;   // over G * 2 * 65536
    if (e >= (long)G * 2 * 65536) return;
    const int g = (int)(e / 131072), rem = (int)(e % 131072), q = rem / 65536, oj = rem % 65536;
    float acc = 0.0f;
    for (int s = 0; s < S; ++s) acc += dWpart[(((long)s * G + g) * 2 + q) * 65536 + oj];
    (q == 0 ? dWa : dWx)[(long)g * 65536 + oj] = acc;
}

// Per-chunk partial sums -> per-channel gradients, in two deterministic
// steps.  Step 1: workgroup (channel group of 32, unit split s) adds the
// units of its split; thread (l, c) takes units l, l+8, ... for channel c
// (32 consecutive channels read 1 KB contiguously), then the 8 threads of a
// channel are added in a fixed order through LDS.  Step 2 adds the splits in
// order.
__global__ __launch_bounds__(256) void psum_partial_kernel(int units, int D, const float *psum, float *part)
{
    __shared__ float red[8][32][NSUM + 1];
    const int c = threadIdx.x & 31, l = threadIdx.x >> 5;
    const int d = blockIdx.x * 32 + c;
    const int s = blockIdx.y;
    const int u0 = (int)((long)units * s / PS_SPLITS), u1 = (int)((long)units * (s + 1) / PS_SPLITS);
    float acc[NSUM] = {};
    if (d < D) {
        for (int un = u0 + l; un < u1; un += 8) {
            const float4 *src = (const float4 *)(psum + ((long)un * D + d) * NSUM);
            const float4 v0 = src[0], v1 = src[1];
            acc[0] += v0.x; acc[1] += v0.y; acc[2] += v0.z; acc[3] += v0.w;
            acc[4] += v1.x; acc[5] += v1.y; acc[6] += v1.z; acc[7] += v1.w;
        }
    }
#pragma unroll
    for (int q = 0; q < NSUM; ++q) red[l][c][q] = acc[q];
    __syncthreads();
    if (l == 0 && d < D) {
        float out[NSUM];
#pragma unroll
        for (int q = 0; q < NSUM; ++q) {
            float v = red[0][c][q];
            for (int k = 1; k < 8; ++k) v += red[k][c][q];
            out[q] = v;
        }
        float4 *dst = (float4 *)(part + ((long)s * D + d) * NSUM);
        dst[0] = make_float4(out[0], out[1], out[2], out[3]);
        dst[1] = make_float4(out[4], out[5], out[6], out[7]);
    }
}

__global__ __launch_bounds__(256) void psum_reduce_kernel(int D, const float *part, float *dcw, float *dcb,
                                                          float *dba, float *dbx, float *dLambda)
{
    const int d = blockIdx.x * 256 + threadIdx.x;
    if (d >= D) return;
    float acc[NSUM] = {};
    for (int s = 0; s < PS_SPLITS; ++s) {
        const float4 *src = (const float4 *)(part + ((long)s * D + d) * NSUM);
        const float4 v0 = src[0], v1 = src[1];
        acc[0] += v0.x; acc[1] += v0.y; acc[2] += v0.z; acc[3] += v0.w;
        acc[4] += v1.x; acc[5] += v1.y; acc[6] += v1.z; acc[7] += v1.w;
    }
    dcw[4 * (long)d + 0] = acc[0];
    dcw[4 * (long)d + 1] = acc[1];
    dcw[4 * (long)d + 2] = acc[2];
    dcw[4 * (long)d + 3] = acc[3];
    dcb[d] = acc[4];
    dba[d] = acc[5];
    dbx[d] = acc[6];
    dLambda[d] = acc[7];
}

// Per device: CU count and resident workgroups per CU of the chunk kernel,
// looked up once.
struct LaunchShape {
    int ncu = 0, occ = 0;
};

template <typename T>
LaunchShape bwd_shape(size_t shmem)
{
    static std::mutex mu;
    static LaunchShape cache[64];
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev < 0 || dev >= 64) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    LaunchShape &ls = cache[dev];
    if (ls.ncu == 0) {
        const void *fn = (const void *)&bwd_chunk_kernel<T>;
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

template <typename T>
void run_bwd(const rglru_desc &d, const rglru_weights &w, const void *u, const void *hist_in,
             const float *h0, const void *dy, const float *dh_last, void *du, float *dcw, float *dcb,
             float *dWa, float *dba, float *dWx, float *dbx, float *dLambda, float *dh0, void *ws,
             hipStream_t s)
{
    const BwdLayout L = bwd_layout(d.B, d.T, d.D, d.H, sizeof(T));
    char *base = (char *)ws;
    const int NC = (int)((d.T + CHUNK - 1) / CHUNK);
    const int G = (int)d.H;
    const size_t NW = (size_t)d.B * NC * d.D;

    // pass 1: states before each chunk (the forward kernel shares the header)
    float *hstart = (float *)(base + L.hstart);
    launch_fwd_states(d, w, u, hist_in, h0, hstart, ws, s);

    // pass 2
    T *Wt = (T *)(base + L.Wt);
    hipLaunchKernelGGL((transpose_w_kernel<T>), dim3(8, 16, G), dim3(256), 0, s, (const T *)w.W_a,
                       (const T *)w.W_x, Wt);

    // pass 3
    BwdParams p;
    p.B = (int)d.B;
    p.T = (int)d.T;
    p.D = (int)d.D;
    p.NC = NC;
    p.G = G;
    p.c = d.c;
    p.u = u;
    p.hist_in = hist_in;
    p.dy = dy;
    p.h0 = h0;
    p.dh_last = dh_last;
    p.cw = w.conv_w;
    p.cb = w.conv_b;
    p.ba = w.b_a;
    p.bx = w.b_x;
    p.Lambda = w.Lambda;
    p.Wa = w.W_a;
    p.Wx = w.W_x;
    p.Wt = Wt;
    p.hstart = hstart;
    p.du = du;
    p.dh0 = dh0;
    p.dZt = (float *)(base + L.dZt);
    p.Xt = (float *)(base + L.Xt);
    p.psum = (float *)(base + L.psum);
    p.hdr = (WsHeader *)ws;
    p.claim = (uint32_t *)(base + L.claims);
    p.units = (int)(d.B * NC);
    p.aggA = (uint64_t *)(base + L.bwd_words);
    p.aggX = p.aggA + NW;
    p.incl = p.aggX + NW;
    p.halo = p.incl + NW;
    {
        const size_t shmem = 2 * 32 * XTile<T>::STRIDE * sizeof(T) + 16;
        const LaunchShape ls = bwd_shape<T>(shmem);
        long wpg = ((long)ls.ncu * ls.occ) / G;   // workgroups per block
        if (wpg < 1) wpg = 1;
        if (wpg > p.units) wpg = p.units;
        bwd_chunk_kernel<T><<<dim3((unsigned)(G * wpg)), dim3(512), shmem, s>>>(p);
    }

    // pass 4
    const int chunks = (int)(d.B * NC);
    float *dWpart = (float *)(base + L.dWpart);
    if (sizeof(T) == 2)
        hipLaunchKernelGGL(dw_kernel_bf16, dim3(2 * G, L.S), dim3(512), 0, s, chunks, G, L.S,
                           (const float *)p.dZt, (const float *)p.Xt, dWpart);
    else
        hipLaunchKernelGGL(dw_kernel_f32, dim3(2 * G * 256, L.S), dim3(256), 0, s, chunks, G, L.S,
                           (const float *)p.dZt, (const float *)p.Xt, dWpart);

    // pass 5
    hipLaunchKernelGGL(dw_reduce_kernel, dim3((unsigned)((G * 2 * 65536 + 255) / 256)), dim3(256), 0, s,
                       G, L.S, (const float *)dWpart, dWa, dWx);
    float *ppart = (float *)(base + L.ppart);
    hipLaunchKernelGGL(psum_partial_kernel, dim3((unsigned)((d.D + 31) / 32), PS_SPLITS), dim3(256), 0, s,
                       chunks, (int)d.D, (const float *)p.psum, ppart);
    hipLaunchKernelGGL(psum_reduce_kernel, dim3((unsigned)((d.D + 255) / 256)), dim3(256), 0, s, (int)d.D,
                       (const float *)ppart, dcw, dcb, dba, dbx, dLambda);
}

}  // namespace

size_t bwd_workspace_bytes(int64_t B, int64_t T, int64_t D, int64_t H)
{
    return bwd_layout(B, T, D, H, 4).total;   // sized for fp32 I/O, enough for bf16 too
}

void launch_scan_bwd(const rglru_desc &d, const rglru_weights &w, const void *u, const void *hist_in,
                     const float *h0, const void *dy, const float *dh_last, void *du, float *dcw,
                     float *dcb, float *dWa, float *dba, float *dWx, float *dbx, float *dLambda,
                     float *dh0, void *ws, hipStream_t s)
{
    if (d.io == RGLRU_BF16)
        run_bwd<bf16>(d, w, u, hist_in, h0, dy, dh_last, du, dcw, dcb, dWa, dba, dWx, dbx, dLambda, dh0,
                      ws, s);
    else
        run_bwd<float>(d, w, u, hist_in, h0, dy, dh_last, du, dcw, dcb, dWa, dba, dWx, dbx, dLambda, dh0,
                       ws, s);
}

}  // namespace rglru
