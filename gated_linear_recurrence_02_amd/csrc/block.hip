// block.hip -- the recurrent block around the RG-LRU (page "Griffin Guide:
// RecurrentGemma, RG-LRU & Hybrid Attention", section "The Recurrent Block
// Architecture", parts "Temporal Filtering via Separable 1D Convolutions" and
// "Non-Linear Multiplicative Gating with GeLU", and the RecurrentBlock class of
// its PyTorch listing): two bias-free input projections to the RG-LRU width D,
// conv + RG-LRU on branch 1, the exact (erf) GeLU of branch 2 multiplied in,
// and a bias-free output projection back to d_model.  The residual add belongs
// to the decoder layer, outside the block.
//
//   b1 = x proj_in_1^T        [B*T][D]    GEMM (gemm.hip)
//   b2 = x proj_in_2^T        [B*T][D]    GEMM
//   z  = RG-LRU(conv(b1)) * GeLU(b2)      the fused forward, mode 4 (the merge
//                                         happens where y would be stored; z
//                                         overwrites b2 in place: every element
//                                         of b2 is read by the lane that writes
//                                         z there, before it writes)
//   out = z proj_out^T        [B*T][d_model]  GEMM
//
// The projections are dense GEMMs on the matrix cores (gemm.hip: bf16
// inputs, fp32 accumulation, bf16 output for bf16 I/O; fp32 throughout for
// fp32 I/O).  Workspace: the scan's carries first (its header must start out
// zero), then b1 and b2.

#include "common.h"
#include "internal.h"

namespace rglru {

namespace {

size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

// ---------------------------------------------------------- residual layer
// Values of one 16-byte piece (8 bf16 or 4 fp32) as floats.
template <typename T> struct Piece;
template <> struct Piece<bf16> {
    static constexpr int N = 8;
    __device__ static void load(const bf16 *p, float *v)
    {
        const bf16x8 q = *(const bf16x8 *)p;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (float)q[i];
    }
    __device__ static void store(bf16 *p, const float *v)
    {
        bf16x8 q;
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = (bf16)v[i];
        *(bf16x8 *)p = q;
    }
};
template <> struct Piece<float> {
    static constexpr int N = 4;
    __device__ static void load(const float *p, float *v)
    {
        const f32x4 q = *(const f32x4 *)p;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = q[i];
    }
    __device__ static void store(float *p, const float *v) { *(f32x4 *)p = f32x4{v[0], v[1], v[2], v[3]}; }
};

// RMSNorm of one row per wave: out = x / sqrt(mean x^2 + eps) * (1 + w), fp32
// sums.  Rows whose width is a multiple of the 16-byte piece and at most
// 64 x 8 pieces stay in registers between the two passes; other widths read
// the row again (it is still in cache).
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(long M, int D, const T *x, const float *w, float eps, T *out)
{
    constexpr int N = Piece<T>::N, MAXP = 8;
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= M) return;
    const T *xr = x + row * D;
    T *orow = out + row * D;
    float ss = 0.0f;
    if (D % N == 0 && D <= 64 * N * MAXP) {
        const int np = D / N;
        float v[MAXP][N];
#pragma unroll
        for (int k = 0; k < MAXP; ++k) {
            const int pc = lane + 64 * k;
            if (pc < np) {
                Piece<T>::load(xr + pc * N, v[k]);
#pragma unroll
                for (int i = 0; i < N; ++i) ss = fmaf(v[k][i], v[k][i], ss);
            }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
        const float r = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
        for (int k = 0; k < MAXP; ++k) {
            const int pc = lane + 64 * k;
            if (pc < np) {
                float o[N];
#pragma unroll
                for (int i = 0; i < N; ++i) o[i] = v[k][i] * r * (1.0f + w[pc * N + i]);
                Piece<T>::store(orow + pc * N, o);
            }
        }
        return;
    }
    for (int d = lane; d < D; d += 64) {
        const float v = to_f32(xr[d]);
        ss = fmaf(v, v, ss);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    const float r = 1.0f / sqrtf(ss / (float)D + eps);
    for (int d = lane; d < D; d += 64) orow[d] = from_f32<T>(to_f32(xr[d]) * r * (1.0f + w[d]));
}

// g <- GELU_tanh(g) * u, in place, one 16-byte piece per thread (the width is
// a multiple of a piece; the tail thread-range covers the rest element-wise).
// GELU_tanh(v) = v sigma(2 sqrt(2/pi)(v + 0.044715 v^3)): the tanh form
// rewritten through 1 + tanh(a) = 2 sigma(2a), which has no cancellation for
// negative v.
__device__ __forceinline__ float gelu_tanh(float v)
{
    const float a2 = 1.5957691216057308f * fmaf(0.044715f * v, v * v, v);   // 2 sqrt(2/pi) (v + 0.044715 v^3)
    return v * hw_rcp(1.0f + hw_exp2(-a2 * LOG2E));
}

template <typename T>
__global__ __launch_bounds__(256) void gelu_tanh_mul_kernel(long n, T *g, const T *u)
{
    constexpr int N = Piece<T>::N;
    const long i = ((long)blockIdx.x * 256 + threadIdx.x) * N;
    if (i + N <= n) {
        float gv[N], uv[N];
        Piece<T>::load(g + i, gv);
        Piece<T>::load(u + i, uv);
#pragma unroll
        for (int k = 0; k < N; ++k) gv[k] = gelu_tanh(gv[k]) * uv[k];
        Piece<T>::store(g + i, gv);
    } else {
        for (long k = i; k < n; ++k) g[k] = from_f32<T>(gelu_tanh(to_f32(g[k])) * to_f32(u[k]));
    }
}

}  // namespace

BlockLayout block_layout(int64_t B, int64_t T, int64_t D, size_t esz)
{
    BlockLayout L;
    L.scan = 0;
    L.b1 = round256(fwd_workspace_bytes(B, T, D));
    L.b2 = L.b1 + round256((size_t)B * T * D * esz);
    L.bytes = L.b2 + round256((size_t)B * T * D * esz);
    return L;
}

namespace {

// out = block(x) (+ residual when given: the proj_out GEMM adds it)
int block_core(const rglru_desc &d, int64_t d_model, const rglru_weights &w, const rglru_block &blk,
               const void *x, const void *hist_in, const float *h0, void *out, const void *residual,
               float *h_last, void *hist_out, void *ws, hipStream_t s)
{
    const size_t esz = d.io == RGLRU_BF16 ? 2 : 4;
    const BlockLayout L = block_layout(d.B, d.T, d.D, esz);
    char *base = (char *)ws;
    void *b1 = base + L.b1, *b2 = base + L.b2;
    const int64_t M = d.B * d.T;
    {
        int st;
        if ((st = launch_gemm(d.io, M, d.D, d_model, x, blk.proj_in_1, nullptr, b1, s)) != RGLRU_OK) return st;
        if ((st = launch_gemm(d.io, M, d.D, d_model, x, blk.proj_in_2, nullptr, b2, s)) != RGLRU_OK) return st;
    }
    launch_scan_fwd_merge(d, w, b1, b2, hist_in, h0, b2, h_last, hist_out, base + L.scan, s);
    if (hipGetLastError() != hipSuccess) return RGLRU_ERR_LAUNCH;
    {
        int st;
        if ((st = launch_gemm(d.io, M, d_model, d.D, b2, blk.proj_out, residual, out, s)) != RGLRU_OK) return st;
    }
    return RGLRU_OK;
}

}  // namespace

int launch_block_fwd(const rglru_desc &d, int64_t d_model, const rglru_weights &w, const rglru_block &blk,
                     const void *x, const void *hist_in, const float *h0, void *out, float *h_last,
                     void *hist_out, void *ws, hipStream_t s)
{
    return block_core(d, d_model, w, blk, x, hist_in, h0, out, nullptr, h_last, hist_out, ws, s);
}

LayerLayout layer_layout(int64_t B, int64_t T, int64_t D, int64_t d_model, int64_t d_ff, size_t esz)
{
    LayerLayout L;
    L.block = 0;
    const size_t act = round256((size_t)B * T * d_model * esz), ff = round256((size_t)B * T * d_ff * esz);
    L.xn = block_layout(B, T, D, esz).bytes;
    L.xt = L.xn + act;
    L.g = L.xt + act;
    L.u = L.g + ff;
    L.bytes = L.u + ff;
    return L;
}

namespace {

int rmsnorm_launch(int io, long M, int64_t D, const void *x, const float *w, float eps, void *out, hipStream_t s)
{
    const unsigned grid = (unsigned)((M + 3) / 4);
    if (io == RGLRU_BF16)
        rmsnorm_kernel<bf16><<<grid, 256, 0, s>>>(M, (int)D, (const bf16 *)x, w, eps, (bf16 *)out);
    else
        rmsnorm_kernel<float><<<grid, 256, 0, s>>>(M, (int)D, (const float *)x, w, eps, (float *)out);
    return hipGetLastError() == hipSuccess ? RGLRU_OK : RGLRU_ERR_LAUNCH;
}

// y = x~ + down(GELU_tanh(gate RMSNorm(x~)) * up RMSNorm(x~)); xn, g, u are scratch
int mlp_tail(int io, long M, int64_t d_model, const rglru_layer &lw, const void *xt, void *xn, void *g, void *u,
             void *y, hipStream_t s)
{
    const size_t esz = io == RGLRU_BF16 ? 2 : 4;
    int st = rmsnorm_launch(io, M, d_model, xt, lw.cnorm_w, lw.eps, xn, s);
    if (st) return st;
    {
        int st;
        if ((st = launch_gemm(io, M, lw.d_ff, d_model, xn, lw.gate_w, nullptr, g, s)) != RGLRU_OK) return st;
        if ((st = launch_gemm(io, M, lw.d_ff, d_model, xn, lw.up_w, nullptr, u, s)) != RGLRU_OK) return st;
    }
    const long nff = M * lw.d_ff;
    const long pieces = (nff + (long)(16 / esz) - 1) / (long)(16 / esz);
    const unsigned ff_grid = (unsigned)((pieces + 255) / 256);
    if (io == RGLRU_BF16)
        gelu_tanh_mul_kernel<bf16><<<ff_grid, 256, 0, s>>>(nff, (bf16 *)g, (const bf16 *)u);
    else
        gelu_tanh_mul_kernel<float><<<ff_grid, 256, 0, s>>>(nff, (float *)g, (const float *)u);
    if (hipGetLastError() != hipSuccess) return RGLRU_ERR_LAUNCH;
    {
        int st;
        if ((st = launch_gemm(io, M, d_model, lw.d_ff, g, lw.down_w, xt, y, s)) != RGLRU_OK) return st;
    }
    return RGLRU_OK;
}

// Rotary embedding in place on x [M][H][dh]: row m has position pos0 + m % T;
// pairs (j, j + rot/2) turn by pos * base^(-2j/rot).  The angle is formed
// and reduced modulo 2 pi in double, so large positions keep their accuracy.
template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(long M, int T_, int H, int dh, int rot, double log2_base,
                                                   long pos0, T *x)
{
    const int half = rot / 2;
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= M * H * half) return;
    const int j = (int)(i % half);
    const long mh = i / half;   // row * H + head
    const long m = mh / H;
    const double pos = (double)(pos0 + m % T_);
    double ang = pos * exp2(-2.0 * j / rot * log2_base);
    ang -= 6.283185307179586 * floor(ang / 6.283185307179586);
    float sn, cs;
    sincosf((float)ang, &sn, &cs);
    T *v = x + mh * dh;
    const float a = to_f32(v[j]), b = to_f32(v[j + half]);
    v[j] = from_f32<T>(a * cs - b * sn);
    v[j + half] = from_f32<T>(a * sn + b * cs);
}

}  // namespace

AttnLayerLayout attn_layer_layout(const rglru_attn_desc &d, int64_t d_model, int64_t d_ff)
{
    const size_t esz = d.io == RGLRU_BF16 ? 2 : 4;
    const size_t M = d.B * d.T;
    AttnLayerLayout L;
    L.xn = 0;
    L.q = L.xn + round256(M * d_model * esz);
    L.k = L.q + round256(M * d.Hq * d.dh * esz);
    L.v = L.k + round256(M * d.dh * esz);
    L.o = L.v + round256(M * d.dh * esz);
    L.xt = L.o + round256(M * d.Hq * d.dh * esz);
    L.g = L.xt + round256(M * d_model * esz);
    L.u = L.g + round256(M * d_ff * esz);
    L.bytes = L.u + round256(M * d_ff * esz);
    return L;
}

int launch_attn_layer_fwd(const rglru_attn_desc &d, int64_t d_model, int rot, float rope_base, int64_t pos0,
                          const rglru_attn_proj &ap, const rglru_layer &lw, const void *x, void *y, void *kc,
                          void *vc, void *ws, hipStream_t s)
{
    const AttnLayerLayout L = attn_layer_layout(d, d_model, lw.d_ff);
    char *base = (char *)ws;
    void *xn = base + L.xn, *q = base + L.q, *k = base + L.k, *v = base + L.v, *o = base + L.o,
         *xt = base + L.xt, *g = base + L.g, *u = base + L.u;
    const long M = d.B * d.T;
    const int64_t HD = d.Hq * d.dh;
    int st = rmsnorm_launch(d.io, M, d_model, x, lw.tnorm_w, lw.eps, xn, s);
    if (st) return st;
    {
        int st;
        if ((st = launch_gemm(d.io, M, HD, d_model, xn, ap.wq, nullptr, q, s)) != RGLRU_OK) return st;
        if ((st = launch_gemm(d.io, M, d.dh, d_model, xn, ap.wk, nullptr, k, s)) != RGLRU_OK) return st;
        if ((st = launch_gemm(d.io, M, d.dh, d_model, xn, ap.wv, nullptr, v, s)) != RGLRU_OK) return st;
    }
    if (rot > 0) {
        const double l2b = log2((double)rope_base);
        const long nq = M * d.Hq * (rot / 2), nk = M * (rot / 2);
        if (d.io == RGLRU_BF16) {
            rope_kernel<bf16><<<(unsigned)((nq + 255) / 256), 256, 0, s>>>(M, (int)d.T, (int)d.Hq, (int)d.dh, rot,
                                                                          l2b, pos0, (bf16 *)q);
            rope_kernel<bf16><<<(unsigned)((nk + 255) / 256), 256, 0, s>>>(M, (int)d.T, 1, (int)d.dh, rot, l2b,
                                                                          pos0, (bf16 *)k);
        } else {
            rope_kernel<float><<<(unsigned)((nq + 255) / 256), 256, 0, s>>>(M, (int)d.T, (int)d.Hq, (int)d.dh, rot,
                                                                           l2b, pos0, (float *)q);
            rope_kernel<float><<<(unsigned)((nk + 255) / 256), 256, 0, s>>>(M, (int)d.T, 1, (int)d.dh, rot, l2b,
                                                                           pos0, (float *)k);
        }
        if (hipGetLastError() != hipSuccess) return RGLRU_ERR_LAUNCH;
    }
    launch_attn_fwd(d, q, k, v, o, kc, vc, s);
    if (hipGetLastError() != hipSuccess) return RGLRU_ERR_LAUNCH;
    {
        int st;
        if ((st = launch_gemm(d.io, M, d_model, HD, o, ap.wo, x, xt, s)) != RGLRU_OK) return st;
    }
    return mlp_tail(d.io, M, d_model, lw, xt, xn, g, u, y, s);
}

int launch_layer_fwd(const rglru_desc &d, int64_t d_model, const rglru_weights &w, const rglru_block &blk,
                     const rglru_layer &lw, const void *x, const void *hist_in, const float *h0, void *y,
                     float *h_last, void *hist_out, void *ws, hipStream_t s)
{
    const size_t esz = d.io == RGLRU_BF16 ? 2 : 4;
    const LayerLayout L = layer_layout(d.B, d.T, d.D, d_model, lw.d_ff, esz);
    char *base = (char *)ws;
    void *xn = base + L.xn, *xt = base + L.xt, *g = base + L.g, *u = base + L.u;
    const long M = d.B * d.T;
    // x~ = x + block(RMSNorm(x))
    int st = rmsnorm_launch(d.io, M, d_model, x, lw.tnorm_w, lw.eps, xn, s);
    if (st) return st;
    st = block_core(d, d_model, w, blk, xn, hist_in, h0, xt, x, h_last, hist_out, base + L.block, s);
    if (st) return st;
    // y = x~ + MLP(RMSNorm(x~))
    return mlp_tail(d.io, M, d_model, lw, xt, xn, g, u, y, s);
}

}  // namespace rglru
