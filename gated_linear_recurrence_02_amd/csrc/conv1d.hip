// conv1d.hip -- a1: causal depthwise Conv1D of width 4 with bias.
//
// Page "Griffin Guide: RecurrentGemma, RG-LRU & Hybrid Attention", section
// "Temporal Filtering via Separable 1D Convolutions", and the listing's
// Conv1d(padding = 3, groups = channels) truncated to the first T outputs:
//     x[b][t][d] = conv_b[d] + sum_k conv_w[d][k] u[b][t-3+k][d]
// with positions < 0 taken from the carried history (zeros without one).
//
// HBM-bound streaming kernel.  One thread owns V channels (16 bytes of a row)
// of one stream over SEG consecutive tokens and slides the 4-tap window in
// registers, so every u row is read once per thread plus a 3-row halo.  Rows
// are read and written as 16-byte vectors; lanes of a wave cover consecutive
// channel groups, so a wave touches whole 1 KB row segments.  Whole segments
// request all their rows at once (SEG loads in flight per thread), which is
// what keeps enough bytes in flight to approach HBM bandwidth.  Outputs go out
// as nontemporal stores: nothing here reads them again, and streaming them
// past the caches measured 17% faster at 2B width than plain stores.
#include "common.h"
#include "internal.h"

namespace rglru {

namespace {

constexpr int SEG = 32;
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Vec;
template <> struct Vec<float> { static constexpr int N = 4; };
template <> struct Vec<bf16> { static constexpr int N = 8; };

template <typename T, bool VEC>
__device__ __forceinline__ void load_row(const T *u, const T *hist_in, int T_, int D, int b, int pos,
                                         int d0, int nv, float (&out)[Vec<T>::N])
{
    constexpr int V = Vec<T>::N;
    const T *src = nullptr;
    if (pos >= 0) src = u + ((long)b * T_ + pos) * D + d0;
    else if (hist_in) src = hist_in + ((long)b * 3 + 3 + pos) * D + d0;
    if (!src) {
#pragma unroll
        for (int v = 0; v < V; ++v) out[v] = 0.0f;
        return;
    }
    if (VEC) {
        T tmp[V];
        *(uint4 *)tmp = *(const uint4 *)src;
#pragma unroll
        for (int v = 0; v < V; ++v) out[v] = to_f32(tmp[v]);
    } else {
#pragma unroll
        for (int v = 0; v < V; ++v) out[v] = v < nv ? to_f32(src[v]) : 0.0f;
    }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(256) void conv1d_kernel(int B, int T_, int D, int nseg, const T *u,
                                                     const float *cw, const float *cb,
                                                     const T *hist_in, T *x, T *hist_out)
{
    constexpr int V = Vec<T>::N;
    const int G = (D + V - 1) / V;
    const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (long)B * nseg * G) return;
    const int g = (int)(gid % G);
    const long rest = gid / G;
    const int seg = (int)(rest % nseg);
    const int b = (int)(rest / nseg);
    const int d0 = g * V;
    const int nv = min(V, D - d0);

    float w[V][4], bias[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int d = min(d0 + v, D - 1);
        const f32x4 t4 = *(const f32x4 *)(cw + (long)d * 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) w[v][k] = t4[k];
        bias[v] = cb ? cb[d] : 0.0f;
    }

    const int t0 = seg * SEG;
    const int t1 = min(T_, t0 + SEG);
    float win[3][V];
#pragma unroll
    for (int m = 0; m < 3; ++m) load_row<T, VEC>(u, hist_in, T_, D, b, t0 - 3 + m, d0, nv, win[m]);

    auto step = [&](int t, const float (&cur)[V]) {
        T out[V];
#pragma unroll
        for (int v = 0; v < V; ++v) {
            float acc = fmaf(w[v][0], win[0][v], bias[v]);
            acc = fmaf(w[v][1], win[1][v], acc);
            acc = fmaf(w[v][2], win[2][v], acc);
            acc = fmaf(w[v][3], cur[v], acc);
            out[v] = from_f32<T>(acc);
            win[0][v] = win[1][v];
            win[1][v] = win[2][v];
            win[2][v] = cur[v];
        }
        T *dst = x + ((long)b * T_ + t) * D + d0;
        if (VEC) {
            __builtin_nontemporal_store(*(const nt_u32x4 *)out, (nt_u32x4 *)dst);
        } else {
#pragma unroll
            for (int v = 0; v < V; ++v)
                if (v < nv) dst[v] = out[v];
        }
    };
    if (VEC && t1 - t0 == SEG) {
        uint4 raw[SEG];
        const T *src = u + ((long)b * T_ + t0) * D + d0;
#pragma unroll
        for (int k = 0; k < SEG; ++k) raw[k] = *(const uint4 *)(src + (long)k * D);
#pragma unroll
        for (int k = 0; k < SEG; ++k) {
            const T *tmp = (const T *)&raw[k];
            float cur[V];
#pragma unroll
            for (int v = 0; v < V; ++v) cur[v] = to_f32(tmp[v]);
            step(t0 + k, cur);
        }
    } else {
        for (int t = t0; t < t1; ++t) {
            float cur[V];
            load_row<T, VEC>(u, hist_in, T_, D, b, t, d0, nv, cur);
            step(t, cur);
        }
    }

    // history out: the pre-conv inputs at T-3, T-2, T-1, copied bit for bit
    if (hist_out && t1 == T_) {
        for (int j = 0; j < 3; ++j) {
            const int pos = T_ - 3 + j;
            for (int v = 0; v < nv; ++v) {
                T val = from_f32<T>(0.0f);
                if (pos >= 0) val = u[((long)b * T_ + pos) * D + d0 + v];
                else if (hist_in) val = hist_in[((long)b * 3 + 3 + pos) * D + d0 + v];
                hist_out[((long)b * 3 + j) * D + d0 + v] = val;
            }
        }
    }
}

template <typename T>
void launch_conv_t(const rglru_desc &d, const float *cw, const float *cb, const void *u,
                   const void *hist_in, void *x, void *hist_out, hipStream_t s)
{
    constexpr int V = Vec<T>::N;
    const int B = (int)d.B, T_ = (int)d.T, D = (int)d.D;
    const int nseg = (T_ + SEG - 1) / SEG;
    const long threads = (long)B * nseg * ((D + V - 1) / V);
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (D % V == 0)
        hipLaunchKernelGGL((conv1d_kernel<T, true>), grid, dim3(256), 0, s, B, T_, D, nseg,
                           (const T *)u, cw, cb, (const T *)hist_in, (T *)x, (T *)hist_out);
    else
        hipLaunchKernelGGL((conv1d_kernel<T, false>), grid, dim3(256), 0, s, B, T_, D, nseg,
                           (const T *)u, cw, cb, (const T *)hist_in, (T *)x, (T *)hist_out);
}

}  // namespace

void launch_conv1d(const rglru_desc &d, const float *cw, const float *cb, const void *u,
                   const void *hist_in, void *x, void *hist_out, hipStream_t s)
{
    if (d.io == RGLRU_BF16) launch_conv_t<bf16>(d, cw, cb, u, hist_in, x, hist_out, s);
    else launch_conv_t<float>(d, cw, cb, u, hist_in, x, hist_out, s);
}

}  // namespace rglru
