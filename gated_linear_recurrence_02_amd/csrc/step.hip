// step.hip -- a6: one decode step for B independent streams.
//
// Page "Griffin Guide: RecurrentGemma, RG-LRU & Hybrid Attention": the
// listing's RGLRU.step (gates on the new token, decay, new state
// a_t h + sqrt(1 - a_t^2) i_t x_t returned as the output), preceded by the
// width-4 causal conv of "Temporal Filtering via Separable 1D Convolutions"
// evaluated on the carried 3-token history.
//
// One workgroup (8 waves) = 32 streams x one 256-channel block.  The streams
// play the role the tokens play in the prefill kernel: lane l = 32*half + n of
// wave w owns channel 256g + 32w + n of streams 32*blockIdx.x + 16*half .. +15.
// The conv runs in registers from the history, the conv outputs form the
// 32 x 256 LDS tile of the gate products, and the state, output and history
// are rewritten in place by the lane that read them.
#include "common.h"
#include "gatemath.h"
#include "internal.h"

namespace rglru {

namespace {

template <typename T>
__global__ __launch_bounds__(512) void step_kernel(int B, int D, float c, const T *u_t,
                                                   const float *cw, const float *cb, const T *Wa,
                                                   const float *ba, const T *Wx, const float *bx,
                                                   const float *Lambda, T *hist, float *hstate,
                                                   T *y_t)
{
    constexpr int S = XTile<T>::STRIDE;
    __shared__ __attribute__((aligned(16))) T Xs[32 * S];
    const int g = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 31, half = lane >> 5;
    const int d = g * 256 + wave * 32 + n;
    const int s0 = blockIdx.x * 32 + 16 * half;

    const float w0 = cw[4 * (long)d + 0], w1 = cw[4 * (long)d + 1];
    const float w2 = cw[4 * (long)d + 2], w3 = cw[4 * (long)d + 3];
    const float bias = cb ? cb[d] : 0.0f;

    float x[16];
    T hv0[16], hv1[16], hv2[16], uv[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int s = s0 + k;
        if (s < B) {
            hv0[k] = hist[((long)s * 3 + 0) * D + d];
            hv1[k] = hist[((long)s * 3 + 1) * D + d];
            hv2[k] = hist[((long)s * 3 + 2) * D + d];
            uv[k] = u_t[(long)s * D + d];
        } else {
            hv0[k] = hv1[k] = hv2[k] = uv[k] = from_f32<T>(0.0f);
        }
        x[k] = fmaf(w3, to_f32(uv[k]),
                    fmaf(w2, to_f32(hv2[k]), fmaf(w1, to_f32(hv1[k]), fmaf(w0, to_f32(hv0[k]), bias))));
        Xs[(16 * half + k) * S + wave * 32 + n] = from_f32<T>(x[k]);
    }
    __syncthreads();

    float za[16], zx[16];
    gate_tile(Xs, Wa + (size_t)g * 65536, Wx + (size_t)g * 65536, wave, lane, za, zx);

    const float ncs = -c * softplus_acc(-Lambda[d]);
    const float bav = ba ? ba[d] : 0.0f, bxv = bx ? bx[d] : 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int s = s0 + k;
        if (s >= B) continue;
        const float rr = sigmoid_acc(za[k] + bav);
        const float ii = sigmoid_acc(zx[k] + bxv);
        const float l = ncs * rr;
        const float a = expf(l);
        const float beta = sqrtf(-expm1f(2.0f * l));
        const float hn = fmaf(a, hstate[(long)s * D + d], beta * ii * x[k]);
        hstate[(long)s * D + d] = hn;
        y_t[(long)s * D + d] = from_f32<T>(hn);
        hist[((long)s * 3 + 0) * D + d] = hv1[k];
        hist[((long)s * 3 + 1) * D + d] = hv2[k];
        hist[((long)s * 3 + 2) * D + d] = uv[k];
    }
}

template <typename T>
void launch_step_t(const rglru_desc &d, const rglru_weights &w, const void *u_t, void *hist,
                   float *h, void *y_t, hipStream_t s)
{
    const dim3 grid((unsigned)((d.B + 31) / 32), (unsigned)d.H);
    hipLaunchKernelGGL((step_kernel<T>), grid, dim3(512), 0, s, (int)d.B, (int)d.D, d.c,
                       (const T *)u_t, w.conv_w, w.conv_b, (const T *)w.W_a, w.b_a,
                       (const T *)w.W_x, w.b_x, w.Lambda, (T *)hist, h, (T *)y_t);
}

}  // namespace

void launch_step(const rglru_desc &d, const rglru_weights &w, const void *u_t, void *hist,
                 float *h, void *y_t, hipStream_t s)
{
    if (d.io == RGLRU_BF16) launch_step_t<bf16>(d, w, u_t, hist, h, y_t, s);
    else launch_step_t<float>(d, w, u_t, hist, h, y_t, s);
}

}  // namespace rglru
