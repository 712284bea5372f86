// step.hip -- a6: one decode step for B independent streams.
//
// Page "Griffin Guide: RecurrentGemma, RG-LRU & Hybrid Attention": the
// listing's RGLRU.step (gates on the new token, decay, new state
// a_t h + sqrt(1 - a_t^2) i_t x_t returned as the output), preceded by the
// width-4 causal conv of "Temporal Filtering via Separable 1D Convolutions"
// evaluated on the carried 3-token history.
//
// A decode step is small (B x D elements, ~18 MB touched at B = 256,
// D = 2560, most of it resident in L2 / Infinity Cache between calls), so the
// kernel is shaped for parallelism and latency, not reuse: one workgroup
// (8 waves) per (16 streams, 256-channel block), 160 workgroups at B = 256,
// D = 2560.
//   1. every load is issued at once, in the order the values are needed:
//      the conv's inputs and taps, the gate weights the lane needs, then its
//      own outputs' state and gate biases -- 2 channels x 4 streams;
//   2. every thread computes the conv of 8 channels of one stream of the
//      block's input tile (16 streams x 256 channels) into LDS (bf16 for
//      the matrix cores, fp32 for the update), and the first 256 threads the
//      decay constant of one channel; after the barrier the same thread
//      writes its 8 channels of history back, shifted by one token;
//   3. bf16: wave w computes the gate products of output channels
//      32w .. 32w+31 (two 16-channel tiles) for the 16 streams with
//      v_mfma_f32_16x16x32_bf16 (A = x tile rows, B = W rows read from
//      memory), which leaves lane l with streams 4(l/16)+i of channels
//      32w + 16t + l%16; fp32: the same outputs by fp32 FMAs;
//   4. gates, decay, normalisation and the state update for those 8
//      elements; state and output are rewritten in place.
// A workgroup reads and rewrites the history of its own (streams, block)
// only, after the barrier that ends the reads of step 1.
#include "common.h"
#include "gatemath.h"
#include "internal.h"

namespace rglru {

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4v;

constexpr int SB = 16;   // streams per workgroup

__device__ __forceinline__ void load8(const bf16 *p, float v[8])
{
    const bf16x8 q = *(const bf16x8 *)p;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)q[e];
}

__device__ __forceinline__ void load8(const float *p, float v[8])
{
    const f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[e] = a[e];
        v[4 + e] = b[e];
    }
}

__device__ __forceinline__ void store8(bf16 *p, const float v[8])
{
    bf16x8 q;
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = (bf16)v[e];
    *(bf16x8 *)p = q;
}

__device__ __forceinline__ void store8(float *p, const float v[8])
{
    *(f32x4 *)p = f32x4{v[0], v[1], v[2], v[3]};
    *(f32x4 *)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// B operands of the lane's gate products: rows oc0 + 16t + l%16 of W_a and
// W_x, K-steps of 32 (lane group l/16 holds 8 consecutive inputs of a step);
// requested at kernel start so that their latency overlaps steps 1 and 2
template <typename T> struct WOps {
    bf16x8 a[2][8], x[2][8];
};
template <> struct WOps<float> {};

__device__ __forceinline__ void load_wops(WOps<bf16> &w, const bf16 *Wa_h, const bf16 *Wx_h, int oc0, int lane)
{
    const int m = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const bf16 *wa = Wa_h + (size_t)(oc0 + 16 * ct + m) * 256 + 8 * kq;
        const bf16 *wx = Wx_h + (size_t)(oc0 + 16 * ct + m) * 256 + 8 * kq;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            w.a[ct][ks] = *(const bf16x8 *)(wa + 32 * ks);
            w.x[ct][ks] = *(const bf16x8 *)(wx + 32 * ks);
        }
    }
}
__device__ __forceinline__ void load_wops(WOps<float> &, const float *, const float *, int, int) {}

// gate pre-activations of the lane's 8 outputs -- streams 4(l/16)+i (i < 4)
// of channels oc0 + 16t + l%16 (t < 2) -- bf16: two 16-channel tiles x
// 8 K-steps x 2 gates on the matrix cores; element e = 4t + i
__device__ __forceinline__ void step_gates(const bf16 *Xs, const WOps<bf16> &w, const bf16 *, const bf16 *,
                                           int, int lane, float za[8], float zx[8])
{
    constexpr int S = XTile<bf16>::STRIDE;
    const int m = lane & 15, kq = lane >> 4;
    const bf16 *xrow = Xs + m * S + 8 * kq;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        f32x4v A = {}, X = {};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const bf16x8 av = *(const bf16x8 *)(xrow + 32 * ks);
            A = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, w.a[ct][ks], A, 0, 0, 0);
            X = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, w.x[ct][ks], X, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            za[4 * ct + i] = A[i];
            zx[4 * ct + i] = X[i];
        }
    }
}

// fp32: the same outputs with fp32 FMAs in input-channel order
__device__ __forceinline__ void step_gates(const float *Xs, const WOps<float> &, const float *Wa_h,
                                           const float *Wx_h, int oc0, int lane, float za[8], float zx[8])
{
    constexpr int S = XTile<float>::STRIDE;
    const int m = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int e = 0; e < 8; ++e) za[e] = zx[e] = 0.0f;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const float *wa = Wa_h + (size_t)(oc0 + 16 * ct + m) * 256;
        const float *wx = Wx_h + (size_t)(oc0 + 16 * ct + m) * 256;
        for (int k = 0; k < 256; ++k) {
            const float a = wa[k], x = wx[k];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float xv = Xs[(4 * kq + i) * S + k];
                za[4 * ct + i] = fmaf(a, xv, za[4 * ct + i]);
                zx[4 * ct + i] = fmaf(x, xv, zx[4 * ct + i]);
            }
        }
    }
}

template <typename T>
__global__ __launch_bounds__(512) void step_kernel(int B, int D, float c, const T *u_t, const float *cw,
                                                   const float *cb, const T *Wa, const float *ba,
                                                   const T *Wx, const float *bx, const float *Lambda,
                                                   T *hist, float *hstate, T *y_t)
{
    constexpr int S = XTile<T>::STRIDE;
    constexpr int S32 = XTile<float>::STRIDE;
    __shared__ __attribute__((aligned(16))) T Xs[SB * S];          // conv output, MFMA operand
    __shared__ __attribute__((aligned(16))) float X32[SB * S32];   // the same in fp32
    __shared__ float ncs_s[256];   // -c softplus(-Lambda) of the block's channels
    // Workgroup id -> (stream tile, block), block-major over the XCDs:
    // consecutive ids go round-robin to the 8 XCDs, so ids that share id % 8
    // get consecutive (block, tile) pairs and each XCD's L2 holds the gate
    // weights of two or three blocks rather than all of them.  The map is a
    // permutation of the ids whatever the hardware does.
    const int nwg = gridDim.x, ntile = (B + SB - 1) / SB;
    const int xcd = blockIdx.x % 8, loc = blockIdx.x / 8;
    const int pair = xcd * (nwg / 8) + (xcd < nwg % 8 ? xcd : nwg % 8) + loc;
    const int sb0 = (pair % ntile) * SB, g = pair / ntile;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    // optional per-channel vectors: a null one reads a valid array and is
    // replaced by zeros, so that no load sits behind a branch
    const float *cbp = cb ? cb : Lambda, *bap = ba ? ba : Lambda, *bxp = bx ? bx : Lambda;

    // 1. every load, in the order the values are needed: the conv's inputs
    //    and taps (8 channels of one stream per thread), the gate weights of
    //    the lane's outputs, then the lane's outputs' state and gate biases
    //    -- element e = 4t + i is stream sb0 + 4(l/16) + i of channel
    //    oc0 + 16t + l%16 of the block.  Streams past B read stream B - 1 and
    //    are not stored.
    const int cg = tid & 31, sl = tid >> 5;
    const long sc = sb0 + sl < B ? sb0 + sl : B - 1;
    const int dc = g * 256 + 8 * cg;
    float a0[8], a1[8], a2[8], a3[8];
    load8(hist + (sc * 3 + 0) * D + dc, a0);
    load8(hist + (sc * 3 + 1) * D + dc, a1);
    load8(hist + (sc * 3 + 2) * D + dc, a2);
    load8(u_t + sc * D + dc, a3);
    f32x4 taps[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) taps[e] = *(const f32x4 *)(cw + 4 * (long)(dc + e));
    float cbv[8];
    load8(cbp + dc, cbv);
    const float lam = Lambda[g * 256 + (tid & 255)];   // used by the first 256 threads

    const int oc0 = 32 * wave;
    WOps<T> wop;
    load_wops(wop, Wa + (size_t)g * 65536, Wx + (size_t)g * 65536, oc0, lane);
    float hv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int s0 = sb0 + 4 * (lane >> 4) + (e & 3);
        const long s = s0 < B ? s0 : B - 1;
        hv[e] = hstate[s * D + g * 256 + oc0 + 16 * (e >> 2) + (lane & 15)];
    }
    float bav[2], bxv[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int d = g * 256 + oc0 + 16 * t + (lane & 15);
        bav[t] = bap[d];
        bxv[t] = bxp[d];
    }
    __builtin_amdgcn_sched_barrier(0);   // keep every request ahead of the first wait

    // 2. conv of the input tile into LDS; the decay constants of the block
    {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const f32x4 t = taps[e];
            const float bias = cb ? cbv[e] : 0.0f;
            x[e] = fmaf(t[3], a3[e], fmaf(t[2], a2[e], fmaf(t[1], a1[e], fmaf(t[0], a0[e], bias))));
        }
        store8(Xs + sl * S + 8 * cg, x);
        store8(X32 + sl * S32 + 8 * cg, x);
        const float ncs = -c * softplus_acc(-lam);
        if (tid < 256) ncs_s[tid] = ncs;
    }
    __syncthreads();   // the tiles are complete and every read of the history is done

    // the history moves one token on: the thread that read 8 channels of a
    // stream writes them back one position earlier, with the new input last
    if (sb0 + sl < B) {
        store8(hist + (sc * 3 + 0) * D + dc, a1);
        store8(hist + (sc * 3 + 1) * D + dc, a2);
        store8(hist + (sc * 3 + 2) * D + dc, a3);
    }

    // 3. gate pre-activations of the lane's outputs
    float za[8], zx[8];
    step_gates(Xs, wop, Wa + (size_t)g * 65536, Wx + (size_t)g * 65536, oc0, lane, za, zx);

    // 4. gates, decay, normalisation, state update
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int ch = oc0 + 16 * t + (lane & 15);
        const int d = g * 256 + ch;
        const float ncs = ncs_s[ch];
        const float bat = ba ? bav[t] : 0.0f, bxt = bx ? bxv[t] : 0.0f;
        const float kba = -LOG2E * bat, kbx = -LOG2E * bxt, kdec = LOG2E * ncs;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * t + i;
            const int sr = 4 * (lane >> 4) + i, s = sb0 + sr;
            const float x = X32[sr * S32 + ch];
            float a, bb;
            if constexpr (sizeof(T) == 2) {
                const float rr = hw_rcp(1.0f + hw_exp2(fmaf(za[e], -LOG2E, kba)));
                const float ii = hw_rcp(1.0f + hw_exp2(fmaf(zx[e], -LOG2E, kbx)));
                a = hw_exp2(rr * kdec);
                bb = hw_sqrt(fmaf(-a, a, 1.0f)) * ii * x;
            } else {
                const float rr = sigmoid_acc(za[e] + bat);
                const float ii = sigmoid_acc(zx[e] + bxt);
                const float l = ncs * rr;
                a = expf(l);
                bb = sqrtf(-expm1f(2.0f * l)) * ii * x;
            }
            const float hn = fmaf(a, hv[e], bb);
            if (s < B) {
                hstate[(long)s * D + d] = hn;
                y_t[(long)s * D + d] = from_f32<T>(hn);
            }
        }
    }
}

template <typename T>
void launch_step_t(const rglru_desc &d, const rglru_weights &w, const void *u_t, void *hist,
                   float *h, void *y_t, hipStream_t s)
{
    const dim3 grid((unsigned)(((d.B + SB - 1) / SB) * d.H));
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
