// step.hip -- a6: one decode step for B independent streams.
//
// Page "Griffin Guide: RecurrentGemma, RG-LRU & Hybrid Attention": the
// listing's RGLRU.step (gates on the new token, decay, new state
// a_t h + sqrt(1 - a_t^2) i_t x_t returned as the output), preceded by the
// width-4 causal conv of "Temporal Filtering via Separable 1D Convolutions"
// evaluated on the carried 3-token history.
//
// A decode step is small (B x D elements, ~18 MB touched at B = 256,
// D = 2560, most of it resident in L2 / Infinity Cache between calls) and
// its time is latency: one global round trip, two barriers, a short
// matrix-core phase and the elementwise update.  One workgroup of 8 waves
// per (64 streams, 256-channel block g, 64 output channels oc0 .. oc0+63
// of the block): 4 x 10 x 4 = 160 workgroups at B = 256, D = 2560, one per
// CU.
//   1. every load is issued at once: the conv inputs of the 64 streams x
//      256 input channels of the block (history rows and the new token), the
//      block's conv taps and bias and the 64 rows of W_a and W_x of the
//      workgroup's outputs (both staged into LDS with global_load_lds, whole
//      1 KB pieces), and for each lane's own outputs the state and gate
//      biases;
//   2. after the first barrier: the conv of the input tile into LDS (bf16,
//      the matrix-core B operand; fp32 for the workgroup's own 64 channels,
//      which the update uses), the history of the own channels moved one
//      token on into hist_out, and -c softplus(-Lambda) of the own channels;
//   3. after the second: wave w computes the gate pre-activations of the 16
//      channels 16 (w % 4) .. +15 x the 32 streams 32 (w / 4) .. +31 with
//      v_mfma_f32_16x16x32_bf16 (fp32 I/O: the same outputs by fp32 FMAs);
//   4. gates, decay, normalisation, state update: 16-byte state loads and
//      stores, h rewritten in place, y stored.
// The 4 workgroups of one (streams, block) pair read the same inputs; the
// blockIdx -> work map puts them on one XCD so that its L2 serves the
// repeats.  History in and out are separate buffers: the other workgroups
// of the pair still read the old history of the channels whose new history
// a workgroup writes.
#include <mutex>

#include "common.h"
#include "internal.h"

namespace rglru {

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4v;

constexpr int SS = 64;            // streams per workgroup
constexpr int SC = 64;            // output channels per workgroup
constexpr int NSLICE = 256 / SC;  // workgroups per (streams, block) pair
constexpr int NT = 512;           // threads per workgroup

// LDS of one workgroup: the conv output tile (streams x 256 input channels,
// rows padded by 16 bytes), (bf16) the 2 x 64 weight rows and the fp32 conv
// output of the own channels, -c softplus(-Lambda) of the own channels, and
// the conv taps and bias of the block's 256 channels.  The weight rows are
// 512 bytes, unpadded, with the 16-byte slots of row r XOR-swizzled by
// r & 15, so that the 16 rows one operand read touches hit 16 different
// slots.
template <typename T> struct StepLds {
    static constexpr int V = 16 / sizeof(T);       // elements per 16-byte vector
    static constexpr int XS = 256 + V;             // padded row stride
    static constexpr int X32S = SC + 4;
    T x[SS * XS];
    bf16 w[sizeof(T) == 2 ? 2 * SC * 256 : 8];
    float x32[sizeof(T) == 2 ? SS * X32S : 4];
    float ncs[SC];
    f32x4 taps[256];
    float cb[256];
};

template <typename T> struct StepParams {
    int B, D;
    float c;
    const T *u_t, *hist_in;
    T *hist_out;
    const float *cw, *cb;
    const T *Wa, *Wx;
    const float *ba, *bx, *Lambda;
    float *h;
    T *y;
};

template <typename T> struct Vec;
template <> struct Vec<bf16> { typedef bf16x8 type; };
template <> struct Vec<float> { typedef f32x4 type; };

template <typename T>
__device__ __forceinline__ void to_f32(const typename Vec<T>::type &q, float *v)
{
#pragma unroll
    for (int e = 0; e < StepLds<T>::V; ++e) v[e] = (float)q[e];
}

typedef __attribute__((address_space(3))) void lds_void;
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int nt_u32x2 __attribute__((ext_vector_type(2)));

// Outputs are streamed past L2 (nontemporal): nothing in the step reads
// them again, and dirty lines left in L2 would be written back at the end
// of every step.
template <typename V16> __device__ __forceinline__ void nt_store16(void *dst, const V16 &v)
{
    static_assert(sizeof(V16) == 16, "16-byte store");
    __builtin_nontemporal_store(__builtin_bit_cast(nt_u32x4, v), (nt_u32x4 *)dst);
}
template <typename V8> __device__ __forceinline__ void nt_store8(void *dst, const V8 &v)
{
    static_assert(sizeof(V8) == 8, "8-byte store");
    __builtin_nontemporal_store(__builtin_bit_cast(nt_u32x2, v), (nt_u32x2 *)dst);
}

// softplus(v) = max(v, 0) + log1p(e^-|v|) for the bf16 path, from the
// hardware exp2 and reciprocal: e^-|v| with the rounding of |v| log2(e)
// corrected to first order, then log1p(z) = 2 atanh(s), s = z / (2 + z)
// <= 1/3, by its odd series to s^15 (truncation below 2^-29 relative).
// Relative error a few ulp, uniformly in v.
__device__ __forceinline__ float softplus_fast(float v)
{
    constexpr float LOG2E_LO = 1.925963033500011e-8f;   // log2(e) - LOG2E
    constexpr float LN2 = 0.6931471805599453f;
    const float x = -fabsf(v);
    const float t = x * LOG2E;
    const float err = fmaf(x, LOG2E, -t) + x * LOG2E_LO;   // x log2(e) - t
    const float z = hw_exp2(t) * fmaf(err, LN2, 1.0f);
    const float sv = z * hw_rcp(2.0f + z);
    const float s2 = sv * sv;
    float q = 2.0f / 15.0f;
    q = fmaf(q, s2, 2.0f / 13.0f);
    q = fmaf(q, s2, 2.0f / 11.0f);
    q = fmaf(q, s2, 2.0f / 9.0f);
    q = fmaf(q, s2, 2.0f / 7.0f);
    q = fmaf(q, s2, 2.0f / 5.0f);
    q = fmaf(q, s2, 2.0f / 3.0f);
    q = fmaf(q, s2, 2.0f);
    return fmaxf(v, 0.0f) + sv * q;
}

template <typename T>
__global__ __launch_bounds__(NT) void step_kernel(StepParams<T> p)
{
    typedef typename Vec<T>::type vec;
    constexpr int V = StepLds<T>::V, XS = StepLds<T>::XS, X32S = StepLds<T>::X32S;
    constexpr int NG = 256 / V;         // channel groups of one stream row
    constexpr int RS = NT / NG;         // stream rows one pass of the workgroup covers
    constexpr int SPT = SS / RS;        // streams per thread in the conv
    extern __shared__ __attribute__((aligned(16))) char smem[];
    StepLds<T> &L = *reinterpret_cast<StepLds<T> *>(smem);

    const int B = p.B, D = p.D;
    // Workgroup id -> (stream tile, block, channel slice).  Consecutive ids
    // go round-robin to the 8 XCDs; `lin` renumbers them so that ids sharing
    // an XCD get consecutive numbers, and the slices of one (tile, block)
    // pair have consecutive numbers.  A permutation of the ids whatever the
    // hardware does.
    const int nwg = gridDim.x, ntile = (B + SS - 1) / SS;
    const int xcd = blockIdx.x % 8, loc = blockIdx.x / 8;
    const int lin = xcd * (nwg / 8) + (xcd < nwg % 8 ? xcd : nwg % 8) + loc;
    const int pair = lin / NSLICE, oc0 = (lin % NSLICE) * SC;
    const int sb0 = (pair % ntile) * SS, g = pair / ntile;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int m = lane & 15, kq = lane >> 4;
    const long gb = (long)g * 256;

    // 1. loads, all issued before the first wait.
    //  - conv taps and bias of the block's channels into LDS (one 1 KB wave
    //    instruction each: wave w < 4 the taps of channels 64w .. 64w+63,
    //    wave 4 the bias);
    if (wave < 4)
        __builtin_amdgcn_global_load_lds((const void *)(p.cw + 4 * (gb + tid)), (lds_void *)(L.taps + 64 * wave),
                                         16, 0, 0);
    if (p.cb) {
        if (wave == 4)
            __builtin_amdgcn_global_load_lds((const void *)(p.cb + gb + 4 * lane), (lds_void *)L.cb, 16, 0, 0);
    } else if (tid < 256) {
        L.cb[tid] = 0.0f;
    }
    //  - conv inputs: thread t covers channels V cg .. V cg + V-1 of streams
    //    sb0 + sl + RS j (j < SPT); streams past B read stream B-1 and store
    //    nothing;
    const int cg = tid % NG, sl = tid / NG;
    const long dc = gb + V * cg;
    vec hv[SPT][4];
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        const int s0 = sb0 + sl + RS * j;
        const long s = s0 < B ? s0 : B - 1;
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            if (p.hist_in) hv[j][r] = *(const vec *)(p.hist_in + (s * 3 + r) * D + dc);
            else hv[j][r] = vec{};
        }
        hv[j][3] = *(const vec *)(p.u_t + s * D + dc);
    }
    //  - bf16: the weight rows oc0 .. oc0+63 of block g, both gates, in 64
    //    wave instructions of two rows each, 8 per wave: instruction n stages
    //    rows 2(n % 32), +1 of gate n / 32; lane l the slot l % 32 of row
    //    2(n % 32) + l / 32, which holds column vector slot ^ (row & 15);
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int n = 8 * k + wave, gate = n >> 5, r = 2 * (n & 31) + (lane >> 5);
            const int cv = (lane & 31) ^ (r & 15);
            const T *src = (gate ? p.Wx : p.Wa) + (size_t)g * 65536 + (size_t)(oc0 + r) * 256 + 8 * cv;
            __builtin_amdgcn_global_load_lds((const void *)src, (lds_void *)(L.w + (gate * SC + 2 * (n & 31)) * 256),
                                             16, 0, 0);
        }
    }
    //  - the lane's outputs: channels oc0 + 16 ct + 4 kq + r (ct = wave % 4,
    //    r < 4) of the block for streams sb0 + 16 st + m (st = 2 (wave / 4)
    //    and + 1): state and gate biases as 16-byte vectors; Lambda of
    //    channel oc0 + tid (tid < SC)
    const int ct = wave & 3, st0 = 2 * (wave >> 2);
    const int cl = 16 * ct + 4 * kq;   // first channel of the lane in the slice
    const long dl = gb + oc0 + cl;
    f32x4 hs[2];
    long srow[2];
    int so[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        so[st] = sb0 + 16 * (st0 + st) + m;
        srow[st] = (long)(so[st] < B ? so[st] : B - 1) * D;
        hs[st] = *(const f32x4 *)(p.h + srow[st] + dl);
    }
    const f32x4 bav = p.ba ? *(const f32x4 *)(p.ba + dl) : f32x4{};
    const f32x4 bxv = p.bx ? *(const f32x4 *)(p.bx + dl) : f32x4{};
    const float lam = tid < SC ? p.Lambda[gb + oc0 + tid] : 0.0f;
    // every staged byte has landed (and the conv inputs with it)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // 2. conv into LDS; the own channels' history moved on into hist_out;
    //    the decay constants of the own channels
    const bool own = V * cg >= oc0 && V * cg < oc0 + SC;
    {
        f32x4 taps[V];
        float cbv[V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
            taps[e] = L.taps[V * cg + e];
            cbv[e] = L.cb[V * cg + e];
        }
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            const int sr = sl + RS * j;
            float a[4][V], x[V];
#pragma unroll
            for (int r = 0; r < 4; ++r) to_f32<T>(hv[j][r], a[r]);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const f32x4 t = taps[e];
                x[e] = fmaf(t[3], a[3][e], fmaf(t[2], a[2][e], fmaf(t[1], a[1][e], fmaf(t[0], a[0][e], cbv[e]))));
            }
            vec q;
#pragma unroll
            for (int e = 0; e < V; ++e) q[e] = from_f32<T>(x[e]);
            *(vec *)(L.x + sr * XS + V * cg) = q;
            if constexpr (sizeof(T) == 2) {
                if (own) {
                    float *dst = L.x32 + sr * X32S + (V * cg - oc0);
                    *(f32x4 *)dst = f32x4{x[0], x[1], x[2], x[3]};
                    *(f32x4 *)(dst + 4) = f32x4{x[4], x[5], x[6], x[7]};
                }
            }
            if (own && p.hist_out && sb0 + sr < B) {
                const long s = sb0 + sr;
                nt_store16(p.hist_out + (s * 3 + 0) * D + dc, hv[j][1]);
                nt_store16(p.hist_out + (s * 3 + 1) * D + dc, hv[j][2]);
                nt_store16(p.hist_out + (s * 3 + 2) * D + dc, hv[j][3]);
            }
        }
    }
    if (tid < SC) L.ncs[tid] = -p.c * (sizeof(T) == 2 ? softplus_fast(-lam) : softplus_acc(-lam));
    // LDS only: the history stores need not have completed
    lds_barrier();

    // 3. gate pre-activations z[st][r]: channel cl + r of the slice, stream
    //    16 (st0 + st) + m of the tile (weight rows = A operand, conv outputs
    //    = B)
    float za[2][4], zx[2][4];
    if constexpr (sizeof(T) == 2) {
        f32x4v A[2] = {}, X[2] = {};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int slot = (kq + 4 * ks) ^ m;   // row 16 ct + m: swizzled by m
            const bf16x8 wa = *(const bf16x8 *)(L.w + (16 * ct + m) * 256 + 8 * slot);
            const bf16x8 wx = *(const bf16x8 *)(L.w + (SC + 16 * ct + m) * 256 + 8 * slot);
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const bf16x8 xv = *(const bf16x8 *)(L.x + (16 * (st0 + st) + m) * XS + 8 * kq + 32 * ks);
                A[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, xv, A[st], 0, 0, 0);
                X[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wx, xv, X[st], 0, 0, 0);
            }
        }
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                za[st][r] = A[st][r];
                zx[st][r] = X[st][r];
            }
    } else {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int r = 0; r < 4; ++r) za[st][r] = zx[st][r] = 0.0f;
        const size_t wrow = (size_t)g * 65536 + (size_t)(oc0 + cl) * 256;
        for (int k = 0; k < 256; k += 4) {
            f32x4 xv[2], wav[4], wxv[4];
#pragma unroll
            for (int st = 0; st < 2; ++st) xv[st] = *(const f32x4 *)(L.x + (16 * (st0 + st) + m) * XS + k);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                wav[r] = *(const f32x4 *)(p.Wa + wrow + (size_t)r * 256 + k);
                wxv[r] = *(const f32x4 *)(p.Wx + wrow + (size_t)r * 256 + k);
            }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        za[st][r] = fmaf(wav[r][kk], xv[st][kk], za[st][r]);
                        zx[st][r] = fmaf(wxv[r][kk], xv[st][kk], zx[st][r]);
                    }
        }
    }

    // 4. gates, decay, normalisation, state update
    const f32x4 ncs = *(const f32x4 *)(L.ncs + cl);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        const int sr = 16 * (st0 + st) + m;
        f32x4 xs;
        if constexpr (sizeof(T) == 2) xs = *(const f32x4 *)(L.x32 + sr * X32S + cl);
        else xs = *(const f32x4 *)(L.x + sr * XS + oc0 + cl);
        f32x4 hn;
        vec yq{};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float a, bb;
            if constexpr (sizeof(T) == 2) {
                const float rr = hw_rcp(1.0f + hw_exp2((za[st][r] + bav[r]) * -LOG2E));
                const float ii = hw_rcp(1.0f + hw_exp2((zx[st][r] + bxv[r]) * -LOG2E));
                a = hw_exp2(rr * (LOG2E * ncs[r]));
                bb = hw_sqrt(fmaf(-a, a, 1.0f)) * ii * xs[r];
            } else {
                const float rr = sigmoid_acc(za[st][r] + bav[r]);
                const float ii = sigmoid_acc(zx[st][r] + bxv[r]);
                const float l = ncs[r] * rr;
                a = expf(l);
                bb = sqrtf(-expm1f(2.0f * l)) * ii * xs[r];
            }
            hn[r] = fmaf(a, hs[st][r], bb);
            yq[r] = from_f32<T>(hn[r]);
        }
        if (so[st] < B) {
            nt_store16(p.h + srow[st] + dl, hn);
            if constexpr (sizeof(T) == 2) {
                typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
                nt_store8(p.y + srow[st] + dl, bf16x4{yq[0], yq[1], yq[2], yq[3]});
            } else {
                nt_store16(p.y + srow[st] + dl, f32x4{yq[0], yq[1], yq[2], yq[3]});
            }
        }
    }
}

// the kernels' LDS exceeds the default limit: raise it once per device
template <typename T> void step_lds_attribute()
{
    static std::mutex mu;
    static bool done[64];
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev < 0 || dev >= 64) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    if (!done[dev]) {
        // a failure here surfaces through the launch and hipGetLastError
        (void)hipFuncSetAttribute((const void *)&step_kernel<T>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)sizeof(StepLds<T>));
        done[dev] = true;
    }
}

template <typename T>
void launch_step_t(const rglru_desc &d, const rglru_weights &w, const void *u_t, const void *hist_in,
                   void *hist_out, float *h, void *y_t, hipStream_t s)
{
    StepParams<T> p;
    p.B = (int)d.B;
    p.D = (int)d.D;
    p.c = d.c;
    p.u_t = (const T *)u_t;
    p.hist_in = (const T *)hist_in;
    p.hist_out = (T *)hist_out;
    p.cw = w.conv_w;
    p.cb = w.conv_b;
    p.Wa = (const T *)w.W_a;
    p.Wx = (const T *)w.W_x;
    p.ba = w.b_a;
    p.bx = w.b_x;
    p.Lambda = w.Lambda;
    p.h = h;
    p.y = (T *)y_t;
    step_lds_attribute<T>();
    const dim3 grid((unsigned)(((d.B + SS - 1) / SS) * d.H * NSLICE));
    step_kernel<T><<<grid, dim3(NT), sizeof(StepLds<T>), s>>>(p);
}

}  // namespace

void launch_step(const rglru_desc &d, const rglru_weights &w, const void *u_t, const void *hist_in,
                 void *hist_out, float *h, void *y_t, hipStream_t s)
{
    if (d.io == RGLRU_BF16) launch_step_t<bf16>(d, w, u_t, hist_in, hist_out, h, y_t, s);
    else launch_step_t<float>(d, w, u_t, hist_in, hist_out, h, y_t, s);
}

}  // namespace rglru
