// gates.hip -- a2: block-diagonal gates r = sigma(W_a x + b_a), i = sigma(W_x x + b_x).
//
// Page "Griffin Guide: RecurrentGemma, RG-LRU & Hybrid Attention": the
// recurrence-gate and input-gate equations of "Formulation of the RG-LRU
// Gating Mechanism", with W_a, W_x block-diagonal per "Block-Diagonal Sharding
// for Zero-Communication Tensor Parallelism" (blocks of K = 256 channels).
//
// One workgroup (8 waves) = one 32-row tile of the flattened [B*T] rows times
// one 256-channel block.  The tile is staged in LDS (16-byte loads of whole
// rows), the products run on the matrix cores (bf16) or on fp32 FMAs (fp32);
// lane l of wave w writes channel 32w + l%32 of rows 16(l/32) .. +15.
#include "common.h"
#include "gatemath.h"
#include "internal.h"

namespace rglru {

namespace {

template <typename T>
__global__ __launch_bounds__(512) void gates_kernel(long rows, int D, const T *x, const T *Wa,
                                                    const float *ba, const T *Wx,
                                                    const float *bx, T *r, T *i)
{
    constexpr int S = XTile<T>::STRIDE;
    constexpr int V = 16 / sizeof(T);
    __shared__ __attribute__((aligned(16))) T Xs[32 * S];
    const int g = blockIdx.y;
    const long row0 = (long)blockIdx.x * 32;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

    // stage 32 rows x 256 channels of block g
    for (int e = tid; e < 32 * (256 / V); e += 512) {
        const int rr = e / (256 / V), cv = e % (256 / V);
        uint4 v = {0u, 0u, 0u, 0u};
        if (row0 + rr < rows) v = *(const uint4 *)(x + (row0 + rr) * D + g * 256 + cv * V);
        *(uint4 *)(Xs + rr * S + cv * V) = v;
    }
    __syncthreads();

    float za[16], zx[16];
    gate_tile(Xs, Wa + (size_t)g * 65536, Wx + (size_t)g * 65536, wave, lane, za, zx);

    const int n = lane & 31, half = lane >> 5;
    const int d = g * 256 + 32 * wave + n;
    const float bav = ba ? ba[d] : 0.0f, bxv = bx ? bx[d] : 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const long row = row0 + 16 * half + k;
        if (row < rows) {
            r[row * D + d] = from_f32<T>(sigmoid_acc(za[k] + bav));
            i[row * D + d] = from_f32<T>(sigmoid_acc(zx[k] + bxv));
        }
    }
}

template <typename T>
void launch_gates_t(const rglru_desc &d, const rglru_weights &w, const void *x, void *r, void *i,
                    hipStream_t s)
{
    const long rows = d.B * d.T;
    const dim3 grid((unsigned)((rows + 31) / 32), (unsigned)d.H);
    hipLaunchKernelGGL((gates_kernel<T>), grid, dim3(512), 0, s, rows, (int)d.D, (const T *)x,
                       (const T *)w.W_a, w.b_a, (const T *)w.W_x, w.b_x, (T *)r, (T *)i);
}

}  // namespace

void launch_gates(const rglru_desc &d, const rglru_weights &w, const void *x, void *r, void *i,
                  hipStream_t s)
{
    if (d.io == RGLRU_BF16) launch_gates_t<bf16>(d, w, x, r, i, s);
    else launch_gates_t<float>(d, w, x, r, i, s);
}

}  // namespace rglru
