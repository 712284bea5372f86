// gates.hip -- a2: block-diagonal gates r = sigma(W_a x + b_a), i = sigma(W_x x + b_x).
//
// Page "Griffin Guide: RecurrentGemma, RG-LRU & Hybrid Attention": the
// recurrence-gate and input-gate equations of "Formulation of the RG-LRU
// Gating Mechanism", with W_a, W_x block-diagonal per "Block-Diagonal Sharding
// for Zero-Communication Tensor Parallelism" (blocks of K = 256 channels).
//
// bf16: a persistent kernel like the fused forward -- one workgroup (8 waves)
// per CU serves one 256-channel block g = w % G with the block's W_a and W_x
// held in registers (wave w: rows 32w..32w+31, 128 VGPRs) and walks the
// 32-row tiles of the flattened [B*T] rows assigned to it (tile q,
// q + WPG, ...; no tile waits on another).  The next tile is requested into
// registers (two 16-byte loads per thread) while the current one is on the
// matrix cores; tiles alternate between two LDS buffers.  Lane l of wave w
// gets channel 32w + l%32 of rows 16(l/32) .. +15 back from the MFMA output
// layout; r and i go through an LDS output tile ([token][channel]) and leave
// in 16-byte nontemporal stores rather than as 2-byte stores (streaming them
// past the caches measured 5% faster at 2B width).
// fp32: one workgroup per (tile, block); the tile is staged in LDS and the
// products run on fp32 FMAs.
#include "common.h"
#include "gatemath.h"
#include "internal.h"

namespace rglru {

namespace {

typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));   // nontemporal stores

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

// bf16, persistent and weight-stationary
__global__ __launch_bounds__(512) void gates_kernel_w(long rows, int D, int G, int wpg, const bf16 *x,
                                                      const bf16 *Wa, const float *ba, const bf16 *Wx,
                                                      const float *bx, bf16 *r, bf16 *i)
{
    constexpr int S = XTile<bf16>::STRIDE;
    constexpr int OS = 264;   // output tile row stride (bf16): 256 channels + 8 pad
    __shared__ __attribute__((aligned(16))) bf16 Xs[2][32 * S];
    __shared__ __attribute__((aligned(16))) bf16 Os[2][32 * OS];   // r and i of the tile, [token][channel]
    // (the output tile is rewritten only after the next tile's barrier, which
    // every thread reaches after its reads of it)
    const int g = blockIdx.x % G, rank = blockIdx.x / G;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 31, half = lane >> 5;
    const int d = g * 256 + 32 * wave + n;
    const long ntiles = (rows + 31) / 32;

    bf16x8 wa[16], wx[16];
    {
        const int rr = lane & 31, kg = lane >> 5;
        const bf16 *pa = Wa + (size_t)g * 65536 + (size_t)(32 * wave + rr) * 256 + 8 * kg;
        const bf16 *px = Wx + (size_t)g * 65536 + (size_t)(32 * wave + rr) * 256 + 8 * kg;
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2) {
            wa[s2] = *(const bf16x8 *)(pa + 16 * s2);
            wx[s2] = *(const bf16x8 *)(px + 16 * s2);
        }
    }
    const float kba = -LOG2E * (ba ? ba[d] : 0.0f), kbx = -LOG2E * (bx ? bx[d] : 0.0f);

    // thread t moves 16 bytes of rows t/32 and t/32 + 16 (channels 8(t%32) .. +7)
    const int lr = tid >> 5, lc = 8 * (tid & 31);
    auto fetch = [&](long q, uint4 v[2]) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const long row = q * 32 + lr + 16 * h;
            v[h] = row < rows ? *(const uint4 *)(x + row * D + g * 256 + lc) : uint4{0u, 0u, 0u, 0u};
        }
    };
    uint4 cur[2];
    long q = rank;
    if (q < ntiles) fetch(q, cur);
    for (int it = 0; q < ntiles; q += wpg, ++it) {
        bf16 *X = Xs[it & 1];
#pragma unroll
        for (int h = 0; h < 2; ++h) *(uint4 *)(X + (lr + 16 * h) * S + lc) = cur[h];
        __syncthreads();   // the tile is in LDS; the other buffer's readers are done
        if (q + wpg < ntiles) fetch(q + wpg, cur);

        const int rr = lane & 31, kg = lane >> 5;
        const bf16 *xrow = X + tile_row_token(rr) * S + 8 * kg;
        f32x16 A = {}, Xc = {};
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2) {
            const bf16x8 av = *(const bf16x8 *)(xrow + 16 * s2);
            A = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, wa[s2], A, 0, 0, 0);
            Xc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, wx[s2], Xc, 0, 0, 0);
        }
        // r and i to the output tile, then out in 16-byte pieces
        {
            uint32_t oo = (uint32_t)(16 * half * OS + 32 * wave + n);
            asm volatile("" : "+v"(oo));
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                Os[0][oo + k * OS] = (bf16)hw_rcp(1.0f + hw_exp2(fmaf(A[k], -LOG2E, kba)));
                Os[1][oo + k * OS] = (bf16)hw_rcp(1.0f + hw_exp2(fmaf(Xc[k], -LOG2E, kbx)));
            }
        }
        __syncthreads();   // the output tile is complete
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const long row = q * 32 + lr + 16 * h;
            if (row < rows) {
                __builtin_nontemporal_store(*(const nt_u32x4 *)(&Os[0][(lr + 16 * h) * OS + lc]),
                                            (nt_u32x4 *)(r + row * D + g * 256 + lc));
                __builtin_nontemporal_store(*(const nt_u32x4 *)(&Os[1][(lr + 16 * h) * OS + lc]),
                                            (nt_u32x4 *)(i + row * D + g * 256 + lc));
            }
        }
    }
}

template <typename T>
void launch_gates_t(const rglru_desc &d, const rglru_weights &w, const void *x, void *r, void *i,
                    hipStream_t s)
{
    const long rows = d.B * d.T;
    if constexpr (sizeof(T) == 2) {
        int dev = 0, ncu = 0;
        (void)hipGetDevice(&dev);
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
        if (ncu < 1) ncu = 1;
        const long ntiles = (rows + 31) / 32;
        long wpg = ncu / d.H;   // one workgroup per CU
        if (wpg < 1) wpg = 1;
        if (wpg > ntiles) wpg = ntiles;
        hipLaunchKernelGGL(gates_kernel_w, dim3((unsigned)(d.H * wpg)), dim3(512), 0, s, rows, (int)d.D,
                           (int)d.H, (int)wpg, (const bf16 *)x, (const bf16 *)w.W_a, w.b_a,
                           (const bf16 *)w.W_x, w.b_x, (bf16 *)r, (bf16 *)i);
    } else {
        const dim3 grid((unsigned)((rows + 31) / 32), (unsigned)d.H);
        hipLaunchKernelGGL((gates_kernel<T>), grid, dim3(512), 0, s, rows, (int)d.D, (const T *)x,
                           (const T *)w.W_a, w.b_a, (const T *)w.W_x, w.b_x, (T *)r, (T *)i);
    }
}

}  // namespace

void launch_gates(const rglru_desc &d, const rglru_weights &w, const void *x, void *r, void *i,
                  hipStream_t s)
{
    if (d.io == RGLRU_BF16) launch_gates_t<bf16>(d, w, x, r, i, s);
    else launch_gates_t<float>(d, w, x, r, i, s);
}

}  // namespace rglru
