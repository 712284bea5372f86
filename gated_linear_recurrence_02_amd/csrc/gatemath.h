// gatemath.h -- the block-diagonal gate products on one 32-token tile.
//
// A workgroup of 8 waves covers one 256-channel block h.  The 32 x 256 input
// tile X (tokens x input channels of block h) sits in LDS; wave w produces the
// pre-activations of output channels 32w .. 32w+31 for both gates:
//     za[k] = sum_j W_a[h][32w + n][j] X[tok][j],  zx likewise with W_x,
// for lane l = 32*half + n and tok = 16*half + k (k = 0..15).
//
// bf16: two v_mfma_f32_32x32x16_bf16 per 16-wide K step (one per gate); the A
// operand is the X tile (rows permuted by tile_row_token so that each lane
// receives 16 consecutive tokens of one channel), the B operand is W read
// straight from global memory (16 bytes of one W row per lane), fp32
// accumulation.  fp32: plain fp32 FMAs in input-channel order.
#pragma once

#include "common.h"

namespace rglru {

template <typename T> struct XTile;
template <> struct XTile<bf16> { static constexpr int STRIDE = 256 + 8; };   // 528-byte rows
template <> struct XTile<float> { static constexpr int STRIDE = 256 + 4; };  // 1040-byte rows

__device__ __forceinline__ void gate_tile(const bf16 *Xs, const bf16 *Wa_h, const bf16 *Wx_h,
                                          int wave, int lane, float za[16], float zx[16])
{
    constexpr int S = XTile<bf16>::STRIDE;
    const int r = lane & 31, kg = lane >> 5;
    const bf16 *xrow = Xs + tile_row_token(r) * S + 8 * kg;
    const bf16 *wa = Wa_h + (size_t)(32 * wave + r) * 256 + 8 * kg;
    const bf16 *wx = Wx_h + (size_t)(32 * wave + r) * 256 + 8 * kg;
    f32x16 A = {}, X = {};
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        const bf16x8 av = *(const bf16x8 *)(xrow + 16 * s);
        const bf16x8 ba = *(const bf16x8 *)(wa + 16 * s);
        const bf16x8 bx = *(const bf16x8 *)(wx + 16 * s);
        A = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, ba, A, 0, 0, 0);
        X = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bx, X, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        za[k] = A[k];
        zx[k] = X[k];
    }
}

__device__ __forceinline__ void gate_tile(const float *Xs, const float *Wa_h, const float *Wx_h,
                                          int wave, int lane, float za[16], float zx[16])
{
    constexpr int S = XTile<float>::STRIDE;
    const int n = lane & 31, half = lane >> 5;
    const float *wa = Wa_h + (size_t)(32 * wave + n) * 256;
    const float *wx = Wx_h + (size_t)(32 * wave + n) * 256;
    const float *xs = Xs + (16 * half) * S;
#pragma unroll
    for (int k = 0; k < 16; ++k) za[k] = zx[k] = 0.0f;
    for (int j = 0; j < 256; ++j) {
        const float wav = wa[j], wxv = wx[j];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const float xv = xs[k * S + j];
            za[k] = fmaf(wav, xv, za[k]);
            zx[k] = fmaf(wxv, xv, zx[k]);
        }
    }
}

}  // namespace rglru
