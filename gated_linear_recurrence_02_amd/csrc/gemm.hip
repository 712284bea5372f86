// gemm.hip -- the dense projections around the RG-LRU (the recurrent block's
// two input projections and its output projection, page "Griffin Guide:
// RecurrentGemma, RG-LRU & Hybrid Attention", section "The Recurrent Block
// Architecture"; the residual layers' gated MLP and the attention layer's
// q/k/v/o projections, page "Griffin", section "Residual Block View"):
//     Y[M][N] = X[M][K] W[N][K]^T (+ R[M][N]),
// all row-major with K contiguous in both operands, fp32 accumulation, Y (and
// R) in the I/O type.
//
// bf16 with K % 64 == 0 (and M K, N K below 2^31): 256 x 256 output tiles
// (256 x 128 for grids too small to fill the CUs), one workgroup of 8 waves
// each (two per SIMD), wave (wm, wn) owning the 64 x 128 (64 x 64) sub-tile at
// (64 wm, 128 wn) ((64 wm, 64 wn)) as 2 x 4 (2 x 2) v_mfma_f32_32x32x16_bf16
// accumulators.  K advances 64 at a time through two LDS buffers: while the
// matrix cores work
// on one, the next 256 x 64 slices of X and W stream into the other straight
// from global memory (buffer loads into LDS, 1 KB per wave instruction = 8
// rows of 128 bytes; a lane's row offset is fixed, the K position is a
// scalar).  A row's eight 16-byte chunks sit XOR-swizzled by row % 8, so that
// the 32 rows one operand read touches spread over the banks; each wave
// reads the operands of the next 16-wide K step while its current products
// run.  Rows past M or N read row M-1 / N-1 and are not stored.  The tile
// order keeps consecutive tiles of one X row band on one XCD, so that its L2
// serves the band's reuse.
//
// Every other case (fp32, or K not a multiple of 64): 64 x 64 tiles through
// LDS with fp32 FMAs, any shape.
#include <stdlib.h>

#include <mutex>

#include "common.h"
#include "internal.h"

namespace rglru {

namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int TBM = 256, TBK = 64;   // MFMA tile rows and K slice; BN (256 or 128) columns
constexpr int GT = 512;              // threads of the MFMA kernel
template <int BN> constexpr int tbuf() { return (TBM + BN) * TBK; }   // bf16 elements of one LDS buffer

struct GemmArgs {
    int M, N, K;
    const void *X, *W, *R;
    void *Y;
};

// The body is a device function template and the two tile widths two plain
// kernels: a __global__ template would be instantiated for the host as well,
// where the buffer-resource type does not exist.
template <int BN>
__device__ __forceinline__ void gemm_nt_mfma_body(const GemmArgs &a)
{
    constexpr int TBN = BN, TBUF = tbuf<BN>();
    constexpr int NJ = BN / 64;   // 32-column accumulator tiles per wave
    extern __shared__ __attribute__((aligned(16))) char smem[];
    bf16 *lds = (bf16 *)smem;
    const int M = a.M, N = a.N, K = a.K;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    // tile order: consecutive numbers share an XCD; the N tiles of one row
    // band are consecutive
    const int ntn = (N + TBN - 1) / TBN;
    const int nwg = gridDim.x, xcd = blockIdx.x % 8, loc = blockIdx.x / 8;
    const int lin = xcd * (nwg / 8) + (xcd < nwg % 8 ? xcd : nwg % 8) + loc;
    const int m0 = (lin / ntn) * TBM, n0 = (lin % ntn) * TBN;

    // staging: 32 wave instructions per operand and K slice, wave w the
    // instructions q = w + 8 i (i < 4); instruction q fills rows 8q .. 8q+7,
    // lane l the 16-byte position l % 8 of row 8q + l / 8, which holds the
    // row's chunk (l % 8) ^ (row % 8).  Byte offsets are 32-bit (M K and N K
    // below 2^31 elements); the slice's K position is the scalar offset.
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.X), 0, (int)((unsigned)M * (unsigned)K * 2u), 0x00020000);
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.W), 0, (int)((unsigned)N * (unsigned)K * 2u), 0x00020000);
    uint32_t offa[4], offb[BN / 64];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = 8 * i + wave, r = 8 * q + (lane >> 3), c = (lane & 7) ^ (r & 7);
        const int ra = m0 + r < M ? m0 + r : M - 1, rb = n0 + r < N ? n0 + r : N - 1;
        offa[i] = ((uint32_t)ra * (uint32_t)K + 8u * c) * 2u;
        if (i < BN / 64) offb[i] = ((uint32_t)rb * (uint32_t)K + 8u * c) * 2u;
    }
    auto stage = [&](int kt, int b) {
        bf16 *la = lds + b * TBUF, *lb = la + TBM * TBK;
        const uint32_t so = (uint32_t)kt * TBK * 2u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = 8 * i + wave;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(la + q * 512), 16, offa[i], so, 0, 0);
            if (i < BN / 64)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(lb + q * 512), 16, offb[i], so, 0, 0);
        }
    };

    const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, kh = lane >> 5;
    f32x16 acc[2][NJ];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};
    // operands of K step ks of the current slice: A rows 64 wm + 32 i + l % 32,
    // B rows (BN / 2) wn + 32 j + l % 32, the lane's 16-byte chunk 2 ks + l / 32
    bf16x8 fa[2][2], fb[2][NJ];
    auto frags = [&](const bf16 *la, const bf16 *lb, int ks, int set) {
        const int c = 2 * ks + kh;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = 64 * wm + 32 * i + l32;
            fa[set][i] = *(const bf16x8 *)(la + r * TBK + 8 * (c ^ (r & 7)));
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int r = (BN / 2) * wn + 32 * j + l32;
            fb[set][j] = *(const bf16x8 *)(lb + r * TBK + 8 * (c ^ (r & 7)));
        }
    };

    const int nk = K / TBK;
    stage(0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        // slice kt has landed (each wave waits for its own requests, the
        // barrier for everyone's), and every wave is done with the other buffer
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (kt + 1 < nk) stage(kt + 1, (kt + 1) & 1);
        const bf16 *la = lds + (kt & 1) * TBUF, *lb = la + TBM * TBK;
        frags(la, lb, 0, 0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4) frags(la, lb, ks + 1, (ks + 1) & 1);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks & 1][i], fb[ks & 1][j], acc[i][j], 0,
                                                                        0, 0);
            // the next step's 2 + NJ operand reads between this step's 2 NJ
            // products (6 between 8, or 4 between 4)
            if (ks + 1 < 4) {
#pragma unroll
                for (int t = 0; t < 2 + NJ; ++t) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
                }
                if constexpr (NJ == 4) __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // 8 - 6
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // accumulator e of tile (i, j): row 32 i + 8 (e / 4) + 4 (l / 32) + e % 4,
    // column 32 j + l % 32 of the wave's sub-tile
    const bf16 *R = (const bf16 *)a.R;
    bf16 *Y = (bf16 *)a.Y;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int col = n0 + (BN / 2) * wn + 32 * j + l32;
            if (col >= N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + 64 * wm + 32 * i + 8 * (e >> 2) + 4 * kh + (e & 3);
                if (row < M) {
                    const size_t o = (size_t)row * N + col;
                    float v = acc[i][j][e];
                    if (R) v += (float)R[o];
                    Y[o] = (bf16)v;
                }
            }
        }
}

__global__ __launch_bounds__(GT) void gemm_nt_mfma(GemmArgs a) { gemm_nt_mfma_body<256>(a); }
__global__ __launch_bounds__(GT) void gemm_nt_mfma_n128(GemmArgs a) { gemm_nt_mfma_body<128>(a); }

// any shape, either I/O type: 64 x 64 tiles, thread (tx, ty) the 4 x 4
// outputs at rows 4 ty.., columns 4 tx.., K in steps of 16 through LDS
template <typename T>
__global__ __launch_bounds__(256) void gemm_nt_generic(GemmArgs a)
{
    __shared__ float As[16][64 + 4], Bs[16][64 + 4];
    const T *X = (const T *)a.X, *W = (const T *)a.W, *R = (const T *)a.R;
    T *Y = (T *)a.Y;
    const int M = a.M, N = a.N, K = a.K;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int ntn = (N + 63) / 64;   // one-dimensional grid: M may exceed 65535 tiles
    const long m0 = (long)(blockIdx.x / ntn) * 64;
    const int n0 = (int)(blockIdx.x % ntn) * 64;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int idx = 256 * q + tid, r = idx >> 4, kk = idx & 15;
            const int k = k0 + kk;
            As[kk][r] = (m0 + r < M && k < K) ? (float)X[(size_t)(m0 + r) * K + k] : 0.0f;
            Bs[kk][r] = (n0 + r < N && k < K) ? (float)W[(size_t)(n0 + r) * K + k] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            float av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                av[i] = As[kk][4 * ty + i];
                bv[i] = Bs[kk][4 * tx + i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const long row = m0 + 4 * ty + i;
            const int col = n0 + 4 * tx + j;
            if (row < M && col < N) {
                const size_t o = (size_t)row * N + col;
                float v = acc[i][j];
                if (R) v += (float)R[o];
                Y[o] = from_f32<T>(v);
            }
        }
}

}  // namespace

bool gemm_uses_mfma(int io, int64_t M, int64_t N, int64_t K)
{
    // 32-bit buffer offsets: M K and N K elements below 2^31
    return io == RGLRU_BF16 && K > 0 && K % TBK == 0 && M * K < ((int64_t)1 << 31) && N * K < ((int64_t)1 << 31);
}

int launch_gemm(int io, int64_t M, int64_t N, int64_t K, const void *X, const void *W, const void *R, void *Y,
                hipStream_t s)
{
    if (M <= 0 || N <= 0 || K <= 0 || M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return RGLRU_ERR_SHAPE;
    GemmArgs a;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.X = X;
    a.W = W;
    a.R = R;
    a.Y = Y;
    if (gemm_uses_mfma(io, M, N, K)) {
        int ncu = 256;
        {
            // 128 / 96 KB of LDS, above the default limit: raised once per
            // device (a failure surfaces at the launch)
            static std::mutex mu;
            static int cus[64];
            int dev = 0;
            (void)hipGetDevice(&dev);
            std::lock_guard<std::mutex> lock(mu);
            if (dev >= 0 && dev < 64) {
                if (!cus[dev]) {
                    (void)hipFuncSetAttribute((const void *)&gemm_nt_mfma,
                                              hipFuncAttributeMaxDynamicSharedMemorySize, 2 * tbuf<256>() * 2);
                    (void)hipFuncSetAttribute((const void *)&gemm_nt_mfma_n128,
                                              hipFuncAttributeMaxDynamicSharedMemorySize, 2 * tbuf<128>() * 2);
                    int n = 0;
                    (void)hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
                    cus[dev] = n > 0 ? n : 256;
                }
                ncu = cus[dev];
            }
        }
        // one workgroup per CU at a time: the launch takes ceil(tiles / CUs)
        // rounds.  A round of half-width tiles took 0.68 of a round of wide
        // ones (more operand reads per product: 16384 x 2560 x 2560 in 5
        // narrow rounds against 3 wide ones was 9% slower), so narrow tiles
        // serve the grids they fit in fewer rounds' worth of time, in practice
        // those with fewer wide tiles than CUs (the 256-wide projections of
        // the attention layer: 64 wide tiles, 128 narrow ones).
        // RGLRU_GEMM_TILE_N=128 or 256 forces a width (tests compare them).
        const long tm = (M + TBM - 1) / TBM;
        const long t256 = tm * ((N + 255) / 256), t128 = tm * ((N + 127) / 128);
        const long r256 = (t256 + ncu - 1) / ncu, r128 = (t128 + ncu - 1) / ncu;
        bool narrow = r128 * 7 < r256 * 10;
        if (const char *f = getenv("RGLRU_GEMM_TILE_N")) {
            if (atoi(f) == 128) narrow = true;
            else if (atoi(f) == 256) narrow = false;
        }
        if (narrow)
            gemm_nt_mfma_n128<<<dim3((unsigned)t128), dim3(GT), 2 * tbuf<128>() * 2, s>>>(a);
        else
            gemm_nt_mfma<<<dim3((unsigned)t256), dim3(GT), 2 * tbuf<256>() * 2, s>>>(a);
    } else {
        const dim3 grid((unsigned)(((N + 63) / 64) * ((M + 63) / 64)));
        if (io == RGLRU_BF16) gemm_nt_generic<bf16><<<grid, dim3(256), 0, s>>>(a);
        else gemm_nt_generic<float><<<grid, dim3(256), 0, s>>>(a);
    }
    return hipGetLastError() == hipSuccess ? RGLRU_OK : RGLRU_ERR_LAUNCH;
}

}  // namespace rglru
