// block.hip -- the recurrent block around the RG-LRU (page "Griffin Guide:
// RecurrentGemma, RG-LRU & Hybrid Attention", section "The Recurrent Block
// Architecture", parts "Temporal Filtering via Separable 1D Convolutions" and
// "Non-Linear Multiplicative Gating with GeLU", and the RecurrentBlock class of
// its PyTorch listing): two bias-free input projections to the RG-LRU width D,
// conv + RG-LRU on branch 1, the exact (erf) GeLU of branch 2 multiplied in,
// and a bias-free output projection back to d_model.  The residual add belongs
// to the decoder layer, outside the block.
//
//   b1 = x proj_in_1^T        [B*T][D]    rocBLAS GEMM
//   b2 = x proj_in_2^T        [B*T][D]    rocBLAS GEMM
//   z  = RG-LRU(conv(b1)) * GeLU(b2)      the fused forward, mode 4 (the merge
//                                         happens where y would be stored; z
//                                         overwrites b2 in place: every element
//                                         of b2 is read by the lane that writes
//                                         z there, before it writes)
//   out = z proj_out^T        [B*T][d_model]  rocBLAS GEMM
//
// The projections are plain dense GEMMs, so they go to the library (bf16
// inputs, fp32 accumulation, bf16 output for bf16 I/O; fp32 throughout for
// fp32 I/O).  Workspace: the scan's carries first (its header must start out
// zero), then b1 and b2.
#include <rocblas/rocblas.h>

#include <mutex>

#include "common.h"
#include "internal.h"

namespace rglru {

namespace {

// One rocBLAS handle per device, made on first use with that device current.
// Calls that share a device share its handle; the stream is set and the GEMM
// enqueued under the lock, so concurrent callers never see each other's stream.
std::mutex blas_mu;
rocblas_handle blas_handles[64];

rocblas_handle blas_handle_locked(int dev)
{
    if (dev < 0 || dev >= 64) return nullptr;
    if (!blas_handles[dev] && rocblas_create_handle(&blas_handles[dev]) != rocblas_status_success)
        blas_handles[dev] = nullptr;
    return blas_handles[dev];
}

// Y[M][N] = X[M][K] W[N][K]^T, all row-major.  Column-major, that is
// Y^T (N x M, ld N) = W^T (op T of the K x N array W, ld K) * X^T (K x M, ld K).
bool gemm_xwt(rocblas_handle h, int io, int64_t M, int64_t N, int64_t K, const void *X, const void *W,
              void *Y)
{
    const rocblas_datatype t = io == RGLRU_BF16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
    const float alpha = 1.0f, beta = 0.0f;
    return rocblas_gemm_ex_64(h, rocblas_operation_transpose, rocblas_operation_none, N, M, K, &alpha, W,
                              t, K, X, t, K, &beta, Y, t, N, Y, t, N, rocblas_datatype_f32_r,
                              rocblas_gemm_algo_standard, 0, 0) == rocblas_status_success;
}

size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

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

int launch_block_fwd(const rglru_desc &d, int64_t d_model, const rglru_weights &w, const rglru_block &blk,
                     const void *x, const void *hist_in, const float *h0, void *out, float *h_last,
                     void *hist_out, void *ws, hipStream_t s)
{
    const size_t esz = d.io == RGLRU_BF16 ? 2 : 4;
    const BlockLayout L = block_layout(d.B, d.T, d.D, esz);
    char *base = (char *)ws;
    void *b1 = base + L.b1, *b2 = base + L.b2;
    const int64_t M = d.B * d.T;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return RGLRU_ERR_LAUNCH;
    {
        std::lock_guard<std::mutex> lock(blas_mu);
        rocblas_handle h = blas_handle_locked(dev);
        if (!h || rocblas_set_stream(h, s) != rocblas_status_success) return RGLRU_ERR_BLAS;
        if (!gemm_xwt(h, d.io, M, d.D, d_model, x, blk.proj_in_1, b1)) return RGLRU_ERR_BLAS;
        if (!gemm_xwt(h, d.io, M, d.D, d_model, x, blk.proj_in_2, b2)) return RGLRU_ERR_BLAS;
    }
    launch_scan_fwd_merge(d, w, b1, b2, hist_in, h0, b2, h_last, hist_out, base + L.scan, s);
    if (hipGetLastError() != hipSuccess) return RGLRU_ERR_LAUNCH;
    {
        std::lock_guard<std::mutex> lock(blas_mu);
        rocblas_handle h = blas_handle_locked(dev);
        if (!h || rocblas_set_stream(h, s) != rocblas_status_success) return RGLRU_ERR_BLAS;
        if (!gemm_xwt(h, d.io, M, d_model, d.D, b2, blk.proj_out, out)) return RGLRU_ERR_BLAS;
    }
    return RGLRU_OK;
}

}  // namespace rglru
