// internal.h -- launchers behind the C ABI (host side, C++ linkage).
// Arguments have been validated by api.hip before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/rglru.h"

namespace rglru {

// Largest number of 256-channel groups a chunked scan serves: its workspace
// keeps one claim counter per group in a region of fixed size.
constexpr int MAX_CLAIM_GROUPS = 4096;
// Byte offset of the look-back timeout word in the header that starts every
// scan workspace (the forward's, the backward's, the block's and the layer's).
constexpr size_t WS_ERROR_OFFSET = 12;

size_t fwd_workspace_bytes(int64_t B, int64_t T, int64_t D);
// esz: bytes per activation element (2 for bf16 I/O, 4 for fp32)
size_t bwd_workspace_bytes(int64_t B, int64_t T, int64_t D, int64_t H, size_t esz);

void launch_conv1d(const rglru_desc &d, const float *cw, const float *cb, const void *u,
                   const void *hist_in, void *x, void *hist_out, hipStream_t s);

void launch_gates(const rglru_desc &d, const rglru_weights &w, const void *x, void *r, void *i,
                  hipStream_t s);

// mode: 0 = conv + gates + scan, 1 = gates + scan, 2 = scan only
void launch_scan_fwd(const rglru_desc &d, const rglru_weights &w, int mode, const void *in,
                     const void *r, const void *i, const void *hist_in, const float *h0, void *y,
                     float *h_last, void *hist_out, void *ws, hipStream_t s);

// mode A, bf16 I/O, K = 256, B T D 2 < 2^31: the one-wave-per-SIMD fused
// forward (fused.hip), taken only with RGLRU_FWD_FUSED=1 in the environment;
// fused_fwd_applies says whether a call takes it.
bool fused_fwd_applies(const rglru_desc &d);
void launch_fused_fwd(const rglru_desc &d, const rglru_weights &w, const void *u, const void *hist_in,
                      const float *h0, void *y, float *h_last, void *hist_out, void *ws, hipStream_t s);

// mode A forward that stores no outputs but the state before every 32-token
// chunk ([B][NC][D] fp32) and the gate values r, i of every token (layout of
// GateStore in common.h) -- the first pass of the backward
void launch_fwd_states(const rglru_desc &d, const rglru_weights &w, const void *u,
                       const void *hist_in, const float *h0, float *hstart_out, void *ri_out,
                       void *ws, hipStream_t s);

// mode A with the recurrent block's merge: z = y * GeLU(g) is stored instead
// of y (g: branch-2 pre-activation, [B][T][D] io)
void launch_scan_fwd_merge(const rglru_desc &d, const rglru_weights &w, const void *u, const void *g,
                           const void *hist_in, const float *h0, void *z, float *h_last, void *hist_out,
                           void *ws, hipStream_t s);

// Y[M][N] = X[M][K] W[N][K]^T (+ R when not null), row-major, fp32
// accumulation, io types (gemm.hip); returns an rglru_status
int launch_gemm(int io, int64_t M, int64_t N, int64_t K, const void *X, const void *W, const void *R, void *Y,
                hipStream_t s);
bool gemm_uses_mfma(int io, int64_t M, int64_t N, int64_t K);

// Recurrent block: byte offsets inside its workspace (scan carries at 0,
// then the two projections b1 and b2) and the whole size
struct BlockLayout {
    size_t scan, b1, b2, bytes;
};
BlockLayout block_layout(int64_t B, int64_t T, int64_t D, size_t esz);

// returns an rglru_status
int launch_block_fwd(const rglru_desc &d, int64_t d_model, const rglru_weights &w, const rglru_block &blk,
                     const void *x, const void *hist_in, const float *h0, void *out, float *h_last,
                     void *hist_out, void *ws, hipStream_t s);

// Residual layer (block.hip): byte offsets of its workspace -- the block's
// workspace, the normed input xn, the residual stream x~, the MLP's gate and
// up activations -- and the whole size
struct LayerLayout {
    size_t block, xn, xt, g, u, bytes;
};
LayerLayout layer_layout(int64_t B, int64_t T, int64_t D, int64_t d_model, int64_t d_ff, size_t esz);
int launch_layer_fwd(const rglru_desc &d, int64_t d_model, const rglru_weights &w, const rglru_block &blk,
                     const rglru_layer &lw, const void *x, const void *hist_in, const float *h0, void *y,
                     float *h_last, void *hist_out, void *ws, hipStream_t s);

// Attention residual layer (block.hip): workspace offsets of xn, q, k, v, o,
// x~ and the MLP activations
struct AttnLayerLayout {
    size_t xn, q, k, v, o, xt, g, u, bytes;
};
AttnLayerLayout attn_layer_layout(const rglru_attn_desc &d, int64_t d_model, int64_t d_ff);
int launch_attn_layer_fwd(const rglru_attn_desc &d, int64_t d_model, int rot, float rope_base, int64_t pos0,
                          const rglru_attn_proj &ap, const rglru_layer &lw, const void *x, void *y, void *kc,
                          void *vc, void *ws, hipStream_t s);

// local sliding-window MQA (attn.hip)
bool attn_fast_prefill(const rglru_attn_desc &d);
bool attn_fast_step(const rglru_attn_desc &d);
size_t attn_workspace_bytes(const rglru_attn_desc &d);
void launch_attn_fwd(const rglru_attn_desc &d, const void *q, const void *k, const void *v, void *o, void *kc,
                     void *vc, hipStream_t s);
void launch_attn_step(const rglru_attn_desc &d, const void *q_t, const void *k_t, const void *v_t, void *kc,
                      void *vc, const int32_t *pos, void *o_t, void *ws, hipStream_t s);

void launch_step(const rglru_desc &d, const rglru_weights &w, const void *u_t, const void *hist_in,
                 void *hist_out, float *h, void *y_t, hipStream_t s);

void launch_scan_bwd(const rglru_desc &d, const rglru_weights &w, const void *u, const void *hist_in,
                     const float *h0, const void *dy, const float *dh_last, void *du, float *dcw,
                     float *dcb, float *dWa, float *dba, float *dWx, float *dbx, float *dLambda,
                     float *dh0, void *ws, hipStream_t s);

}  // namespace rglru
