/*
 * rglru.h -- C ABI of the MI355X (gfx950) RG-LRU hot path library
 * (librglru.so): the causal depthwise Conv1D of width 4 followed by the
 * Real-Gated Linear Recurrent Unit of Griffin / Hawk / RecurrentGemma.
 *
 * The operation (page "Griffin Guide: RecurrentGemma, RG-LRU & Hybrid
 * Attention", section "Formulation of the RG-LRU Gating Mechanism"):
 *     r_t = sigma(W_a x_t + b_a)                       recurrence gate
 *     i_t = sigma(W_x x_t + b_x)                       input gate
 *     a_t = a^(c r_t),  a = sigma(Lambda),  c = 8      decay, computed as
 *           log a_t = -c r_t softplus(-Lambda)          (log-space form)
 *     h_t = a_t h_{t-1} + sqrt(1 - a_t^2) (i_t x_t)     state update
 *     y_t = h_t                                        output
 * where x is the output of a causal depthwise convolution of width 4 over
 * the branch-1 activations u (same page, "Temporal Filtering via Separable
 * 1D Convolutions"), and W_a, W_x are block-diagonal with square blocks of
 * width K = D / H (same page, "Block-Diagonal Sharding for
 * Zero-Communication Tensor Parallelism").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every tensor pointer is DEVICE memory owned by the caller.  The
 *   library does not synchronise the host (rglru_workspace_status, a report
 *   the caller asks for, aside): a return of RGLRU_OK means the work was
 *   enqueued on `stream`.  It allocates nothing (rglru_scan_fwd_noalloc's
 *   fixed scratch, loaded with the library, aside) and keeps no state
 *   between calls beyond what the caller's buffers hold.
 * Layouts.  Row-major, channel fastest:
 *     activations u, x, r, i, y, dy, du   [B][T][D]   (dtype desc->io)
 *     conv history hist                   [B][3][D]   (dtype desc->io)
 *         hist[b][j] is the pre-conv input at position t-3+j (oldest first)
 *     state h0, h_last, h, dh_last, dh0   [B][D]      (always fp32)
 *     conv weight conv_w                  [D][4] fp32; tap k multiplies
 *                                          u[t-3+k], tap 3 is the current token
 *     conv bias conv_b, b_a, b_x, Lambda  [D] fp32
 *     gate weights W_a, W_x               [H][K][K] (dtype desc->io);
 *         W[h][o][j] multiplies input channel hK+j into output channel hK+o
 *     gate-weight gradients dW_a, dW_x    [H][K][K] fp32
 * Dtypes.  desc->io is RGLRU_F32 or RGLRU_BF16 (activations, history and gate
 *   weights).  State, biases, Lambda, conv weights and every accumulation are
 *   fp32.
 * Shapes.  B, T, D, H >= 1, D % H == 0, D <= 1048576.  Every call that evaluates the gates
 *   (rglru_gates, rglru_scan_fwd without r/i, rglru_step, rglru_scan_bwd)
 *   needs K = D / H = 256, the block width of the MFMA gate kernels.
 *   rglru_conv1d and the scan-only mode of rglru_scan_fwd accept any D.
 * Alignment.  Every pointer must be 16-byte aligned.
 * Validation.  All checks run on the host before anything is enqueued; on
 *   error nothing is enqueued and no output is touched.  A launch error is
 *   reported as RGLRU_ERR_LAUNCH after the fact (hipGetLastError).
 * Work distribution.  The forward scans are persistent kernels that claim
 *   their work units from counters in the workspace at run time; they need
 *   no co-residency guarantee and may share the device with other work.  A
 *   chunk-carry wait that never sees its data (which only a corrupted or
 *   concurrently reused workspace can cause) gives up after a bounded spin,
 *   sets a timeout word in the workspace header and yields NaN; the call has
 *   returned RGLRU_OK by then (it only enqueues), so rglru_workspace_status
 *   reports it afterwards.  The backward's own kernels never wait on one
 *   another's workgroups.
 * Aliasing.  Outputs must not overlap inputs, except h of rglru_step,
 *   which is read and rewritten in place by design.
 * Determinism.  Every call is bitwise repeatable: identical inputs on the
 *   same device give identical outputs, whatever the timing of the
 *   workgroups.  The chunked scans carry state between 32-token chunks
 *   through published words; a chunk folds the aggregates of the chunks
 *   after the newest published end state onto it in chunk order, which
 *   reproduces the serial recurrence over chunk aggregates exactly, however
 *   far back it had to look.  The backward's reverse scan and reductions run
 *   in a fixed order with no floating-point atomics.
 * Numerics.  NaN and Inf in the inputs propagate; they are not trapped.
 */
#ifndef RGLRU_H
#define RGLRU_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { RGLRU_F32 = 0, RGLRU_BF16 = 1 } rglru_dtype;

typedef enum {
    RGLRU_OK = 0,
    RGLRU_ERR_NULL = -1,       /* a required pointer is NULL                    */
    RGLRU_ERR_SHAPE = -2,      /* bad B, T, D, H, K != 256 where needed, T != 1 */
    RGLRU_ERR_DTYPE = -3,      /* desc->io is not a known rglru_dtype           */
    RGLRU_ERR_ALIGN = -4,      /* a pointer is not 16-byte aligned              */
    RGLRU_ERR_WORKSPACE = -5,  /* workspace NULL or smaller than required       */
    RGLRU_ERR_LAUNCH = -6,     /* the HIP runtime reported a launch error       */
    RGLRU_ERR_ARG = -7,        /* inconsistent arguments (mode, aliasing)       */
    RGLRU_ERR_BLAS = -8,       /* reserved (no call returns it)                 */
    RGLRU_ERR_TIMEOUT = -9,    /* rglru_workspace_status: a chunk-carry wait of
                                  an earlier call gave up (outputs hold NaN)    */
    RGLRU_ERR_SCRATCH = -10    /* rglru_scan_fwd_noalloc: the call needs more
                                  than RGLRU_NOALLOC_SCRATCH_BYTES              */
} rglru_status;

/* Problem description.  c is the decay-exponent scale (8 on the pages). */
typedef struct {
    int64_t B, T, D, H;
    int32_t io;        /* rglru_dtype */
    float c;
} rglru_desc;

/* Parameters (device pointers).  Which ones a call reads is stated at the call. */
typedef struct {
    const float *conv_w;   /* [D][4]  */
    const float *conv_b;   /* [D], NULL means zero bias */
    const void *W_a;       /* [H][K][K], dtype io */
    const float *b_a;      /* [D], NULL means zero */
    const void *W_x;       /* [H][K][K], dtype io */
    const float *b_x;      /* [D], NULL means zero */
    const float *Lambda;   /* [D] */
} rglru_weights;

enum { RGLRU_OP_SCAN_FWD = 0, RGLRU_OP_SCAN_BWD = 1 };

/* Workspace bytes that rglru_scan_fwd (op RGLRU_OP_SCAN_FWD) or rglru_scan_bwd
 * (op RGLRU_OP_SCAN_BWD) needs for `desc`.  The workspace carries the chunk
 * carries of the chunked scan and a small header of counters; it must be
 * ZERO-FILLED before its first use and is left ready for the next call
 * (every call restores the header).  A forward workspace holds only the
 * header, claim counters in a region of fixed size and tagged carry words
 * (stale words carry an earlier call's tag), so one zero-filled buffer of
 * the largest size needed serves forward calls of any shape one after
 * another.  The backward's workspace also keeps plain data (states, gate
 * values, staging) where a later call of another layout could look for
 * carry words, so reuse it without zero-filling it again only for calls with
 * the same desc (B, T, D, H, io).  One workspace must not be used by two
 * calls that can run at the same time.  The chunked scans serve at most 4096
 * groups of 256 channels (D <= 1048576).  Errors: RGLRU_ERR_NULL, _SHAPE,
 * _DTYPE, _ARG (unknown op). */
int rglru_workspace_size(const rglru_desc *desc, int op, size_t *bytes);

/* Timeout report of the scan workspace `ws` (any of the forward's, the
 * backward's, the recurrent block's or the residual layer's, all of which
 * start with the same header): WAITS for the work enqueued on `stream`, reads
 * the header's timeout word and clears it.  Returns RGLRU_OK if no
 * chunk-carry wait of a call that used `ws` has given up since the last
 * report, RGLRU_ERR_TIMEOUT if one has (that call's outputs hold NaN),
 * RGLRU_ERR_NULL / _ALIGN / _WORKSPACE (ws_bytes < 256) for bad arguments and
 * RGLRU_ERR_LAUNCH if the runtime reports an error.  This is the one call of
 * the library that synchronises the host; it allocates nothing. */
int rglru_workspace_status(const void *ws, size_t ws_bytes, hipStream_t stream);

/* a1 -- causal depthwise Conv1D of width 4 with bias (section "Temporal
 * Filtering via Separable 1D Convolutions"; the listing's Conv1d with
 * padding 3 and one group per channel, first T outputs kept):
 *     x[b][t][d] = conv_b[d] + sum_{k=0..3} conv_w[d][k] * u[b][t-3+k][d]
 * Positions t-3+k < 0 read hist_in[b][3+(t-3+k)][d] (zeros if hist_in is
 * NULL).  hist_out (nullable) receives the pre-conv inputs at positions
 * T-3, T-2, T-1 bit for bit (for T < 3 partly from hist_in).  Arithmetic is
 * fp32; x is rounded to io.  Needs conv_w, u, x.  Any D >= 1. */
int rglru_conv1d(const rglru_desc *desc, const float *conv_w, const float *conv_b,
                 const void *u, const void *hist_in, void *x, void *hist_out,
                 hipStream_t stream);

/* a2 -- block-diagonal gates (recurrence-gate and input-gate equations):
 *     r[b][t][hK+o] = sigma(b_a[hK+o] + sum_j W_a[h][o][j] x[b][t][hK+j])
 *     i[b][t][hK+o] = sigma(b_x[hK+o] + sum_j W_x[h][o][j] x[b][t][hK+j])
 * bf16: matrix-core products of bf16 inputs with fp32 accumulation;
 * fp32: fp32 products and sums.  Reads w->W_a, W_x, b_a, b_x.  K = 256. */
int rglru_gates(const rglru_desc *desc, const rglru_weights *w, const void *x,
                void *r, void *i, hipStream_t stream);

/* a3..a5 -- the forward scan (state-update and output equations), i.e. the
 * listing's RGLRU.forward(x, prev_state) -> (y, last_state), optionally with
 * the conv fused in front.  The mode follows from the pointers:
 *   mode A  w->conv_w != NULL, r == i == NULL : `in` is pre-conv u;
 *           conv + gates + decay + scan in one kernel (K = 256).
 *   mode B  w->conv_w == NULL, r == i == NULL : `in` is x; gates + scan (K = 256).
 *   mode C  r and i given (w->conv_w must be NULL) : `in` is x; the decay and
 *           scan only (any D); only w->Lambda is read.
 * h0 (nullable, zeros) is the state before token 0; h_last (nullable)
 * receives h_{T-1}; hist_in / hist_out (nullable, mode A only) carry the conv
 * history as in rglru_conv1d.  y is rounded to io; the state stays fp32.
 * T is split into chunks whose carries are combined through the workspace
 * (see rglru_workspace_size).  Extra errors: RGLRU_ERR_ARG for r without i,
 * hist with modes B/C, or conv_w with r/i. */
int rglru_scan_fwd(const rglru_desc *desc, const rglru_weights *w, const void *in,
                   const void *r, const void *i, const void *hist_in, const float *h0,
                   void *y, float *h_last, void *hist_out, void *ws, size_t ws_bytes,
                   hipStream_t stream);

/* rglru_scan_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same modes, arguments, checks,
 * results and determinism as rglru_scan_fwd, with the chunk carries kept in
 * a scratch array of RGLRU_NOALLOC_SCRATCH_BYTES (64 MiB) that the library
 * holds on each device it runs on until the process ends.  The call
 * allocates nothing; its first call on a device resolves that device's copy
 * of the array and clears it with a kernel on `stream`.  Every call on one
 * device shares the array: calls that can run at the same time on one
 * device (other streams, other host threads) RACE and must be serialised by
 * the caller.  The scratch has no timeout report; a chunk-carry wait that
 * gives up (possible only when calls overlap) leaves NaN in the outputs.
 * Extra error: RGLRU_ERR_SCRATCH when rglru_workspace_size(desc,
 * RGLRU_OP_SCAN_FWD) -- 16640 + 24 B ceil(T/32) D bytes -- exceeds
 * RGLRU_NOALLOC_SCRATCH_BYTES, i.e. B ceil(T/32) D > 2795509: the 32k-token
 * prefill at D = 2560 (2621440) fits, B = 4, T = 8192, D = 4096 does not. */
#define RGLRU_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int rglru_scan_fwd_noalloc(const rglru_desc *desc, const rglru_weights *w, const void *in,
                           const void *r, const void *i, const void *hist_in, const float *h0,
                           void *y, float *h_last, void *hist_out, hipStream_t stream);

/* a6 -- one decode step for B independent streams (the listing's RGLRU.step,
 * with the conv history carried in front): desc->T must be 1.
 *     x = conv_b + conv_w[0] hist_in[0] + conv_w[1] hist_in[1]
 *                + conv_w[2] hist_in[2] + conv_w[3] u_t
 *     h <- a h + sqrt(1 - a^2) i x,   y_t = h,
 *     hist_out <- (hist_in[1], hist_in[2], u_t)
 * hist_in / hist_out [B][3][D] (io; hist_in NULL means zeros, hist_out NULL
 * drops the new history) are separate buffers that must not overlap -- the
 * caller alternates two of them between steps, as with rglru_scan_fwd's --
 * and h [B][D] (fp32) is read and rewritten in place.  Reads every field of
 * w (conv_b, b_a, b_x nullable).  K = 256.  512 consecutive calls equal one
 * rglru_scan_fwd (mode A) over the same 512 tokens, the history copies bit
 * for bit.  Extra error: RGLRU_ERR_ARG if hist_out overlaps hist_in or any
 * other argument. */
int rglru_step(const rglru_desc *desc, const rglru_weights *w, const void *u_t,
               const void *hist_in, void *hist_out, float *h, void *y_t, hipStream_t stream);

/* a7 -- backward of mode A: gradients of L = <dy, y> + <dh_last, h_last>
 * with respect to u, conv_w, conv_b, W_a, b_a, W_x, b_x, Lambda and h0 (the
 * pages state no backward; this is the exact derivative of the forward
 * above).  dh_last, h0, hist_in and dh0 are nullable.  du is io; every other
 * gradient is fp32 and is WRITTEN, not accumulated.  The gradient of hist_in
 * is not produced.  Reads every field of w.  K = 256; D <= 2^24 (its
 * kernels address a chunk's rows with 32-bit offsets) and B <= 65535 (the
 * carry scan runs one grid row per stream); otherwise RGLRU_ERR_SHAPE.  The
 * workspace size depends on desc->io. */
int rglru_scan_bwd(const rglru_desc *desc, const rglru_weights *w, const void *u,
                   const void *hist_in, const float *h0, const void *dy,
                   const float *dh_last, void *du, float *dconv_w, float *dconv_b,
                   float *dW_a, float *db_a, float *dW_x, float *db_x, float *dLambda,
                   float *dh0, void *ws, size_t ws_bytes, hipStream_t stream);

/* Recurrent-block projections (device pointers, dtype desc->io, row-major,
 * stored [out][in] like a bias-free linear layer's weight). */
typedef struct {
    const void *proj_in_1;   /* [D][d_model]: branch 1 (conv + RG-LRU)  */
    const void *proj_in_2;   /* [D][d_model]: branch 2 (GeLU gate)      */
    const void *proj_out;    /* [d_model][D]: back to the model width   */
} rglru_block;

/* Workspace bytes of rglru_block_fwd for desc and d_model: the forward scan's
 * carries (same rules as rglru_workspace_size: ZERO-FILLED before first use,
 * reused only for calls with the same desc and d_model) followed by the two
 * branch activations.  Errors: RGLRU_ERR_NULL, _SHAPE (as rglru_block_fwd),
 * _DTYPE. */
int rglru_block_workspace_size(const rglru_desc *desc, int64_t d_model, size_t *bytes);

/* Recurrent block forward (page "Griffin Guide: RecurrentGemma, RG-LRU &
 * Hybrid Attention", section "The Recurrent Block Architecture", parts
 * "Temporal Filtering via Separable 1D Convolutions" and "Non-Linear
 * Multiplicative Gating with GeLU"; the listing's RecurrentBlock.forward):
 *     b1 = x proj_in_1^T,  b2 = x proj_in_2^T            [B][T][D]
 *     y  = RG-LRU(conv(b1))                              as rglru_scan_fwd mode A
 *     out = (y * GeLU(b2)) proj_out^T                    [B][T][d_model]
 * with GeLU(v) = v Phi(v), Phi the standard normal CDF (the exact form).  The
 * block has no biases and no residual add (that is the decoder layer's).
 * x and out are [B][T][d_model] in desc->io; h0, h_last, hist_in, hist_out
 * (nullable) are the state and conv history of branch 1, as in
 * rglru_scan_fwd.  The three projections are the library's own GEMMs (bf16:
 * on the matrix cores when the inner dimension is a multiple of 64) with
 * fp32 accumulation; b1 and b2 are rounded to io, and so is the merged
 * product that feeds proj_out.  Reads every field of w (conv_b, b_a, b_x
 * nullable).  K = 256; 1 <= d_model <= 2^30 and B*T, D, d_model each below
 * 2^31 for the GEMMs.  A launch error is RGLRU_ERR_LAUNCH (work enqueued
 * before it stays enqueued). */
int rglru_block_fwd(const rglru_desc *desc, int64_t d_model, const rglru_weights *w,
                    const rglru_block *blk, const void *x, const void *hist_in, const float *h0,
                    void *out, float *h_last, void *hist_out, void *ws, size_t ws_bytes,
                    hipStream_t stream);

/* Residual layer with the recurrent block as temporal mixer (a Hawk layer):
 * the pre-norm scaffold of the wiki note "Griffin", section "Residual Block
 * View", with the norms and MLP of the module page
 * "transformer_lens.model_bridge.supported_architectures.recurrent_gemma",
 * "Architecture overview":
 *     x~ = x + block(RMSNorm_t(x))                  (rglru_block_fwd's block)
 *     y  = x~ + down(GELU_tanh(gate RMSNorm_c(x~)) * (up RMSNorm_c(x~)))
 * RMSNorm(v) = v / sqrt(mean v^2 + eps) * (1 + weight); GELU_tanh(v) = v/2
 * (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))); no biases. */
typedef struct {
    const float *tnorm_w;   /* [d_model] fp32, temporal pre-norm weight     */
    const float *cnorm_w;   /* [d_model] fp32, channel pre-norm weight      */
    const void *gate_w;     /* [d_ff][d_model] io                           */
    const void *up_w;       /* [d_ff][d_model] io                           */
    const void *down_w;     /* [d_model][d_ff] io                           */
    int64_t d_ff;           /* MLP width, >= 1                              */
    float eps;              /* RMSNorm epsilon, finite and >= 0             */
} rglru_layer;

/* Workspace bytes of rglru_layer_fwd: the block's workspace (same rules:
 * ZERO-FILLED before first use, reused only for the same shapes) followed by
 * the normed input, the residual stream and the MLP's two activations. */
int rglru_layer_workspace_size(const rglru_desc *desc, int64_t d_model, const rglru_layer *lw, size_t *bytes);

/* Residual-layer forward.  x, y [B][T][d_model] (io); h0, h_last, hist_in,
 * hist_out (nullable) are the recurrent block's state and conv history.
 * Stored intermediates (the normed inputs, b1, b2, the merged product, x~,
 * the MLP activations) are rounded to io; every sum is fp32.  Five GEMMs
 * (the residual adds happen in the epilogues of proj_out and down), two
 * RMSNorm launches, the fused forward with the GeLU merge and one GELU-tanh
 * product launch.  Same shape limits and errors as rglru_block_fwd, plus d_ff. */
int rglru_layer_fwd(const rglru_desc *desc, int64_t d_model, const rglru_weights *w, const rglru_block *blk,
                    const rglru_layer *lw, const void *x, const void *hist_in, const float *h0, void *y,
                    float *h_last, void *hist_out, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Local sliding-window multi-query attention, Griffin's other temporal mixer
 * (wiki note "Griffin", section "Local Attention Path": token t attends to the
 * positions t-W+1 .. t, y_t = sum_i softmax_i(scale q_t . k_i) v_i; page
 * "Griffin Guide: RecurrentGemma, RG-LRU & Hybrid Attention", "Local
 * Sliding-Window Multi-Query Attention (MQA)": every query head shares one key
 * head and one value head; "Bounding the Key-Value Cache Footprint": the
 * decode cache holds the last W positions and evicts ring-buffer fashion).
 * The page's formula shows no score scale; `scale` is the caller's (1/sqrt(dh)
 * is the usual one).  q and k are taken after any rotary embedding, which
 * belongs to the attention block around this operation.
 *
 * Layouts (row-major, dtype io): q, o [B][T][Hq][dh]; k, v [B][T][dh];
 * caches kcache, vcache [B][W][dh], position p of stream b in slot p mod W;
 * decode: q_t, o_t [B][Hq][dh], k_t, v_t [B][dh], pos [B] int32 on the device
 * (the position of the new token, >= 0).  Scores, softmax and sums are fp32;
 * bf16 I/O with dh = 256 runs on the matrix cores (probabilities rounded to
 * bf16 for the P V product), every other shape on a vector-ALU path with
 * accurate exp.  Shapes: B, T, Hq >= 1; 1 <= W <= 2^30; 8 <= dh <= 256,
 * dh % 8 == 0. */
typedef struct {
    int64_t B, T, Hq, dh, W;
    int32_t io;        /* rglru_dtype */
    float scale;
} rglru_attn_desc;

/* Prefill: o for every token.  kcache / vcache (both or neither) receive the
 * keys and values of positions max(0, T-W) .. T-1 in their ring slots, ready
 * for rglru_attn_step at pos = T; other slots are left as they are. */
int rglru_attn_fwd(const rglru_attn_desc *desc, const void *q, const void *k, const void *v, void *o,
                   void *kcache, void *vcache, hipStream_t stream);

/* Workspace bytes of rglru_attn_step (desc->T is ignored): per-split partial
 * sums of the decode.  Contents need no initialisation. */
int rglru_attn_workspace_size(const rglru_attn_desc *desc, size_t *bytes);

/* One decode step for B streams: writes k_t, v_t into slot pos[b] mod W (the
 * slot of position pos[b] - W, evicted) and computes o_t over positions
 * max(0, pos[b]-W+1) .. pos[b] (desc->T is ignored).  Slots of positions
 * below 0 are never read, so a fresh cache needs no initialisation.  The
 * caller advances pos. */
int rglru_attn_step(const rglru_attn_desc *desc, const void *q_t, const void *k_t, const void *v_t,
                    void *kcache, void *vcache, const int32_t *pos, void *o_t, void *ws, size_t ws_bytes,
                    hipStream_t stream);

/* Attention residual layer (Griffin's third block kind): the scaffold of
 * rglru_layer_fwd with local MQA as temporal mixer,
 *     q = RoPE(RMSNorm_t(x) wq^T), k = RoPE(RMSNorm_t(x) wk^T), v = RMSNorm_t(x) wv^T
 *     x~ = x + attn(q, k, v) wo^T            (rglru_attn_fwd, window desc->W)
 *     y  = x~ + gated MLP(RMSNorm_c(x~))     (as in rglru_layer_fwd)
 * The rotary embedding (page "Griffin Guide", "Local Sliding-Window
 * Multi-Query Attention (MQA)": standard RoPE on queries and keys; module
 * page: partial rotary) turns dimension pairs (j, j + rot/2), j < rot/2, of
 * every head by p * rope_base^(-2j/rot) at position p = pos0 + t; dimensions
 * >= rot are left as they are.  Projections are bias-free, stored [out][in]
 * in desc->io.  x, y [B][T][d_model].  kcache / vcache (both or neither)
 * receive the rotated keys and the values of the last W positions in ring
 * order, as rglru_attn_fwd.  Shapes as rglru_attn_fwd and rglru_layer_fwd;
 * 0 <= rot <= dh, rot even; rope_base > 1; 0 <= pos0, pos0 + T < 2^31. */
typedef struct {
    const void *wq;   /* [Hq*dh][d_model] */
    const void *wk;   /* [dh][d_model]    */
    const void *wv;   /* [dh][d_model]    */
    const void *wo;   /* [d_model][Hq*dh] */
} rglru_attn_proj;

/* Workspace bytes of rglru_attn_layer_fwd (no initialisation needed). */
int rglru_attn_layer_workspace_size(const rglru_attn_desc *desc, int64_t d_model, const rglru_layer *lw,
                                    size_t *bytes);

int rglru_attn_layer_fwd(const rglru_attn_desc *desc, int64_t d_model, int32_t rot, float rope_base, int64_t pos0,
                         const rglru_attn_proj *ap, const rglru_layer *lw, const void *x, void *y, void *kcache,
                         void *vcache, void *ws, size_t ws_bytes, hipStream_t stream);

/* Short English text of a status code (static storage). */
const char *rglru_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* RGLRU_H */
