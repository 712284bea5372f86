// api.hip -- the extern "C" entry points of librglru.so (declared and
// documented in include/rglru.h).  Every check runs here, on the host, before
// anything is enqueued; the launchers behind them assume valid arguments.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "internal.h"

using namespace rglru;

// Workspace of rglru_scan_fwd_noalloc, one copy per device (file scope).
constexpr size_t NOALLOC_SCRATCH_BYTES = RGLRU_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t MAX_DIM = (int64_t)1 << 30;
constexpr int64_t BWD_MAX_D = (int64_t)1 << 24;   // 32-bit row offsets in the backward
constexpr int64_t BWD_MAX_B = 65535;               // streams: one grid row each in the carry scan

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t esize(const rglru_desc &d) { return d.io == RGLRU_BF16 ? 2 : 4; }

int check_desc(const rglru_desc *d, bool need_k256)
{
    if (!d) return RGLRU_ERR_NULL;
    if (d->io != RGLRU_F32 && d->io != RGLRU_BF16) return RGLRU_ERR_DTYPE;
    if (d->B < 1 || d->T < 1 || d->D < 1 || d->H < 1) return RGLRU_ERR_SHAPE;
    if (d->B > MAX_DIM || d->T > MAX_DIM || d->D > MAX_DIM || d->D % d->H != 0) return RGLRU_ERR_SHAPE;
    if ((double)d->B * (double)d->T * (double)d->D > 9.0e15) return RGLRU_ERR_SHAPE;
    const int64_t NC = (d->T + 31) / 32, G = (d->D + 255) / 256;
    if ((double)d->B * NC * G >= 2147483647.0) return RGLRU_ERR_SHAPE;   // work units fit a grid
    if (need_k256 && d->D / d->H != 256) return RGLRU_ERR_SHAPE;
    if (G > MAX_CLAIM_GROUPS) return RGLRU_ERR_SHAPE;   // claim counters of the chunked scans
    if (!isfinite(d->c)) return RGLRU_ERR_ARG;
    return RGLRU_OK;
}

// the recurrent block: the scan's checks plus the GEMM sizes (each GEMM
// dimension below 2^31)
int check_block(const rglru_desc *d, int64_t d_model)
{
    int st = check_desc(d, true);
    if (st) return st;
    if (d_model < 1 || d_model > MAX_DIM) return RGLRU_ERR_SHAPE;
    if (d->B * d->T >= 2147483647 || d->D >= 2147483647) return RGLRU_ERR_SHAPE;
    if ((double)d->B * (double)d->T * (double)d_model > 9.0e15) return RGLRU_ERR_SHAPE;
    return RGLRU_OK;
}

// residual layer: the block's checks plus the MLP width and the norm epsilon
int check_layer(const rglru_desc *d, int64_t d_model, const rglru_layer *lw)
{
    int st = check_block(d, d_model);
    if (st) return st;
    if (lw->d_ff < 1 || lw->d_ff >= 2147483647) return RGLRU_ERR_SHAPE;
    if ((double)d->B * (double)d->T * (double)lw->d_ff > 9.0e15) return RGLRU_ERR_SHAPE;
    if (!isfinite(lw->eps) || lw->eps < 0.0f) return RGLRU_ERR_ARG;
    return RGLRU_OK;
}

// local attention: shapes of the descriptor (prefill also needs T)
int check_attn(const rglru_attn_desc *d, bool prefill)
{
    if (!d) return RGLRU_ERR_NULL;
    if (d->io != RGLRU_F32 && d->io != RGLRU_BF16) return RGLRU_ERR_DTYPE;
    if (d->B < 1 || d->Hq < 1 || d->W < 1 || d->dh < 8 || d->dh > 256 || d->dh % 8 != 0)
        return RGLRU_ERR_SHAPE;
    if (d->B > MAX_DIM || d->Hq > 4096 || d->W > MAX_DIM) return RGLRU_ERR_SHAPE;
    if (prefill && (d->T < 1 || d->T > MAX_DIM)) return RGLRU_ERR_SHAPE;
    const double T = prefill ? (double)d->T : 1.0;
    if ((double)d->B * T * d->Hq * d->dh > 9.0e15 || (double)d->B * d->W * d->dh > 9.0e15) return RGLRU_ERR_SHAPE;
    // grids: one workgroup per 128 rows (prefill) or per 4 rows (vector path)
    if ((double)d->B * T * d->Hq / 4.0 >= 2147483647.0) return RGLRU_ERR_SHAPE;
    if (prefill && d->T * d->Hq >= 2147483647) return RGLRU_ERR_SHAPE;
    if (!isfinite(d->scale)) return RGLRU_ERR_ARG;
    return RGLRU_OK;
}

// attention layer: the prefill's checks plus the model and MLP widths
int check_attn_layer(const rglru_attn_desc *d, int64_t d_model, const rglru_layer *lw)
{
    int st = check_attn(d, true);
    if (st) return st;
    if (d_model < 1 || d_model > MAX_DIM || lw->d_ff < 1 || lw->d_ff >= 2147483647) return RGLRU_ERR_SHAPE;
    if (d->B * d->T >= 2147483647 || d->Hq * d->dh >= 2147483647) return RGLRU_ERR_SHAPE;
    if ((double)d->B * d->T * (double)(d_model > lw->d_ff ? d_model : lw->d_ff) > 9.0e15) return RGLRU_ERR_SHAPE;
    if (!isfinite(lw->eps) || lw->eps < 0.0f) return RGLRU_ERR_ARG;
    return RGLRU_OK;
}

struct Range {
    const void *p;
    size_t bytes;
};

bool overlap(Range a, Range b)
{
    if (!a.p || !b.p || !a.bytes || !b.bytes) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// any output range overlapping any input range (or another output)
bool any_alias(const Range *outs, int nout, const Range *ins, int nin)
{
    for (int o = 0; o < nout; ++o) {
        for (int k = 0; k < nin; ++k)
            if (overlap(outs[o], ins[k])) return true;
        for (int k = o + 1; k < nout; ++k)
            if (overlap(outs[o], outs[k])) return true;
    }
    return false;
}

int launch_status()
{
    return hipGetLastError() == hipSuccess ? RGLRU_OK : RGLRU_ERR_LAUNCH;
}

// Checks of the forward scan's arguments, shared by rglru_scan_fwd (own_ws:
// the caller's workspace ws of ws_bytes) and rglru_scan_fwd_noalloc (the
// library's scratch, which no caller buffer can overlap).  *mode receives
// 0, 1 or 2 for modes A, B, C.
int check_scan_fwd(const rglru_desc *desc, const rglru_weights *w, const void *in, const void *r,
                   const void *i, const void *hist_in, const float *h0, const void *y, const float *h_last,
                   const void *hist_out, bool own_ws, const void *ws, size_t ws_bytes, int *mode)
{
    if (!desc || !w) return RGLRU_ERR_NULL;
    if ((r == nullptr) != (i == nullptr)) return RGLRU_ERR_ARG;
    const int m = r ? 2 : (w->conv_w ? 0 : 1);
    if (m == 2 && w->conv_w) return RGLRU_ERR_ARG;
    if (m != 0 && (hist_in || hist_out)) return RGLRU_ERR_ARG;
    int st = check_desc(desc, m != 2);
    if (st) return st;
    if (!in || !y || !w->Lambda) return RGLRU_ERR_NULL;
    if (m != 2 && (!w->W_a || !w->W_x)) return RGLRU_ERR_NULL;
    if (own_ws && !ws) return RGLRU_ERR_WORKSPACE;
    const void *all[] = {in, r, i, hist_in, h0, y, h_last, hist_out, ws, w->conv_w, w->conv_b,
                         w->W_a, w->b_a, w->W_x, w->b_x, w->Lambda};
    for (const void *p : all)
        if (p && !aligned16(p)) return RGLRU_ERR_ALIGN;
    const rglru_desc &d = *desc;
    const size_t need = fwd_workspace_bytes(d.B, d.T, d.D);
    if (own_ws && ws_bytes < need) return RGLRU_ERR_WORKSPACE;
    if (!own_ws && need > NOALLOC_SCRATCH_BYTES) return RGLRU_ERR_SCRATCH;
    const size_t act = d.B * d.T * d.D * esize(d), hist = d.B * 3 * d.D * esize(d);
    const size_t st_b = d.B * d.D * 4, vec = d.D * 4;
    const size_t wb = m == 2 ? 0 : d.H * 65536 * esize(d);
    const Range outs[] = {{y, act}, {h_last, st_b}, {hist_out, hist}, {ws, own_ws ? need : 0}};
    const Range ins[] = {{in, act}, {r, act}, {i, act}, {hist_in, hist}, {h0, st_b},
                         {w->conv_w, m == 0 ? vec * 4 : 0}, {w->conv_b, m == 0 ? vec : 0},
                         {w->W_a, wb}, {w->W_x, wb}, {w->b_a, m == 2 ? 0 : vec},
                         {w->b_x, m == 2 ? 0 : vec}, {w->Lambda, vec}};
    if (any_alias(outs, 4, ins, 12)) return RGLRU_ERR_ARG;
    *mode = m;
    return RGLRU_OK;
}

// ------------------------------------------- scratch of rglru_scan_fwd_noalloc
// The forward scan's workspace for callers that cannot allocate: one array per
// device, loaded with the library's code object and held until the process
// ends.  In host code the name `scratch` is only a stand-in for the symbol;
// the device address of each device's copy comes from hipGetSymbolAddress,
// taken once per device and cleared once (a plain fill kernel, so that a
// captured first call records no memset).  Every later call leaves the
// header as it found it and tags its carry words with its own launch number,
// so no call clears anything again.
constexpr int NOALLOC_MAX_DEVICES = 64;

__global__ void __launch_bounds__(256) scratch_clear_kernel(uint4 *p, size_t n16)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t k = (size_t)blockIdx.x * blockDim.x + threadIdx.x; k < n16; k += stride)
        p[k] = make_uint4(0u, 0u, 0u, 0u);
}

int noalloc_scratch(hipStream_t stream, void **out)
{
    static std::mutex mu;
    static void *ptr[NOALLOC_MAX_DEVICES];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return RGLRU_ERR_LAUNCH;
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return RGLRU_ERR_ARG;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RGLRU_ERR_LAUNCH;
        scratch_clear_kernel<<<dim3(1024), dim3(256), 0, stream>>>((uint4 *)p, NOALLOC_SCRATCH_BYTES / 16);
        if (hipGetLastError() != hipSuccess) return RGLRU_ERR_LAUNCH;
        ptr[dev] = p;
    }
    *out = ptr[dev];
    return RGLRU_OK;
}

}  // namespace

extern "C" {

const char *rglru_status_string(int status)
{
    switch (status) {
    case RGLRU_OK: return "ok";
    case RGLRU_ERR_NULL: return "a required pointer is NULL";
    case RGLRU_ERR_SHAPE: return "bad shape (B, T, D, H, block width K = D/H must be 256, T must be 1 for a step)";
    case RGLRU_ERR_DTYPE: return "unknown io dtype";
    case RGLRU_ERR_ALIGN: return "pointer not 16-byte aligned";
    case RGLRU_ERR_WORKSPACE: return "workspace missing or too small";
    case RGLRU_ERR_LAUNCH: return "HIP launch error";
    case RGLRU_ERR_ARG: return "inconsistent arguments";
    case RGLRU_ERR_BLAS: return "reserved status (not returned)";
    case RGLRU_ERR_SCRATCH: return "problem needs more than the fixed scratch of rglru_scan_fwd_noalloc";
    case RGLRU_ERR_TIMEOUT: return "a chunk-carry wait of an earlier call on this workspace gave up (its outputs hold NaN)";
    default: return "unknown status";
    }
}

int rglru_workspace_status(const void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (!ws) return RGLRU_ERR_NULL;
    if (!aligned16(ws)) return RGLRU_ERR_ALIGN;
    if (ws_bytes < 256) return RGLRU_ERR_WORKSPACE;
    if (hipStreamSynchronize(stream) != hipSuccess) return RGLRU_ERR_LAUNCH;
    uint32_t flag = 0;
    char *word = (char *)ws + WS_ERROR_OFFSET;
    if (hipMemcpy(&flag, word, sizeof(flag), hipMemcpyDeviceToHost) != hipSuccess) return RGLRU_ERR_LAUNCH;
    if (flag == 0) return RGLRU_OK;
    const uint32_t zero = 0;
    if (hipMemcpy(word, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return RGLRU_ERR_LAUNCH;
    return RGLRU_ERR_TIMEOUT;
}

int rglru_workspace_size(const rglru_desc *desc, int op, size_t *bytes)
{
    if (!bytes) return RGLRU_ERR_NULL;
    int st = check_desc(desc, false);
    if (st) return st;
    if (op == RGLRU_OP_SCAN_FWD) *bytes = fwd_workspace_bytes(desc->B, desc->T, desc->D);
    else if (op == RGLRU_OP_SCAN_BWD) {
        if (desc->D / desc->H != 256 || desc->D > BWD_MAX_D) return RGLRU_ERR_SHAPE;
        *bytes = bwd_workspace_bytes(desc->B, desc->T, desc->D, desc->H, esize(*desc));
    } else return RGLRU_ERR_ARG;
    return RGLRU_OK;
}

int rglru_conv1d(const rglru_desc *desc, const float *conv_w, const float *conv_b, const void *u,
                 const void *hist_in, void *x, void *hist_out, hipStream_t stream)
{
    int st = check_desc(desc, false);
    if (st) return st;
    if (!conv_w || !u || !x) return RGLRU_ERR_NULL;
    const void *all[] = {conv_w, conv_b, u, hist_in, x, hist_out};
    for (const void *p : all)
        if (p && !aligned16(p)) return RGLRU_ERR_ALIGN;
    const rglru_desc &d = *desc;
    const size_t act = d.B * d.T * d.D * esize(d), hist = d.B * 3 * d.D * esize(d);
    const Range outs[] = {{x, act}, {hist_out, hist}};
    const Range ins[] = {{conv_w, (size_t)d.D * 16}, {conv_b, (size_t)d.D * 4}, {u, act}, {hist_in, hist}};
    if (any_alias(outs, 2, ins, 4)) return RGLRU_ERR_ARG;
    launch_conv1d(d, conv_w, conv_b, u, hist_in, x, hist_out, stream);
    return launch_status();
}

int rglru_gates(const rglru_desc *desc, const rglru_weights *w, const void *x, void *r, void *i,
                hipStream_t stream)
{
    int st = check_desc(desc, true);
    if (st) return st;
    if (!w || !w->W_a || !w->W_x || !x || !r || !i) return RGLRU_ERR_NULL;
    const void *all[] = {w->W_a, w->W_x, w->b_a, w->b_x, x, r, i};
    for (const void *p : all)
        if (p && !aligned16(p)) return RGLRU_ERR_ALIGN;
    const rglru_desc &d = *desc;
    const size_t act = d.B * d.T * d.D * esize(d), wb = d.H * 65536 * esize(d);
    const Range outs[] = {{r, act}, {i, act}};
    const Range ins[] = {{x, act}, {w->W_a, wb}, {w->W_x, wb}, {w->b_a, (size_t)d.D * 4}, {w->b_x, (size_t)d.D * 4}};
    if (any_alias(outs, 2, ins, 5)) return RGLRU_ERR_ARG;
    launch_gates(d, *w, x, r, i, stream);
    return launch_status();
}

int rglru_scan_fwd(const rglru_desc *desc, const rglru_weights *w, const void *in, const void *r,
                   const void *i, const void *hist_in, const float *h0, void *y, float *h_last,
                   void *hist_out, void *ws, size_t ws_bytes, hipStream_t stream)
{
    int mode = 0;
    const int st = check_scan_fwd(desc, w, in, r, i, hist_in, h0, y, h_last, hist_out, true, ws, ws_bytes, &mode);
    if (st) return st;
    launch_scan_fwd(*desc, *w, mode, in, r, i, hist_in, h0, y, h_last, hist_out, ws, stream);
    return launch_status();
}

int rglru_scan_fwd_noalloc(const rglru_desc *desc, const rglru_weights *w, const void *in, const void *r,
                           const void *i, const void *hist_in, const float *h0, void *y, float *h_last,
                           void *hist_out, hipStream_t stream)
{
    int mode = 0;
    int st = check_scan_fwd(desc, w, in, r, i, hist_in, h0, y, h_last, hist_out, false, nullptr, 0, &mode);
    if (st) return st;
    void *ws = nullptr;
    st = noalloc_scratch(stream, &ws);
    if (st) return st;
    launch_scan_fwd(*desc, *w, mode, in, r, i, hist_in, h0, y, h_last, hist_out, ws, stream);
    return launch_status();
}

int rglru_step(const rglru_desc *desc, const rglru_weights *w, const void *u_t, const void *hist_in,
               void *hist_out, float *h, void *y_t, hipStream_t stream)
{
    int st = check_desc(desc, true);
    if (st) return st;
    if (desc->T != 1) return RGLRU_ERR_SHAPE;
    if (!w || !w->conv_w || !w->W_a || !w->W_x || !w->Lambda || !u_t || !h || !y_t) return RGLRU_ERR_NULL;
    const void *all[] = {u_t, hist_in, hist_out, h, y_t, w->conv_w, w->conv_b, w->W_a, w->b_a, w->W_x, w->b_x,
                         w->Lambda};
    for (const void *p : all)
        if (p && !aligned16(p)) return RGLRU_ERR_ALIGN;
    const rglru_desc &d = *desc;
    const size_t row = d.B * d.D * esize(d), hb = d.B * 3 * d.D * esize(d), sb = d.B * d.D * 4;
    const size_t vec = d.D * 4, wb = d.H * 65536 * esize(d);
    // h is read and rewritten in place by design; no output may overlap another
    // output or an input (hist_out and hist_in included)
    const Range outs[] = {{y_t, row}, {hist_out, hb}, {h, sb}};
    const Range ins[] = {{u_t, row}, {hist_in, hb}, {w->conv_w, vec * 4}, {w->conv_b, vec}, {w->W_a, wb},
                         {w->b_a, vec}, {w->W_x, wb}, {w->b_x, vec}, {w->Lambda, vec}};
    if (any_alias(outs, 3, ins, 9)) return RGLRU_ERR_ARG;
    launch_step(d, *w, u_t, hist_in, hist_out, h, y_t, stream);
    return launch_status();
}

int rglru_scan_bwd(const rglru_desc *desc, const rglru_weights *w, const void *u, const void *hist_in,
                   const float *h0, const void *dy, const float *dh_last, void *du, float *dconv_w,
                   float *dconv_b, float *dW_a, float *db_a, float *dW_x, float *db_x, float *dLambda,
                   float *dh0, void *ws, size_t ws_bytes, hipStream_t stream)
{
    int st = check_desc(desc, true);
    if (st) return st;
    if (desc->D > BWD_MAX_D || desc->B > BWD_MAX_B) return RGLRU_ERR_SHAPE;
    if (!w || !w->conv_w || !w->W_a || !w->W_x || !w->Lambda || !u || !dy || !du || !dconv_w ||
        !dconv_b || !dW_a || !db_a || !dW_x || !db_x || !dLambda)
        return RGLRU_ERR_NULL;
    if (!ws) return RGLRU_ERR_WORKSPACE;
    const void *all[] = {u, hist_in, h0, dy, dh_last, du, dconv_w, dconv_b, dW_a, db_a, dW_x,
                         db_x, dLambda, dh0, ws, w->conv_w, w->conv_b, w->W_a, w->b_a,
                         w->W_x, w->b_x, w->Lambda};
    for (const void *p : all)
        if (p && !aligned16(p)) return RGLRU_ERR_ALIGN;
    const rglru_desc &d = *desc;
    const size_t need = bwd_workspace_bytes(d.B, d.T, d.D, d.H, esize(d));
    if (ws_bytes < need) return RGLRU_ERR_WORKSPACE;
    const size_t act = d.B * d.T * d.D * esize(d), hist = d.B * 3 * d.D * esize(d);
    const size_t sb = d.B * d.D * 4, vec = d.D * 4, wb = d.H * 65536 * esize(d), wf = d.H * 65536 * 4;
    const Range outs[] = {{du, act}, {dconv_w, vec * 4}, {dconv_b, vec}, {dW_a, wf}, {db_a, vec},
                          {dW_x, wf}, {db_x, vec}, {dLambda, vec}, {dh0, sb}, {ws, need}};
    const Range ins[] = {{u, act}, {hist_in, hist}, {h0, sb}, {dy, act}, {dh_last, sb},
                         {w->conv_w, vec * 4}, {w->conv_b, vec}, {w->W_a, wb}, {w->b_a, vec},
                         {w->W_x, wb}, {w->b_x, vec}, {w->Lambda, vec}};
    if (any_alias(outs, 10, ins, 12)) return RGLRU_ERR_ARG;
    launch_scan_bwd(d, *w, u, hist_in, h0, dy, dh_last, du, dconv_w, dconv_b, dW_a, db_a, dW_x, db_x,
                    dLambda, dh0, ws, stream);
    return launch_status();
}

int rglru_block_workspace_size(const rglru_desc *desc, int64_t d_model, size_t *bytes)
{
    if (!bytes) return RGLRU_ERR_NULL;
    int st = check_block(desc, d_model);
    if (st) return st;
    *bytes = block_layout(desc->B, desc->T, desc->D, esize(*desc)).bytes;
    return RGLRU_OK;
}

int rglru_block_fwd(const rglru_desc *desc, int64_t d_model, const rglru_weights *w, const rglru_block *blk,
                    const void *x, const void *hist_in, const float *h0, void *out, float *h_last,
                    void *hist_out, void *ws, size_t ws_bytes, hipStream_t stream)
{
    int st = check_block(desc, d_model);
    if (st) return st;
    if (!w || !blk || !w->conv_w || !w->W_a || !w->W_x || !w->Lambda || !blk->proj_in_1 ||
        !blk->proj_in_2 || !blk->proj_out || !x || !out)
        return RGLRU_ERR_NULL;
    if (!ws) return RGLRU_ERR_WORKSPACE;
    const void *all[] = {x, hist_in, h0, out, h_last, hist_out, ws, w->conv_w, w->conv_b, w->W_a,
                         w->b_a, w->W_x, w->b_x, w->Lambda, blk->proj_in_1, blk->proj_in_2, blk->proj_out};
    for (const void *p : all)
        if (p && !aligned16(p)) return RGLRU_ERR_ALIGN;
    const rglru_desc &d = *desc;
    const size_t need = block_layout(d.B, d.T, d.D, esize(d)).bytes;
    if (ws_bytes < need) return RGLRU_ERR_WORKSPACE;
    const size_t e = esize(d), io_x = d.B * d.T * d_model * e, hist = d.B * 3 * d.D * e;
    const size_t sb = d.B * d.D * 4, vec = d.D * 4, wb = d.H * 65536 * e, pw = d.D * d_model * e;
    const Range outs[] = {{out, io_x}, {h_last, sb}, {hist_out, hist}, {ws, need}};
    const Range ins[] = {{x, io_x}, {hist_in, hist}, {h0, sb}, {w->conv_w, vec * 4}, {w->conv_b, vec},
                         {w->W_a, wb}, {w->b_a, vec}, {w->W_x, wb}, {w->b_x, vec}, {w->Lambda, vec},
                         {blk->proj_in_1, pw}, {blk->proj_in_2, pw}, {blk->proj_out, pw}};
    if (any_alias(outs, 4, ins, 13)) return RGLRU_ERR_ARG;
    st = launch_block_fwd(d, d_model, *w, *blk, x, hist_in, h0, out, h_last, hist_out, ws, stream);
    if (st) return st;
    return launch_status();
}

int rglru_layer_workspace_size(const rglru_desc *desc, int64_t d_model, const rglru_layer *lw, size_t *bytes)
{
    if (!bytes || !lw) return RGLRU_ERR_NULL;
    int st = check_layer(desc, d_model, lw);
    if (st) return st;
    *bytes = layer_layout(desc->B, desc->T, desc->D, d_model, lw->d_ff, esize(*desc)).bytes;
    return RGLRU_OK;
}

int rglru_layer_fwd(const rglru_desc *desc, int64_t d_model, const rglru_weights *w, const rglru_block *blk,
                    const rglru_layer *lw, const void *x, const void *hist_in, const float *h0, void *y,
                    float *h_last, void *hist_out, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (!lw) return RGLRU_ERR_NULL;
    int st = check_layer(desc, d_model, lw);
    if (st) return st;
    if (!w || !blk || !w->conv_w || !w->W_a || !w->W_x || !w->Lambda || !blk->proj_in_1 || !blk->proj_in_2 ||
        !blk->proj_out || !lw->tnorm_w || !lw->cnorm_w || !lw->gate_w || !lw->up_w || !lw->down_w || !x || !y)
        return RGLRU_ERR_NULL;
    if (!ws) return RGLRU_ERR_WORKSPACE;
    const void *all[] = {x, hist_in, h0, y, h_last, hist_out, ws, w->conv_w, w->conv_b, w->W_a, w->b_a, w->W_x,
                         w->b_x, w->Lambda, blk->proj_in_1, blk->proj_in_2, blk->proj_out, lw->tnorm_w,
                         lw->cnorm_w, lw->gate_w, lw->up_w, lw->down_w};
    for (const void *p : all)
        if (p && !aligned16(p)) return RGLRU_ERR_ALIGN;
    const rglru_desc &d = *desc;
    const size_t need = layer_layout(d.B, d.T, d.D, d_model, lw->d_ff, esize(d)).bytes;
    if (ws_bytes < need) return RGLRU_ERR_WORKSPACE;
    const size_t e = esize(d), io_x = d.B * d.T * d_model * e, hist = d.B * 3 * d.D * e;
    const size_t sb = d.B * d.D * 4, vec = d.D * 4, wb = d.H * 65536 * e, pw = d.D * d_model * e;
    const size_t fw = lw->d_ff * d_model * e, nv = d_model * 4;
    const Range outs[] = {{y, io_x}, {h_last, sb}, {hist_out, hist}, {ws, need}};
    const Range ins[] = {{x, io_x}, {hist_in, hist}, {h0, sb}, {w->conv_w, vec * 4}, {w->conv_b, vec},
                         {w->W_a, wb}, {w->b_a, vec}, {w->W_x, wb}, {w->b_x, vec}, {w->Lambda, vec},
                         {blk->proj_in_1, pw}, {blk->proj_in_2, pw}, {blk->proj_out, pw}, {lw->tnorm_w, nv},
                         {lw->cnorm_w, nv}, {lw->gate_w, fw}, {lw->up_w, fw}, {lw->down_w, fw}};
    if (any_alias(outs, 4, ins, 18)) return RGLRU_ERR_ARG;
    st = launch_layer_fwd(d, d_model, *w, *blk, *lw, x, hist_in, h0, y, h_last, hist_out, ws, stream);
    if (st) return st;
    return launch_status();
}

int rglru_attn_layer_workspace_size(const rglru_attn_desc *desc, int64_t d_model, const rglru_layer *lw,
                                    size_t *bytes)
{
    if (!bytes || !lw) return RGLRU_ERR_NULL;
    int st = check_attn_layer(desc, d_model, lw);
    if (st) return st;
    *bytes = attn_layer_layout(*desc, d_model, lw->d_ff).bytes;
    return RGLRU_OK;
}

int rglru_attn_layer_fwd(const rglru_attn_desc *desc, int64_t d_model, int32_t rot, float rope_base, int64_t pos0,
                         const rglru_attn_proj *ap, const rglru_layer *lw, const void *x, void *y, void *kcache,
                         void *vcache, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (!ap || !lw) return RGLRU_ERR_NULL;
    int st = check_attn_layer(desc, d_model, lw);
    if (st) return st;
    const rglru_attn_desc &d = *desc;
    if (rot < 0 || rot > d.dh || rot % 2 != 0 || !(rope_base > 1.0f) || !isfinite(rope_base)) return RGLRU_ERR_ARG;
    if (pos0 < 0 || pos0 + d.T >= 2147483647) return RGLRU_ERR_SHAPE;
    if (!ap->wq || !ap->wk || !ap->wv || !ap->wo || !lw->tnorm_w || !lw->cnorm_w || !lw->gate_w || !lw->up_w ||
        !lw->down_w || !x || !y)
        return RGLRU_ERR_NULL;
    if ((kcache == nullptr) != (vcache == nullptr)) return RGLRU_ERR_ARG;
    if (!ws) return RGLRU_ERR_WORKSPACE;
    const void *all[] = {x, y, kcache, vcache, ws, ap->wq, ap->wk, ap->wv, ap->wo, lw->tnorm_w, lw->cnorm_w,
                         lw->gate_w, lw->up_w, lw->down_w};
    for (const void *p : all)
        if (p && !aligned16(p)) return RGLRU_ERR_ALIGN;
    const size_t need = attn_layer_layout(d, d_model, lw->d_ff).bytes;
    if (ws_bytes < need) return RGLRU_ERR_WORKSPACE;
    const size_t e = d.io == RGLRU_BF16 ? 2 : 4, io_x = d.B * d.T * d_model * e, cb = d.B * d.W * d.dh * e;
    const size_t wqb = d.Hq * d.dh * d_model * e, wkb = d.dh * d_model * e, fw = lw->d_ff * d_model * e,
                 nv = d_model * 4;
    const Range outs[] = {{y, io_x}, {kcache, cb}, {vcache, cb}, {ws, need}};
    const Range ins[] = {{x, io_x}, {ap->wq, wqb}, {ap->wk, wkb}, {ap->wv, wkb}, {ap->wo, wqb},
                         {lw->tnorm_w, nv}, {lw->cnorm_w, nv}, {lw->gate_w, fw}, {lw->up_w, fw}, {lw->down_w, fw}};
    if (any_alias(outs, 4, ins, 10)) return RGLRU_ERR_ARG;
    st = launch_attn_layer_fwd(d, d_model, rot, rope_base, pos0, *ap, *lw, x, y, kcache, vcache, ws, stream);
    if (st) return st;
    return launch_status();
}

int rglru_attn_workspace_size(const rglru_attn_desc *desc, size_t *bytes)
{
    if (!bytes) return RGLRU_ERR_NULL;
    int st = check_attn(desc, false);
    if (st) return st;
    *bytes = attn_workspace_bytes(*desc);
    return RGLRU_OK;
}

int rglru_attn_fwd(const rglru_attn_desc *desc, const void *q, const void *k, const void *v, void *o,
                   void *kcache, void *vcache, hipStream_t stream)
{
    int st = check_attn(desc, true);
    if (st) return st;
    if (!q || !k || !v || !o) return RGLRU_ERR_NULL;
    if ((kcache == nullptr) != (vcache == nullptr)) return RGLRU_ERR_ARG;
    const void *all[] = {q, k, v, o, kcache, vcache};
    for (const void *p : all)
        if (p && !aligned16(p)) return RGLRU_ERR_ALIGN;
    const rglru_attn_desc &d = *desc;
    const size_t e = d.io == RGLRU_BF16 ? 2 : 4;
    const size_t qb = d.B * d.T * d.Hq * d.dh * e, kb = d.B * d.T * d.dh * e, cb = d.B * d.W * d.dh * e;
    const Range outs[] = {{o, qb}, {kcache, cb}, {vcache, cb}};
    const Range ins[] = {{q, qb}, {k, kb}, {v, kb}};
    if (any_alias(outs, 3, ins, 3)) return RGLRU_ERR_ARG;
    launch_attn_fwd(d, q, k, v, o, kcache, vcache, stream);
    return launch_status();
}

int rglru_attn_step(const rglru_attn_desc *desc, const void *q_t, const void *k_t, const void *v_t,
                    void *kcache, void *vcache, const int32_t *pos, void *o_t, void *ws, size_t ws_bytes,
                    hipStream_t stream)
{
    int st = check_attn(desc, false);
    if (st) return st;
    if (!q_t || !k_t || !v_t || !kcache || !vcache || !pos || !o_t) return RGLRU_ERR_NULL;
    if (!ws) return RGLRU_ERR_WORKSPACE;
    const void *all[] = {q_t, k_t, v_t, kcache, vcache, o_t, ws};
    for (const void *p : all)
        if (!aligned16(p)) return RGLRU_ERR_ALIGN;
    if (((uintptr_t)pos & 3u) != 0) return RGLRU_ERR_ALIGN;
    const rglru_attn_desc &d = *desc;
    const size_t need = attn_workspace_bytes(d);
    if (ws_bytes < need) return RGLRU_ERR_WORKSPACE;
    const size_t e = d.io == RGLRU_BF16 ? 2 : 4;
    const size_t qb = d.B * d.Hq * d.dh * e, kb = d.B * d.dh * e, cb = d.B * d.W * d.dh * e;
    // the caches are read and rewritten in place by design
    const Range outs[] = {{o_t, qb}, {kcache, cb}, {vcache, cb}, {ws, need}};
    const Range ins[] = {{q_t, qb}, {k_t, kb}, {v_t, kb}, {pos, (size_t)d.B * 4}};
    if (any_alias(outs, 4, ins, 4)) return RGLRU_ERR_ARG;
    launch_attn_step(d, q_t, k_t, v_t, kcache, vcache, pos, o_t, ws, stream);
    return launch_status();
}

}  // extern "C"
