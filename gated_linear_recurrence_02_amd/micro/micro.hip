// micro.hip -- microbenchmarks of the ceilings the path's kernels are held
// against on this GPU: vector-ALU throughput of plain FMAs and of the
// transcendental instructions the gate and decay math uses (exp2, rcp,
// sqrt), bf16 matrix-core throughput, and plain device copy bandwidth.
// Built into its own library (librglru_micro.so), not part of librglru.so;
// bench.py --micro launches these and times them with HIP events.
//
// Each kernel writes one value per thread so that nothing is optimised away;
// the values themselves mean nothing.
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 8 independent chains per thread, `iters` rounds; KIND 0 fma, 1 exp2,
// 2 rcp, 3 sqrt, 4 exp2 and fma alternating
template <int KIND>
__global__ __launch_bounds__(256) void valu_kernel(float *out, int iters, float s)
{
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = s * (float)(threadIdx.x + j);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (KIND == 0) v[j] = __builtin_fmaf(v[j], s, 0.5f);
            if (KIND == 1) v[j] = __builtin_amdgcn_exp2f(v[j]);
            if (KIND == 2) v[j] = __builtin_amdgcn_rcpf(v[j]);
            if (KIND == 3) v[j] = __builtin_amdgcn_sqrtf(v[j]);
            if (KIND == 4) v[j] = (j & 1) ? __builtin_amdgcn_exp2f(v[j]) : __builtin_fmaf(v[j], s, 0.5f);
        }
    }
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += v[j];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// 4 independent v_mfma_f32_32x32x16_bf16 chains per wave, `iters` rounds
__global__ __launch_bounds__(256) void mfma_kernel(float *out, int iters)
{
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(0.001f * (float)(threadIdx.x + e));
        b[e] = (__bf16)(0.002f * (float)(threadIdx.x - e));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc += c0[e] + c1[e] + c2[e] + c3[e];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// co-execution: 8-wave workgroups, waves w and w + 4 share a SIMD.  mode 0:
// waves 0..3 run MFMA chains, waves 4..7 return at once; mode 1: waves 4..7
// run FMA chains, waves 0..3 return; mode 2: both at once.  If the matrix
// cores and the vector ALU of a SIMD serve two waves at the same time, mode
// 2 takes about as long as the slower of modes 0 and 1.
__global__ __launch_bounds__(512) void mix_kernel(float *out, int mfma_iters, int fma_iters, int mode)
{
    const int wave = threadIdx.x >> 6;
    float acc = 0.0f;
    if (wave < 4 && mode != 1) {
        bf16x8 a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[e] = (__bf16)(0.001f * (float)(threadIdx.x + e));
            b[e] = (__bf16)(0.002f * (float)(threadIdx.x - e));
        }
        f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
        for (int i = 0; i < mfma_iters; ++i) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) acc += c0[e] + c1[e] + c2[e] + c3[e];
    } else if (wave >= 4 && mode != 0) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = 1.0001f * (float)(threadIdx.x + j);
        for (int i = 0; i < fma_iters; ++i) {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = __builtin_fmaf(v[j], 1.0001f, 0.5f);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) acc += v[j];
    }
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// Same-wave interleaving: 4-wave workgroups (one wave per SIMD when one
// workgroup runs per CU); each round issues 4 independent
// v_mfma_f32_32x32x16_bf16 (mode 0 and 2) and 8 independent chains of FPM
// FMAs (mode 1 and 2), scheduled as one MFMA followed by 2 FPM FMAs, four
// times.  If a wave's vector ALU work issues while its own MFMAs execute,
// mode 2 takes about as long as the slower of modes 0 and 1.
template <int MODE, int FPM>
__global__ __launch_bounds__(256) void interleave_kernel(float *out, int iters)
{
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(0.001f * (float)(threadIdx.x + e));
        b[e] = (__bf16)(0.002f * (float)(threadIdx.x - e));
    }
    f32x16 c[4] = {};
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 1.0001f * (float)(threadIdx.x + j);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (MODE != 1) c[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[q], 0, 0, 0);
            if (MODE != 0) {
#pragma unroll
                for (int f = 0; f < FPM / 4; ++f) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) v[j] = __builtin_fmaf(v[j], 1.0001f, 0.5f);
                }
            }
            if (MODE == 2) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 2 * FPM, 0);  // then 2 FPM VALU
            }
        }
    }
    float acc = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc += c[q][e];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += v[j];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}
template <int FPM>
void launch_interleave(int mode, dim3 g, float *out, int iters, hipStream_t s)
{
    if (mode == 0) interleave_kernel<0, FPM><<<g, dim3(256), 0, s>>>(out, iters);
    else if (mode == 1) interleave_kernel<1, FPM><<<g, dim3(256), 0, s>>>(out, iters);
    else interleave_kernel<2, FPM><<<g, dim3(256), 0, s>>>(out, iters);
}
// grid-stride copy of n 16-byte pieces
__global__ __launch_bounds__(256) void copy_kernel(const u32x4 *src, u32x4 *dst, size_t n)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t k = (size_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += stride) dst[k] = src[k];
}

}  // namespace

// kind: 0 fma, 1 exp2, 2 rcp, 3 sqrt, 4 exp2/fma alternating.  out holds
// blocks * 256 floats.  Returns a hipError_t value.
extern "C" int rglru_micro_valu(int kind, int blocks, int iters, float *out, hipStream_t s)
{
    if (kind < 0 || kind > 4 || blocks < 1 || iters < 1 || !out) return (int)hipErrorInvalidValue;
    const dim3 g((unsigned)blocks), b(256);
    if (kind == 0) valu_kernel<0><<<g, b, 0, s>>>(out, iters, 1.0001f);
    else if (kind == 1) valu_kernel<1><<<g, b, 0, s>>>(out, iters, 1.0001f);
    else if (kind == 2) valu_kernel<2><<<g, b, 0, s>>>(out, iters, 1.0001f);
    else if (kind == 3) valu_kernel<3><<<g, b, 0, s>>>(out, iters, 1.0001f);
    else valu_kernel<4><<<g, b, 0, s>>>(out, iters, 1.0001f);
    return (int)hipGetLastError();
}

// 4 * iters MFMAs of 32768 flops per wave; out holds blocks * 256 floats
extern "C" int rglru_micro_mfma(int blocks, int iters, float *out, hipStream_t s)
{
    if (blocks < 1 || iters < 1 || !out) return (int)hipErrorInvalidValue;
    mfma_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(out, iters);
    return (int)hipGetLastError();
}

// mode 0 MFMA waves only, 1 FMA waves only, 2 both; out holds blocks * 512 floats
extern "C" int rglru_micro_mix(int mode, int blocks, int mfma_iters, int fma_iters, float *out, hipStream_t s)
{
    if (mode < 0 || mode > 2 || blocks < 1 || mfma_iters < 1 || fma_iters < 1 || !out)
        return (int)hipErrorInvalidValue;
    mix_kernel<<<dim3((unsigned)blocks), dim3(512), 0, s>>>(out, mfma_iters, fma_iters, mode);
    return (int)hipGetLastError();
}

// mode 0 MFMA only, 1 FMA only, 2 both in one wave; 8 fpm FMAs per round of
// 4 MFMAs, fpm in {4, 8, 16}; out holds blocks * 256 floats
extern "C" int rglru_micro_interleave(int mode, int blocks, int iters, int fpm, float *out, hipStream_t s)
{
    if (mode < 0 || mode > 2 || blocks < 1 || iters < 1 || !out || (fpm != 4 && fpm != 8 && fpm != 16))
        return (int)hipErrorInvalidValue;
    const dim3 g((unsigned)blocks);
    if (fpm == 4) launch_interleave<4>(mode, g, out, iters, s);
    else if (fpm == 8) launch_interleave<8>(mode, g, out, iters, s);
    else launch_interleave<16>(mode, g, out, iters, s);
    return (int)hipGetLastError();
}
// copies `bytes` (a multiple of 16; both pointers 16-byte aligned)
extern "C" int rglru_micro_copy(const void *src, void *dst, size_t bytes, int blocks, hipStream_t s)
{
    if (!src || !dst || bytes % 16 || ((uintptr_t)src | (uintptr_t)dst) % 16 || blocks < 1)
        return (int)hipErrorInvalidValue;
    copy_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>((const u32x4 *)src, (u32x4 *)dst, bytes / 16);
    return (int)hipGetLastError();
}
