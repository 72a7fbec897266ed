// ceilings.hip -- device ceilings the benchmark divides by, measured on the chip it runs on
// (gfx950). Built into libpisa_ceilings.so, apart from libpisa.so: these kernels are
// measurement probes, not part of the selection.
//
// Each probe keeps every lane issuing one instruction kind back to back, over independent
// dependency chains so that latency is hidden, on a grid that fills every CU:
//   kind 0  v_exp_f32      x <- exp2(-x)      (the negation is a source modifier)
//   kind 1  v_log_f32      x <- log2(|x|)     (the absolute value is a source modifier)
//   kind 2  v_fma_f32      x <- x * a + b
//   kind 3  v_mfma_f32_16x16x32_bf16, four independent accumulators per wavefront
// pisa_ceiling_ops() gives the operations one launch performs (lane operations for the
// VALU kinds, flops for the MFMA kind), so rate = ops / launch time.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kChains = 8;        // independent chains per lane (VALU kinds)
constexpr int kUnroll = 16;       // instructions per chain per loop trip

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int KIND>
__global__ __launch_bounds__(kThreads) void valu_probe(int iters, float seed, float* __restrict__ out) {
    float x[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = seed + 0.001f * (float)(threadIdx.x + c);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
            for (int c = 0; c < kChains; ++c) {
                if constexpr (KIND == 0) x[c] = __builtin_amdgcn_exp2f(-x[c]);
                else if constexpr (KIND == 1) x[c] = __builtin_amdgcn_logf(__builtin_fabsf(x[c]));
                else x[c] = __builtin_fmaf(x[c], 0.999f, 0.0001f);
            }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += x[c];
    out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void mfma_probe(int iters, float seed, float* __restrict__ out) {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(seed + 0.01f * (float)i);
        b[i] = (__bf16)(seed - 0.01f * (float)(threadIdx.x & 7));
    }
    f32x4 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Operations of one launch of `kind` with `iters` loop trips on `grid` workgroups of 256
// threads; -1 for an unknown kind.
double pisa_ceiling_ops(int kind, int iters, int grid) {
    const double lanes = (double)grid * kThreads;
    if (kind >= 0 && kind <= 2) return lanes * iters * kUnroll * kChains;
    if (kind == 3) return (double)grid * (kThreads / 64) * iters * kUnroll * 4 * (16.0 * 16.0 * 32.0 * 2.0);
    return -1.0;
}

// Enqueues one probe launch on `stream`. out: device buffer of grid * 256 floats (each lane
// stores its result there so that nothing is optimised away). Returns 0, or -1 on bad
// arguments or a launch error.
int pisa_ceiling_launch(int kind, int iters, int grid, float* out, void* stream) {
    if (iters < 1 || grid < 1 || !out) return -1;
    hipStream_t s = (hipStream_t)stream;
    const float seed = 0.5f;
    switch (kind) {
        case 0: hipLaunchKernelGGL(valu_probe<0>, dim3(grid), dim3(kThreads), 0, s, iters, seed, out); break;
        case 1: hipLaunchKernelGGL(valu_probe<1>, dim3(grid), dim3(kThreads), 0, s, iters, seed, out); break;
        case 2: hipLaunchKernelGGL(valu_probe<2>, dim3(grid), dim3(kThreads), 0, s, iters, seed, out); break;
        case 3: hipLaunchKernelGGL(mfma_probe, dim3(grid), dim3(kThreads), 0, s, iters, seed, out); break;
        default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
