// peak.hip -- measured matrix-core peak of the machine, for the roofline
// report next to the published figure (not part of the attention library).
//
// Every wave runs `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16
// accumulator chains on register operands: no memory traffic, no LDS, so the
// rate it reaches is the sustained bf16 matrix-core rate at the clocks the
// chip holds under that load.
#include <hip/hip_runtime.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float *sink) {
    bf16x8_t a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(float)((threadIdx.x + e) & 7);
        b[e] = (__bf16)(float)((threadIdx.x * 3 + e) & 7);
    }
    f32x16_t acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x16_t{};
    for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    if (s == -1.f) sink[blockIdx.x * 256 + threadIdx.x] = s;  // never true; keeps the work alive
}

extern "C" {

// Launch `blocks` workgroups of 4 waves; returns the kernel's FLOP count
// (2*32*32*16 per MFMA) or -1 on a launch error.  `sink` must hold
// blocks*256 floats (never written in practice).
double hd_probe_mfma_bf16(int blocks, int iters, float *sink, void *stream) {
    if (blocks < 1 || iters < 1 || sink == nullptr) return -1.0;
    hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters, sink);
    if (hipGetLastError() != hipSuccess) return -1.0;
    return (double)blocks * 4 * iters * 8 * (2.0 * 32 * 32 * 16);
}

}  // extern "C"
