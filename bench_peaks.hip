// bench_peaks.hip -- the machine's sustained rates, measured by bench.py and
// reported next to MI355X's published peaks (measurement only; not part of
// the attention library).
//
//   hd_probe_mfma_bf16  every wave runs `iters` rounds of 8 independent
//                       v_mfma_f32_32x32x16_bf16 accumulator chains on
//                       register operands: no memory traffic and no LDS, so
//                       its rate is the sustained bf16 matrix-core rate at the
//                       clock the chip holds under that load.  The operands
//                       are small constants, the lowest-power case.
//   hd_probe_mfma_bf16_random  the same chains on random bf16 operands that
//                       change from one MFMA to the next (8 A and 8 B
//                       fragments per lane, loaded once, B rotating over the
//                       chains): the matrix-core rate with the switching
//                       activity of real data, at the clock the chip holds
//                       under that power.
//   hd_probe_hbm_read   a read-only stream over a large buffer: 16-byte
//                       non-temporal loads, eight in flight per lane, folded
//                       into one register (XOR) per lane; nothing is written
//                       unless the fold hits a value it cannot reach with the
//                       buffer bench.py fills.  The buffer is far larger than
//                       the 256 MB last-level cache, so its rate is the HBM
//                       read ceiling a read-dominated kernel (decode) can
//                       approach.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

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

__global__ __launch_bounds__(256) void mfma_random_kernel(int rounds, const bf16x8_t *ops, int64_t nops,
                                                          float *sink) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    bf16x8_t a[8], b[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        a[c] = ops[(gid * 16 + c) % nops];
        b[c] = ops[(gid * 16 + 8 + c) % nops];
    }
    f32x16_t acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x16_t{};
    for (int i = 0; i < rounds; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int c = 0; c < 8; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[(c + j) & 7], acc[c], 0, 0, 0);
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    if (s == -1.f) sink[blockIdx.x * 256 + threadIdx.x] = s;  // (almost) never true; keeps the work alive
}

constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4_t *src, int64_t nvec, unsigned *sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; v + (kReadUnroll - 1) * stride < nvec; v += kReadUnroll * stride) {
        u32x4_t x[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) x[u] = __builtin_nontemporal_load(src + v + u * stride);
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= x[u];
    }
    for (; v < nvec; v += stride) acc ^= __builtin_nontemporal_load(src + v);
    const unsigned f = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (f == 0x9e3779b9u) sink[blockIdx.x * 256 + threadIdx.x] = f;  // unreachable for a constant fill
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

// Random-operand variant: `rounds` rounds of 64 MFMAs per wave on operands
// taken from the nops bf16x8 fragments at `ops` (device memory); returns the
// FLOP count or -1 on a bad argument or launch error.
double hd_probe_mfma_bf16_random(int blocks, int rounds, const void *ops, int64_t nops, float *sink,
                                 void *stream) {
    if (blocks < 1 || rounds < 1 || ops == nullptr || nops < 16 || sink == nullptr ||
        (reinterpret_cast<uintptr_t>(ops) & 15))
        return -1.0;
    hipLaunchKernelGGL(mfma_random_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), rounds,
                       static_cast<const bf16x8_t *>(ops), nops, sink);
    if (hipGetLastError() != hipSuccess) return -1.0;
    return (double)blocks * 4 * rounds * 64 * (2.0 * 32 * 32 * 16);
}

// Read nbytes (a multiple of 16) from the 16-byte aligned device buffer src
// with `blocks` workgroups of 256 lanes; returns the bytes read or -1 on a bad
// argument or launch error.  `sink` must hold blocks*256 unsigned ints (never
// written while the buffer holds a constant byte fill).
double hd_probe_hbm_read(const void *src, int64_t nbytes, int blocks, unsigned *sink, void *stream) {
    if (src == nullptr || sink == nullptr || blocks < 1 || nbytes < 16 || (nbytes & 15) ||
        (reinterpret_cast<uintptr_t>(src) & 15))
        return -1.0;
    hipLaunchKernelGGL(hbm_read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4_t *>(src), nbytes / 16, sink);
    if (hipGetLastError() != hipSuccess) return -1.0;
    return (double)nbytes;
}

}  // extern "C"
