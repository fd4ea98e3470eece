// rope.hip -- rotary position embedding at the expanded positions.
//
// "Hidden Decoding at Scale", "Multi-Stream Expansion and Training Objective":
// the expanded sequence is fed to the Transformer with contiguous RoPE
// positions, so S_t (token i, stream s, t = i*n + s) is rotated by position t,
// not by its token index.  Rotate-half form: with h = d/2 and frequency
// f_c = theta^(-2c/d),
//   out[c]     = x[c] cos(p f_c) - x[c+h] sin(p f_c)
//   out[c + h] = x[c+h] cos(p f_c) + x[c] sin(p f_c)
// HBM-bound: each (position, frequency) angle is computed once for all heads
// of the row.  The angle is reduced in double precision (p f_c reaches ~1e5
// radians at 131072 positions) before a float sine / cosine.
#include "hd_internal.h"

namespace hd {

namespace {

// One thread per (b, t, 8-pair chunk): the eight angles of its chunk are
// computed once and applied to every head of the row (16-byte loads/stores of
// x[c0 .. c0+7] and x[c0+h .. c0+h+7]).
template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(RopeArgs a) {
    constexpr int VE = 16 / sizeof(T);  // elements per 16-byte access
    const int h = a.d / 2, nch = h / 8;  // 8 pairs per chunk
    const unsigned idx = blockIdx.x * 256u + threadIdx.x;  // (b*T + t)*nch + chunk
    if (idx >= (unsigned)a.B * (unsigned)a.T * (unsigned)nch) return;
    const unsigned bt = idx / (unsigned)nch;
    const int c0 = (int)(idx - bt * (unsigned)nch) * 8;
    const unsigned b = bt / (unsigned)a.T, t = bt - b * (unsigned)a.T;
    const int64_t pos = (int64_t)t * a.t_mul + a.t_add + (a.pos_base != nullptr ? a.pos_mul * (int64_t)a.pos_base[b] : 0);
    float cs[8], sn[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        // angle in turns: pos * f_c / (2 pi), reduced to [-1/2, 1/2) in double
        const double turns = (double)pos * a.freq_turns[c0 + j];
        const float red = (float)(turns - rint(turns));
        sincosf(red * 6.28318530717958647692f, &sn[j], &cs[j]);
    }
    const T *xrow = static_cast<const T *>(a.x) + (int64_t)bt * a.H * a.d;
    T *orow = static_cast<T *>(a.out) + (int64_t)bt * a.H * a.d;
    for (int hh = 0; hh < a.H; ++hh) {
        const T *xp = xrow + hh * a.d;
        T *op = orow + hh * a.d;
        T x0[8], x1[8];
#pragma unroll
        for (int u = 0; u < 8; u += VE) {
            *reinterpret_cast<uint4 *>(&x0[u]) = *reinterpret_cast<const uint4 *>(xp + c0 + u);
            *reinterpret_cast<uint4 *>(&x1[u]) = *reinterpret_cast<const uint4 *>(xp + c0 + h + u);
        }
        T y0[8], y1[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float a0 = (float)x0[j], a1 = (float)x1[j];
            y0[j] = (T)(a0 * cs[j] - a1 * sn[j]);
            y1[j] = (T)(a1 * cs[j] + a0 * sn[j]);
        }
#pragma unroll
        for (int u = 0; u < 8; u += VE) {
            *reinterpret_cast<uint4 *>(op + c0 + u) = *reinterpret_cast<const uint4 *>(&y0[u]);
            *reinterpret_cast<uint4 *>(op + c0 + h + u) = *reinterpret_cast<const uint4 *>(&y1[u]);
        }
    }
}

}  // namespace

hipError_t launch_rope(const RopeArgs &a, bool bf16_data, hipStream_t st) {
    const int64_t work = (int64_t)a.B * a.T * (a.d / 16);
    if (work >= ((int64_t)1 << 32)) return hipErrorInvalidConfiguration;
    const int64_t grid = (work + 255) / 256;
    if (bf16_data) hipLaunchKernelGGL(rope_kernel<bf16>, dim3((unsigned)grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL(rope_kernel<float>, dim3((unsigned)grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace hd
