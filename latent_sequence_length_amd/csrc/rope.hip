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

constexpr int kRopeHeads = 4;  // heads per thread

// One thread per (b, t, 8-pair chunk, block of kRopeHeads heads): the eight
// angles of its chunk are computed once and applied to the block's heads;
// all of the block's 16-byte loads (x[c0 .. c0+7] and x[c0+h .. c0+h+7] of
// each head) are issued before any arithmetic, so a wave keeps 8 loads in
// flight per lane.  Consecutive threads take consecutive chunks of one head
// row, then the next row: a wave covers whole 256-byte head rows.
template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(RopeArgs a) {
    constexpr int VE = 16 / sizeof(T);  // elements per 16-byte access
    const int h = a.d / 2, nch = h / 8;  // 8 pairs per chunk
    const int nhb = (a.H + kRopeHeads - 1) / kRopeHeads;
    const unsigned idx = blockIdx.x * 256u + threadIdx.x;  // ((b*T + t)*nhb + hb)*nch + chunk
    if (idx >= (unsigned)a.B * (unsigned)a.T * (unsigned)nhb * (unsigned)nch) return;
    const unsigned rowi = idx / (unsigned)nch;
    const int c0 = (int)(idx - rowi * (unsigned)nch) * 8;
    const unsigned bt = rowi / (unsigned)nhb;
    const int hb = (int)(rowi - bt * (unsigned)nhb);
    const unsigned b = bt / (unsigned)a.T, t = bt - b * (unsigned)a.T;
    const int64_t pos = (int64_t)t * a.t_mul + a.t_add + (a.pos_base != nullptr ? a.pos_mul * (int64_t)a.pos_base[b] : 0);
    const int h0 = hb * kRopeHeads, nh = min(kRopeHeads, a.H - h0);
    const T *xrow = static_cast<const T *>(a.x) + ((int64_t)bt * a.H + h0) * a.d;
    T *orow = static_cast<T *>(a.out) + ((int64_t)bt * a.H + h0) * a.d;
    double fr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) fr[j] = a.freq_turns[c0 + j];
    // Loads of heads past the end of the row re-read its last head (stores
    // are skipped for them): no branch around the loads, all in flight at once.
    uint4 x0[kRopeHeads][8 / VE], x1[kRopeHeads][8 / VE];
#pragma unroll
    for (int k = 0; k < kRopeHeads; ++k) {
        const T *xp = xrow + min(k, nh - 1) * a.d;
#pragma unroll
        for (int u = 0; u < 8 / VE; ++u) {
            x0[k][u] = *reinterpret_cast<const uint4 *>(xp + c0 + u * VE);
            x1[k][u] = *reinterpret_cast<const uint4 *>(xp + c0 + h + u * VE);
        }
    }
    float cs[8], sn[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        // angle in turns: pos * f_c / (2 pi), reduced to [-1/2, 1/2) in double
        const double turns = (double)pos * fr[j];
        const float red = (float)(turns - rint(turns));
        sincosf(red * 6.28318530717958647692f, &sn[j], &cs[j]);
    }
#pragma unroll
    for (int k = 0; k < kRopeHeads; ++k) {
        if (k < nh) {
            T v0[8], v1[8], y0[8], y1[8];
#pragma unroll
            for (int u = 0; u < 8 / VE; ++u) {
                *reinterpret_cast<uint4 *>(&v0[u * VE]) = x0[k][u];
                *reinterpret_cast<uint4 *>(&v1[u * VE]) = x1[k][u];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float a0 = (float)v0[j], a1 = (float)v1[j];
                y0[j] = (T)(a0 * cs[j] - a1 * sn[j]);
                y1[j] = (T)(a1 * cs[j] + a0 * sn[j]);
            }
            T *op = orow + k * a.d;
#pragma unroll
            for (int u = 0; u < 8; u += VE) {
                *reinterpret_cast<uint4 *>(op + c0 + u) = *reinterpret_cast<const uint4 *>(&y0[u]);
                *reinterpret_cast<uint4 *>(op + c0 + h + u) = *reinterpret_cast<const uint4 *>(&y1[u]);
            }
        }
    }
}

}  // namespace

hipError_t launch_rope(const RopeArgs &a, bool bf16_data, hipStream_t st) {
    const int64_t work = (int64_t)a.B * a.T * ((a.H + kRopeHeads - 1) / kRopeHeads) * (a.d / 16);
    if (work >= ((int64_t)1 << 32)) return hipErrorInvalidConfiguration;
    const int64_t grid = (work + 255) / 256;
    if (bf16_data) hipLaunchKernelGGL(rope_kernel<bf16>, dim3((unsigned)grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL(rope_kernel<float>, dim3((unsigned)grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace hd
