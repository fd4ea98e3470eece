// embed.hip -- multi-stream expansion gather ("Hidden Decoding at Scale",
// "Multi-Stream Expansion and Training Objective": S_t = E_k(x_i) at expanded
// position t = (i-1)n + k, here 0-based t = i*n + s).
//
// A pure HBM stream: every output row is a byte copy of one table row.  One
// wavefront copies one row with 16-byte lane accesses (a 14 KB bf16 row of
// dim 7168 is 14 fully coalesced 1 KB wave transactions); a workgroup of four
// waves handles four rows at a time and strides over the grid.
#include "hd_internal.h"

namespace hd {

namespace {

constexpr int kWaves = 4;

__global__ __launch_bounds__(256) void expand_embed_v16(EmbedArgs a, int64_t nrows) {
    const int lane = threadIdx.x & 63;
    const int64_t wave0 = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int64_t nvec = a.row_bytes >> 4;
    const int Ln = a.L * a.n;
    for (int64_t r = wave0; r < nrows; r += (int64_t)gridDim.x * kWaves) {
        const int b = (int)(r / Ln);
        const int rem = (int)(r - (int64_t)b * Ln);
        const int i = rem / a.n, s = rem - i * a.n;
        const int64_t id = a.ids[(int64_t)b * a.L + i];
        const u32x4 *src = reinterpret_cast<const u32x4 *>(a.tables[s] + id * a.row_bytes);
        u32x4 *dst = reinterpret_cast<u32x4 *>(a.out + r * a.row_bytes);
        int64_t c = lane;
        // Four independent 16-byte loads in flight per lane before the stores.
        for (; c + 192 < nvec; c += 256) {
            u32x4 x0 = __builtin_nontemporal_load(src + c);
            u32x4 x1 = __builtin_nontemporal_load(src + c + 64);
            u32x4 x2 = __builtin_nontemporal_load(src + c + 128);
            u32x4 x3 = __builtin_nontemporal_load(src + c + 192);
            dst[c] = x0; dst[c + 64] = x1; dst[c + 128] = x2; dst[c + 192] = x3;
        }
        for (; c < nvec; c += 64) dst[c] = __builtin_nontemporal_load(src + c);
    }
}

// Fallback for rows whose size is not a multiple of 16 bytes: 2-byte units
// (every supported dtype is 2 or 4 bytes wide).
__global__ __launch_bounds__(256) void expand_embed_u16(EmbedArgs a, int64_t nrows) {
    const int lane = threadIdx.x & 63;
    const int64_t wave0 = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int64_t nunit = a.row_bytes >> 1;
    const int Ln = a.L * a.n;
    for (int64_t r = wave0; r < nrows; r += (int64_t)gridDim.x * kWaves) {
        const int b = (int)(r / Ln);
        const int rem = (int)(r - (int64_t)b * Ln);
        const int i = rem / a.n, s = rem - i * a.n;
        const int64_t id = a.ids[(int64_t)b * a.L + i];
        const uint16_t *src = reinterpret_cast<const uint16_t *>(a.tables[s] + id * a.row_bytes);
        uint16_t *dst = reinterpret_cast<uint16_t *>(a.out + r * a.row_bytes);
        for (int64_t c = lane; c < nunit; c += 64) dst[c] = src[c];
    }
}

}  // namespace

hipError_t launch_expand_embed(const EmbedArgs &a, hipStream_t st) {
    const int64_t nrows = (int64_t)a.B * a.L * a.n;
    int64_t blocks = (nrows + kWaves - 1) / kWaves;
    if (blocks > 65536) blocks = 65536;
    if (a.row_bytes % 16 == 0)
        hipLaunchKernelGGL(expand_embed_v16, dim3((unsigned)blocks), dim3(256), 0, st, a, nrows);
    else
        hipLaunchKernelGGL(expand_embed_u16, dim3((unsigned)blocks), dim3(256), 0, st, a, nrows);
    return hipGetLastError();
}

}  // namespace hd
