// sfa_f32.hip -- float32 Stream-Factorized Attention (prefill and decode) on
// the vector ALUs.
//
// The float32 path exists for exactness checks on small problems (float32
// inputs, float32 arithmetic end to end); the matrix-core path in
// sfa_fwd_bf16.hip / sfa_decode_bf16.hip is the production one.  One thread
// owns one query row and streams its visible keys once with an online
// softmax; the key set follows "Hidden Decoding at Scale", "Stream-Factorized
// Attention", Figure 2 (see FwdArgs for the sub-sequence form of both masks).
#include "hd_internal.h"

namespace hd {

namespace {

template <int D>
__global__ __launch_bounds__(64) void sfa_fwd_f32_kernel(FwdArgs p) {
    const int64_t row = (int64_t)blockIdx.x * 64 + threadIdx.x;  // (b, sub, i, h)
    const int64_t nrows = (int64_t)p.B * p.nsub * p.Lq * p.Hq;
    if (row >= nrows) return;
    const int h = (int)(row % p.Hq);
    int64_t r = row / p.Hq;
    const int i = (int)(r % p.Lq); r /= p.Lq;
    const int sub = (int)(r % p.nsub);
    const int b = (int)(r / p.nsub);
    const int kvh = h / (p.Hq / p.Hkv);
    const int64_t kpos0 = (int64_t)b * p.nL + p.kbase + sub;  // key element 0
    const int64_t qrow = (int64_t)b * p.qrows + (int64_t)sub * p.qsub + (int64_t)i * p.qstride;
    const float *qg = static_cast<const float *>(p.q);
    const float *kg = static_cast<const float *>(p.k);
    const float *vg = static_cast<const float *>(p.v);

    float qv[D], acc[D];
    const float *qp = qg + (qrow * p.Hq + h) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) { qv[c] = qp[c]; acc[c] = 0.f; }
    float m = -INFINITY, l = 0.f;
    const int lim = i * p.qmul + p.qadd;  // last visible key element
    if (p.rope) {  // rotate-half at the query's expanded position, angle reduced in double
        const double pos = (double)(p.kbase + sub + (int64_t)lim * p.stride);
#pragma unroll
        for (int c = 0; c < D / 2; ++c) {
            const double turns = pos * p.rope_ft[c];
            float sn, cs;
            sincosf((float)(turns - rint(turns)) * 6.28318530717958647692f, &sn, &cs);
            const float x0 = qv[c], x1 = qv[c + D / 2];
            qv[c] = x0 * cs - x1 * sn;
            qv[c + D / 2] = x1 * cs + x0 * sn;
        }
    }
    const int jbeg = p.weff ? max(0, lim - p.weff + 1) : 0;
    for (int j = jbeg; j <= lim; ++j) {
        const int64_t off = ((kpos0 + (int64_t)j * p.stride) * p.Hkv + kvh) * D;
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) s = fmaf(qv[c], kg[off + c], s);
        s *= p.scale;
        const float mn = fmaxf(m, s);
        const float alpha = expf(m - mn);  // m = -inf on the first key: 0
        const float e = expf(s - mn);
        l = l * alpha + e;
#pragma unroll
        for (int c = 0; c < D; ++c) acc[c] = fmaf(e, vg[off + c], acc[c] * alpha);
        m = mn;
    }
    float *op = static_cast<float *>(p.o) + (qrow * p.Hq + h) * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int c = 0; c < D; ++c) op[c] = acc[c] * inv;
    if (p.lse != nullptr) p.lse[((int64_t)b * p.Hq + h) * p.qrows + (qrow - (int64_t)b * p.qrows)] = m + logf(l);
}

// Decode: one thread per (b, s, h) query; also appends the new rows.
template <int D>
__global__ __launch_bounds__(64) void sfa_decode_f32_kernel(DecArgs p) {
    const int64_t row = (int64_t)blockIdx.x * 64 + threadIdx.x;  // (b, query stream, h)
    const int64_t nrows = (int64_t)p.B * p.nqs * p.Hq;
    if (row >= nrows) return;
    const int h = (int)(row % p.Hq);
    const int s = p.qs0 + (int)((row / p.Hq) % p.nqs);
    const int b = (int)(row / p.Hq / p.nqs);
    const int g = p.Hq / p.Hkv, kvh = h / g;
    const int len = p.cache_len[b];
    if (len < 0 || len >= p.T_cap) {  // contract violation: NaN row, nothing read
        float *op = static_cast<float *>(p.o) + row * D;
#pragma unroll
        for (int c = 0; c < D; ++c) reinterpret_cast<unsigned *>(op)[c] = 0x7fc00000u;  // quiet NaN
        return;
    }
    const float *qg = static_cast<const float *>(p.q);
    const float *kn = static_cast<const float *>(p.k_new);
    const float *vn = static_cast<const float *>(p.v_new);
    float *kc = static_cast<float *>(p.k_cache);
    float *vc = static_cast<float *>(p.v_cache);
    const int64_t cache_row = (int64_t)p.n * p.Hkv * D;  // elements per cached token

    float qv[D], acc[D];
    const float *qp = qg + row * D;
#pragma unroll
    for (int c = 0; c < D; ++c) { qv[c] = qp[c]; acc[c] = 0.f; }
    float m = -INFINITY, l = 0.f;
    const int64_t tq = (int64_t)len * p.n + s;
    // Candidate keys: expanded positions t_k <= t_q (both masks are causal).
    const int64_t tlo = p.window ? max((int64_t)0, (int64_t)(len - p.window) * p.n) : 0;
    for (int64_t tk = tlo; tk <= tq; ++tk) {
        const int64_t tok = tk / p.n;
        const int sk = (int)(tk - tok * p.n);
        bool vis;
        if (p.mode == 0) vis = (sk == s) && (p.window == 0 || len - tok < p.window);
        else vis = (p.window == 0 || tq - tk < (int64_t)p.n * p.window);
        if (!vis) continue;
        const float *kr, *vr;
        if (tok < len) {
            const int64_t off = ((int64_t)b * p.T_cap + tok) * cache_row + ((int64_t)sk * p.Hkv + kvh) * D;
            kr = kc + off; vr = vc + off;
        } else {
            const int64_t off = (((int64_t)b * p.n + sk) * p.Hkv + kvh) * D;
            kr = kn + off; vr = vn + off;
        }
        float sc = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) sc = fmaf(qv[c], kr[c], sc);
        sc *= p.scale;
        const float mn = fmaxf(m, sc);
        const float alpha = expf(m - mn);
        const float e = expf(sc - mn);
        l = l * alpha + e;
#pragma unroll
        for (int c = 0; c < D; ++c) acc[c] = fmaf(e, vr[c], acc[c] * alpha);
        m = mn;
    }
    float *op = static_cast<float *>(p.o) + row * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int c = 0; c < D; ++c) op[c] = acc[c] * inv;
}

// Append k_new/v_new at token cache_len[b].  Runs after the attention kernel
// on the same stream, which reads the new rows from k_new/v_new directly.
__global__ __launch_bounds__(256) void append_f32_kernel(DecArgs p) {
    const int64_t per_b = (int64_t)p.n * p.Hkv * p.d;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= per_b * p.B) return;
    const int b = (int)(idx / per_b);
    const int64_t e = idx - (int64_t)b * per_b;
    const int len = p.cache_len[b];
    if (len < 0 || len >= p.T_cap) return;  // contract violation: the cache is left as it is
    const int64_t dst = ((int64_t)b * p.T_cap + len) * per_b + e;
    static_cast<float *>(p.k_cache)[dst] = static_cast<const float *>(p.k_new)[idx];
    static_cast<float *>(p.v_cache)[dst] = static_cast<const float *>(p.v_new)[idx];
}

}  // namespace

hipError_t launch_sfa_fwd_f32(const FwdArgs &a, hipStream_t st) {
    const int64_t nrows = (int64_t)a.B * a.nsub * a.Lq * a.Hq;
    const int64_t grid = (nrows + 63) / 64;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    switch (a.d) {
        case 32: hipLaunchKernelGGL(sfa_fwd_f32_kernel<32>, dim3((unsigned)grid), dim3(64), 0, st, a); break;
        case 64: hipLaunchKernelGGL(sfa_fwd_f32_kernel<64>, dim3((unsigned)grid), dim3(64), 0, st, a); break;
        case 128: hipLaunchKernelGGL(sfa_fwd_f32_kernel<128>, dim3((unsigned)grid), dim3(64), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_sfa_decode_f32(const DecArgs &a, hipStream_t st) {
    const int64_t nrows = (int64_t)a.B * a.nqs * a.Hq;
    const unsigned grid = (unsigned)((nrows + 63) / 64);
    switch (a.d) {
        case 32: hipLaunchKernelGGL(sfa_decode_f32_kernel<32>, dim3(grid), dim3(64), 0, st, a); break;
        case 64: hipLaunchKernelGGL(sfa_decode_f32_kernel<64>, dim3(grid), dim3(64), 0, st, a); break;
        case 128: hipLaunchKernelGGL(sfa_decode_f32_kernel<128>, dim3(grid), dim3(64), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t total = (int64_t)a.B * a.n * a.Hkv * a.d;
    hipLaunchKernelGGL(append_f32_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace hd
