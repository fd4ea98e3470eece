// sfa_bwd.hip -- backward of Stream-Factorized Attention prefill: dQ, dK, dV
// of the scalar sum(dO * O), for bf16 (matrix cores, fp32 accumulation) and
// float32 (vector ALUs, exactness checks).
//
// The pages define the forward ("Hidden Decoding at Scale", "Stream-Factorized
// Attention", Figure 2 masks); training through it needs the derivative of
// that forward, which is the standard one of masked softmax attention.  For a
// query row i with visible keys j, P_ij = exp(scale q_i.k_j - lse_i) (lse from
// the forward) and D_i = dO_i . O_i:
//   dP_ij = dO_i . v_j,   dS_ij = P_ij (dP_ij - D_i)
//   dQ_i  = scale sum_j dS_ij k_j
//   dK_j  = scale sum_i dS_ij q_i,   dV_j = sum_i P_ij dO_i
// where the sums over i run over the query heads of the kv head's GQA group.
// Both masks use the strided sub-sequence form of FwdArgs: intra-stream
// attention is n independent causal attentions on the streams, cross-stream
// one causal attention over all positions.
//
// Three launches, no atomics, every output element written once:
//   1. D_i = dO_i . O_i for every query row (fp32, into the workspace);
//   2. dK, dV: a workgroup owns 256 keys of one (batch, kv head, sub-sequence)
//      and walks the query tiles (all heads of the group) that see them, the
//      tiles of up to four heads per round (d = 128: copied direct to LDS and
//      double-buffered; d = 32/64: staged through registers).  When the layer
//      has too few key blocks to fill the chip (the causal triangle then
//      leaves the first blocks with most of the work), the query range is cut
//      into segments, each workgroup writes fp32 partial sums for one segment
//      and a reduction kernel adds the segments in a fixed order;
//   3. dQ: a wave owns 32 queries of one head and walks the key tiles they see
//      (the forward's loop, recomputing P from lse); d = 128 shares 64-key
//      tiles copied direct to LDS among 8 waves, d = 32/64 stages 128 keys per
//      barrier through registers.
#include <algorithm>

#include "attn_common.h"

namespace hd {

namespace {

constexpr int BKT = 64;   // keys per tile (dQ kernel)
constexpr int BQT = 32;   // queries per tile (dK/dV kernel)
constexpr int BKW = 256;  // keys per workgroup (dK/dV kernel)

// ---------------------------------------------------------------------------
// 1. D = dO . O per query row; 16 lanes per row, fp32.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_drow_kernel(BwdArgs p) {
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);  // (b*qrows + t)*Hq + h
    const int part = threadIdx.x & 15;
    const int64_t nrows = (int64_t)p.B * p.qrows * p.Hq;
    constexpr int PER = D / 16;
    float acc = 0.f;
    if (row < nrows) {
        const T *o = static_cast<const T *>(p.o) + row * D + part * PER;
        const T *g = static_cast<const T *>(p.dout) + row * D + part * PER;
#pragma unroll
        for (int c = 0; c < PER; ++c) acc = fmaf((float)o[c], (float)g[c], acc);
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 16);
    if (row < nrows && part == 0) {
        const int64_t h = row % p.Hq, t = (row / p.Hq) % p.qrows, b = row / p.Hq / p.qrows;
        p.drow[(b * p.Hq + h) * p.qrows + t] = acc;
    }
}

// Key element j of sub-sequence (b, sub) -> K/V row (expanded position).
__device__ __forceinline__ int64_t sub_pos(const BwdArgs &p, int b, int sub, int j) {
    return (int64_t)b * p.nL + p.kbase + sub + (int64_t)j * p.stride;
}

// Query i of sub-sequence (b, sub) -> Q / O / dO row.
__device__ __forceinline__ int64_t q_row(const BwdArgs &p, int b, int sub, int i) {
    return (int64_t)b * p.qrows + (int64_t)sub * p.qsub + (int64_t)i * p.qstride;
}

// Index of a query row's lse / D entry: [b][h][row within the batch row].
__device__ __forceinline__ int64_t row_stat(const BwdArgs &p, int b, int h, int64_t qrow) {
    return ((int64_t)b * p.Hq + h) * p.qrows + (qrow - (int64_t)b * p.qrows);
}

// First query whose band reaches key element j (lim(i) >= j), or 0.
__device__ __forceinline__ int first_query(const BwdArgs &p, int j) {
    return j <= p.qadd ? 0 : (j - p.qadd + p.qmul - 1) / p.qmul;
}

// One past the last query whose window still holds key element j (Lq without a window).
__device__ __forceinline__ int query_end(const BwdArgs &p, int j) {
    if (p.weff == 0) return p.Lq;
    const int num = j + p.weff - 1 - p.qadd;  // lim(i) <= num
    return num < 0 ? 0 : min(p.Lq, num / p.qmul + 1);
}

// ---------------------------------------------------------------------------
// float32: one thread per query row (dQ) or per key row (dK, dV).
template <int D>
__global__ __launch_bounds__(64) void bwd_dq_f32_kernel(BwdArgs p) {
    const int64_t row = (int64_t)blockIdx.x * 64 + threadIdx.x;  // (b, sub, i, h)
    const int64_t nrows = (int64_t)p.B * p.nsub * p.Lq * p.Hq;
    if (row >= nrows) return;
    const int h = (int)(row % p.Hq);
    int64_t r = row / p.Hq;
    const int i = (int)(r % p.Lq); r /= p.Lq;
    const int sub = (int)(r % p.nsub);
    const int b = (int)(r / p.nsub);
    const int kvh = h / (p.Hq / p.Hkv);
    const int64_t pos = q_row(p, b, sub, i);
    const float *qp = static_cast<const float *>(p.q) + (pos * p.Hq + h) * D;
    const float *gp = static_cast<const float *>(p.dout) + (pos * p.Hq + h) * D;
    const float *kg = static_cast<const float *>(p.k);
    const float *vg = static_cast<const float *>(p.v);
    float qv[D], gv[D], acc[D];
#pragma unroll
    for (int c = 0; c < D; ++c) { qv[c] = qp[c]; gv[c] = gp[c]; acc[c] = 0.f; }
    const float lse = p.lse[row_stat(p, b, h, pos)], Dr = p.drow[row_stat(p, b, h, pos)];
    const int lim = i * p.qmul + p.qadd;  // last visible key element
    const int jbeg = p.weff ? max(0, lim - p.weff + 1) : 0;
    for (int j = jbeg; j <= lim; ++j) {
        const int64_t off = (sub_pos(p, b, sub, j) * p.Hkv + kvh) * D;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) {
            s = fmaf(qv[c], kg[off + c], s);
            dp = fmaf(gv[c], vg[off + c], dp);
        }
        const float ds = expf(s * p.scale - lse) * (dp - Dr);
#pragma unroll
        for (int c = 0; c < D; ++c) acc[c] = fmaf(ds, kg[off + c], acc[c]);
    }
    float *out = static_cast<float *>(p.dq) + (pos * p.Hq + h) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) out[c] = p.scale * acc[c];
}

template <int D>
__global__ __launch_bounds__(64) void bwd_dkdv_f32_kernel(BwdArgs p) {
    __shared__ float ks[64][D + 1], vs[64][D + 1];  // this thread's key / value row
    const int64_t row = (int64_t)blockIdx.x * 64 + threadIdx.x;  // (b, sub, j, kvh)
    const int64_t nrows = (int64_t)p.B * p.nsub * p.Lsub * p.Hkv;
    if (row >= nrows) return;
    const int kvh = (int)(row % p.Hkv);
    int64_t r = row / p.Hkv;
    const int j = (int)(r % p.Lsub); r /= p.Lsub;
    const int sub = (int)(r % p.nsub);
    const int b = (int)(r / p.nsub);
    const int g = p.Hq / p.Hkv;
    const int64_t kpos = sub_pos(p, b, sub, j);
    const float *kr = static_cast<const float *>(p.k) + (kpos * p.Hkv + kvh) * D;
    const float *vr = static_cast<const float *>(p.v) + (kpos * p.Hkv + kvh) * D;
    float *myk = ks[threadIdx.x], *myv = vs[threadIdx.x];
    for (int c = 0; c < D; ++c) { myk[c] = kr[c]; myv[c] = vr[c]; }
    float ak[D], av[D];
#pragma unroll
    for (int c = 0; c < D; ++c) ak[c] = av[c] = 0.f;
    const int ibeg = first_query(p, j), iend = query_end(p, j);
    for (int hh = 0; hh < g; ++hh) {
        const int h = kvh * g + hh;
        for (int i = ibeg; i < iend; ++i) {
            const int64_t qpos = q_row(p, b, sub, i);
            const float *qp = static_cast<const float *>(p.q) + (qpos * p.Hq + h) * D;
            const float *gp = static_cast<const float *>(p.dout) + (qpos * p.Hq + h) * D;
            float s = 0.f, dp = 0.f;
            for (int c = 0; c < D; ++c) {
                s = fmaf(qp[c], myk[c], s);
                dp = fmaf(gp[c], myv[c], dp);
            }
            const float pr = expf(s * p.scale - p.lse[row_stat(p, b, h, qpos)]);
            const float ds = pr * (dp - p.drow[row_stat(p, b, h, qpos)]);
#pragma unroll
            for (int c = 0; c < D; ++c) {
                ak[c] = fmaf(ds, qp[c], ak[c]);
                av[c] = fmaf(pr, gp[c], av[c]);
            }
        }
    }
    float *dk = static_cast<float *>(p.dk) + (kpos * p.Hkv + kvh) * D;
    float *dv = static_cast<float *>(p.dv) + (kpos * p.Hkv + kvh) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) {
        dk[c] = p.scale * ak[c];
        dv[c] = av[c];
    }
}

// ---------------------------------------------------------------------------
// bf16 kernels on v_mfma_f32_32x32x16_bf16 (operand layouts as in the forward:
// lane l supplies row l % 32 of A / column l % 32 of B with k-slots
// 8*(l/32) .. +7; register r of the accumulator holds C[8*(r/4) + 4*(l/32) +
// r%4][l % 32]).  LDS tiles are row-major with a 16-byte pad per row.  A
// transposed operand (a 32-row block of a tile read down its columns) comes
// from two ds_read_b64_tr_b16: within a 16-lane group that instruction gives
// lane i element e of the 8 bytes read by lane 4e + i/4, so lane j of the
// group addresses row r0 + j/4, columns c0 + 4*(j%4); the result holds
// column c0 + (lane % 16) of rows r0 .. r0+3.

template <int D>
__device__ __forceinline__ bf16x8 read_rows_tr(const char *tile, int row0, int col0, int hi, int l16, int g2) {
    constexpr int PITCH = 2 * D + 16;
    s16x4 h2[2];
#pragma unroll
    for (int jh = 0; jh < 2; ++jh) {
        const int row = row0 + 8 * jh + 4 * hi + (l16 >> 2);
        const int col = col0 + 16 * g2 + 4 * (l16 & 3);
        h2[jh] = lds_read_tr16(tile + row * PITCH + col * 2);
    }
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(h2[0], h2[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// Copy `rows` rows of D bf16 (global row stride `rstride` elements, first row
// `base`) into a padded LDS tile; rows at or past `nvalid` are zero.
template <int D, int ROWS, int NT = 256>
__device__ __forceinline__ void stage_rows(char *tile, const bf16 *base, int64_t rstride, int nvalid) {
    constexpr int CH = D / 8, PITCH = 2 * D + 16, PER = (ROWS * CH + NT - 1) / NT;
    uint4 x[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {  // all loads first, then all stores
        const int c = threadIdx.x + NT * u, r = c / CH, cc = c - r * CH;
        x[u] = uint4{0, 0, 0, 0};
        if (c < ROWS * CH && r < nvalid) x[u] = *reinterpret_cast<const uint4 *>(base + r * rstride + cc * 8);
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int c = threadIdx.x + NT * u, r = c / CH, cc = c - r * CH;
        if (c < ROWS * CH) *reinterpret_cast<uint4 *>(tile + r * PITCH + cc * 16) = x[u];
    }
}

// Store a [D dims x 32] accumulator block set (lane = row l % 32 of the
// output, registers = dims) as bf16, times `mul`.
template <int D>
__device__ __forceinline__ void store_rows(bf16 *out, const f32x16 (&acc)[D / 32], float mul, int hi) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            bf16x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = (bf16)(acc[db][4 * r4 + e] * mul);
            *reinterpret_cast<bf16x4 *>(out + db * 32 + 8 * r4 + 4 * hi) = y;
        }
}

// 2. dK, dV.  Workgroup = 8 waves x 32 keys of one (b, kv head, sub), two
// waves per SIMD and one workgroup per CU, so every staged query tile serves
// 256 keys (half the L2-to-LDS traffic of a 4-wave group); per query tile
// (32 queries of one head of the group):
//   S = Q K^T, dP = dO V^T      [32 q x 32 k]: lane = key, registers = queries
//   P = exp(S*scale - lse), dS = P (dP - D)
//   dV^T += dO^T P, dK^T += Q^T dS   [D x 32 k]
// GQ: the query map is not the identity (final-stream queries).
template <int D, bool GQ>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_bf16_kernel(BwdArgs p, int nseg, int segq) {
    constexpr int PITCH = 2 * D + 16;
    constexpr int HS = 4;  // heads of the group staged per round
    __shared__ __attribute__((aligned(16))) char Qs[HS][BQT * PITCH];
    __shared__ __attribute__((aligned(16))) char Gs[HS][BQT * PITCH];
    __shared__ __attribute__((aligned(16))) float Ls[HS][BQT], Ds[HS][BQT];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5, l16 = lane & 15, g2 = (lane >> 4) & 1;
    const int g = p.Hq / p.Hkv;

    // workgroup -> (key block, query segment, b, kv head, sub); the low key
    // blocks of every group (they see the most queries) are dispatched first
    const int ngroups = p.B * p.Hkv * p.nsub;
    const int kseg = (int)(blockIdx.x / ngroups);
    const int kblk = kseg / nseg, seg = kseg % nseg;
    int rest = (int)(blockIdx.x % ngroups);
    const int sub = rest % p.nsub; rest /= p.nsub;
    const int kvh = rest % p.Hkv;
    const int b = rest / p.Hkv;
    const int j0 = kblk * BKW;
    const int jw0 = j0 + 32 * wave;  // this wave's first key
    const int myk = jw0 + l32;
    const bool kvalid = myk < p.Lsub;

    const int64_t qrs = (int64_t)p.Hq * D, krs = (int64_t)p.Hkv * D;
    const int64_t kpos = sub_pos(p, b, sub, kvalid ? myk : 0);
    // B operands K^T and V^T: lane = key, k-slots = dims 16*ks + 8*hi .. +7
    bf16x8 kf[D / 16], vf[D / 16];
    {
        const bf16 *kr = static_cast<const bf16 *>(p.k) + kpos * krs + (int64_t)kvh * D + 8 * hi;
        const bf16 *vr = static_cast<const bf16 *>(p.v) + kpos * krs + (int64_t)kvh * D + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            kf[ks] = kvalid ? *reinterpret_cast<const bf16x8 *>(kr + 16 * ks) : bf16x8{};
            vf[ks] = kvalid ? *reinterpret_cast<const bf16x8 *>(vr + 16 * ks) : bf16x8{};
        }
    }
    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dk[db] = dv[db] = f32x16{};

    const float c2 = p.scale * kLog2e;
    const int qmul = GQ ? p.qmul : 1, qadd = GQ ? p.qadd : 0;
    // queries that see keys [j0, j0 + BKW): lim(i) >= j0 and lim(i) - j < weff,
    // within this workgroup's segment [seg*segq, qend)
    const int qend = nseg > 1 ? min(p.Lq, (seg + 1) * segq) : p.Lq;
    const int ibeg = max(first_query(p, j0), seg * segq);
    const int iend = min(query_end(p, min(j0 + BKW, p.Lsub) - 1), qend);
    if (nseg > 1 && ibeg >= iend) return;  // empty segment: the reduction skips it
    for (int h0 = 0; h0 < g; h0 += HS) {
        const int nh = min(HS, g - h0);
        for (int i0 = ibeg; i0 < iend; i0 += BQT) {
            __syncthreads();  // previous tiles consumed
            const int nvalid = min(BQT, qend - i0);
            const int64_t qpos0 = q_row(p, b, sub, i0);
            for (int hh = 0; hh < nh; ++hh) {
                const int h = kvh * g + h0 + hh;
                stage_rows<D, BQT, 512>(Qs[hh], static_cast<const bf16 *>(p.q) + qpos0 * qrs + (int64_t)h * D,
                                   p.qstride * qrs, nvalid);
                stage_rows<D, BQT, 512>(Gs[hh], static_cast<const bf16 *>(p.dout) + qpos0 * qrs + (int64_t)h * D,
                                   p.qstride * qrs, nvalid);
            }
            if (tid < BQT * nh) {
                const int hh = tid / BQT, r = tid % BQT;
                const int64_t st = row_stat(p, b, kvh * g + h0 + hh, qpos0 + (int64_t)min(r, nvalid - 1) * p.qstride);
                Ls[hh][r] = r < nvalid ? p.lse[st] * kLog2e : 0.f;
                Ds[hh][r] = r < nvalid ? p.drow[st] : 0.f;
            }
            __syncthreads();

            const int lim_first = i0 * qmul + qadd, lim_last = (i0 + BQT - 1) * qmul + qadd;
            const bool active = (lim_last >= jw0) && (p.weff == 0 || lim_first < jw0 + 31 + p.weff) && jw0 < p.Lsub;
            if (!active) continue;
            const bool need_mask = (lim_first < jw0 + 31) || (i0 + BQT > qend) || (jw0 + 32 > p.Lsub) ||
                                   (p.weff != 0 && lim_last - jw0 >= p.weff);
            for (int hh = 0; hh < nh; ++hh) {
                const char *qs = Qs[hh], *gs = Gs[hh];
                f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) {
                    const bf16x8 qa = *reinterpret_cast<const bf16x8 *>(qs + l32 * PITCH + (16 * ks + 8 * hi) * 2);
                    const bf16x8 ga = *reinterpret_cast<const bf16x8 *>(gs + l32 * PITCH + (16 * ks + 8 * hi) * 2);
                    s = mfma32(qa, kf[ks], s);
                    dp = mfma32(ga, vf[ks], dp);
                }
                // register r = 8*m2 + jj holds query 16*m2 + 8*(jj/4) + 4*hi + jj%4
                bf16x8 pop[2], dsop[2];
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) {
                        const int r = 8 * m2 + jj;
                        const int qi = 16 * m2 + 8 * (jj >> 2) + 4 * hi + (jj & 3);
                        const int i = i0 + qi, li = i * qmul + qadd;
                        bool vis = true;
                        if (need_mask)
                            vis = kvalid && i < qend && li >= myk && (p.weff == 0 || li - myk < p.weff);
                        const float e = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -Ls[hh][qi]));
                        const float pr = vis ? e : 0.f;  // a select, not a branch
                        pop[m2][jj] = (bf16)pr;
                        dsop[m2][jj] = (bf16)(pr * (dp[r] - Ds[hh][qi]));
                    }
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) {
                        dv[db] = mfma32(read_rows_tr<D>(gs, 16 * m2, 32 * db, hi, l16, g2), pop[m2], dv[db]);
                        dk[db] = mfma32(read_rows_tr<D>(qs, 16 * m2, 32 * db, hi, l16, g2), dsop[m2], dk[db]);
                    }
            }
        }
    }
    if (kvalid && nseg > 1) {
        // partial row [seg][b][sub][kvh][j]: dK (unscaled) then dV, fp32
        float *pr = p.part + (((((int64_t)seg * p.B + b) * p.nsub + sub) * p.Hkv + kvh) * p.Lsub + myk) * (2 * D);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int c = db * 32 + 8 * r4 + 4 * hi;
                *reinterpret_cast<float4 *>(pr + c) =
                    float4{dk[db][4 * r4], dk[db][4 * r4 + 1], dk[db][4 * r4 + 2], dk[db][4 * r4 + 3]};
                *reinterpret_cast<float4 *>(pr + D + c) =
                    float4{dv[db][4 * r4], dv[db][4 * r4 + 1], dv[db][4 * r4 + 2], dv[db][4 * r4 + 3]};
            }
    } else if (kvalid) {
        const int64_t off = kpos * krs + (int64_t)kvh * D;
        store_rows<D>(static_cast<bf16 *>(p.dk) + off, dk, p.scale, hi);
        store_rows<D>(static_cast<bf16 *>(p.dv) + off, dv, 1.f, hi);
    }
}

// Sum of the segments' partial dK / dV rows in segment order (segments whose
// query range misses the key's block wrote nothing and are skipped), scaled
// and rounded to bf16.  One thread per 4 values of a (b, sub, kvh, key) row.
template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_reduce_kernel(BwdArgs p, int nseg, int segq) {
    constexpr int C4 = 2 * D / 4;  // float4 chunks per row (dK then dV)
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t rows = (int64_t)p.B * p.nsub * p.Hkv * p.Lsub;
    if (t >= rows * C4) return;
    const int c = (int)(t % C4);
    const int64_t row = t / C4;  // ((b * nsub + sub) * Hkv + kvh) * Lsub + j
    const int j = (int)(row % p.Lsub);
    const int kvh = (int)((row / p.Lsub) % p.Hkv);
    const int sub = (int)((row / p.Lsub / p.Hkv) % p.nsub);
    const int b = (int)(row / p.Lsub / p.Hkv / p.nsub);
    const int j0 = j / BKW * BKW;
    const int ib0 = first_query(p, j0), ie0 = query_end(p, min(j0 + BKW, p.Lsub) - 1);
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < nseg; ++s) {
        const int ib = max(ib0, s * segq), ie = min(ie0, min(p.Lq, (s + 1) * segq));
        if (ib >= ie) continue;
        const float4 x = *reinterpret_cast<const float4 *>(p.part + ((int64_t)s * rows + row) * (2 * D) + 4 * c);
        acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
    }
    const bool is_k = 4 * c < D;
    const float mul = is_k ? p.scale : 1.f;
    const int dim = is_k ? 4 * c : 4 * c - D;
    bf16 *out = static_cast<bf16 *>(is_k ? p.dk : p.dv) + (sub_pos(p, b, sub, j) * p.Hkv + kvh) * D + dim;
    *reinterpret_cast<bf16x4 *>(out) = bf16x4{(bf16)(acc.x * mul), (bf16)(acc.y * mul), (bf16)(acc.z * mul), (bf16)(acc.w * mul)};
}

// 3. dQ.  Workgroup = 4 waves = HG heads of one GQA group x TB blocks of 32
// queries (HG*TB = 4), sharing 64-key K/V tiles; per tile:
//   S^T = K Q^T, dP^T = V dO^T   [64 k x 32 q]: lane = query, registers = keys
//   dS^T = P^T (dP^T - D);  dQ^T += K^T dS^T   [D x 32 q]
template <int D, bool GQ>
__global__ __launch_bounds__(256, 2) void bwd_dq_bf16_kernel(BwdArgs p, int HG, int TB, int nqblk) {
    constexpr int PITCH = 2 * D + 16;
    __shared__ __attribute__((aligned(16))) char Ks[2][BKT * PITCH];  // two 64-key sub-tiles per round
    __shared__ __attribute__((aligned(16))) char Vs[2][BKT * PITCH];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5, l16 = lane & 15, g2 = (lane >> 4) & 1;
    const int g = p.Hq / p.Hkv, ngrp = g / HG;

    // workgroup -> (q block, b, kv head, head group, sub); longest blocks first
    const int nrest = p.B * p.Hkv * ngrp * p.nsub;
    const int qblk = nqblk - 1 - (int)(blockIdx.x / nrest);
    int rest = (int)(blockIdx.x % nrest);
    const int sub = rest % p.nsub; rest /= p.nsub;
    const int hgrp = rest % ngrp; rest /= ngrp;
    const int kvh = rest % p.Hkv;
    const int b = rest / p.Hkv;

    const int q0 = qblk * 32 * TB;
    const int h = kvh * g + hgrp * HG + wave % HG;
    const int qw0 = q0 + 32 * (wave / HG);
    const int myq = qw0 + l32;
    const bool qvalid = myq < p.Lq;
    const int qmul = GQ ? p.qmul : 1, qadd = GQ ? p.qadd : 0;
    const int mylim = myq * qmul + qadd, lim0 = qw0 * qmul + qadd, lim1 = (qw0 + 31) * qmul + qadd;
    const int64_t qrs = (int64_t)p.Hq * D, krs = (int64_t)p.Hkv * D;
    const int64_t pos = q_row(p, b, sub, qvalid ? myq : 0);

    // B operands Q^T and dO^T: lane = query, k-slots = dims 16*ks + 8*hi .. +7
    bf16x8 qf[D / 16], gf[D / 16];
    {
        const bf16 *qr = static_cast<const bf16 *>(p.q) + pos * qrs + (int64_t)h * D + 8 * hi;
        const bf16 *gr = static_cast<const bf16 *>(p.dout) + pos * qrs + (int64_t)h * D + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            qf[ks] = qvalid ? *reinterpret_cast<const bf16x8 *>(qr + 16 * ks) : bf16x8{};
            gf[ks] = qvalid ? *reinterpret_cast<const bf16x8 *>(gr + 16 * ks) : bf16x8{};
        }
    }
    const float c2 = p.scale * kLog2e;
    const float lse2 = qvalid ? p.lse[row_stat(p, b, h, pos)] * kLog2e : 0.f;
    const float Dq = qvalid ? p.drow[row_stat(p, b, h, pos)] : 0.f;
    f32x16 dq[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dq[db] = f32x16{};

    const int kend = min((min(q0 + 32 * TB, p.Lq) - 1) * qmul + qadd + 1, p.Lsub);
    const int kbeg = p.weff ? max(0, q0 * qmul + qadd - p.weff + 1) : 0;
    for (int tr = kbeg & ~(BKT - 1); tr < kend; tr += 2 * BKT) {
        __syncthreads();  // previous tiles consumed
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int t0 = tr + u * BKT;
            const int nvalid = max(0, min(BKT, min(p.Lsub, kend) - t0));
            const int64_t kpos0 = sub_pos(p, b, sub, nvalid ? t0 : 0);
            stage_rows<D, BKT>(Ks[u], static_cast<const bf16 *>(p.k) + kpos0 * krs + (int64_t)kvh * D,
                               p.stride * krs, nvalid);
            stage_rows<D, BKT>(Vs[u], static_cast<const bf16 *>(p.v) + kpos0 * krs + (int64_t)kvh * D,
                               p.stride * krs, nvalid);
        }
        __syncthreads();
        for (int u = 0; u < 2; ++u) {
            const int t0 = tr + u * BKT;
            const char *ks_ = Ks[u], *vs_ = Vs[u];
            const bool active = (t0 < kend) && (t0 <= lim1) && (p.weff == 0 || t0 + BKT - 1 > lim0 - p.weff);
            if (!active) continue;
            const bool need_mask =
                (t0 + BKT - 1 > lim0) || (t0 + BKT > p.Lsub) || (p.weff != 0 && t0 <= lim1 - p.weff);
            f32x16 s[2], dp[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                s[kb] = dp[kb] = f32x16{};
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) {
                    const int off = (kb * 32 + l32) * PITCH + (16 * ks + 8 * hi) * 2;
                    s[kb] = mfma32(*reinterpret_cast<const bf16x8 *>(ks_ + off), qf[ks], s[kb]);
                    dp[kb] = mfma32(*reinterpret_cast<const bf16x8 *>(vs_ + off), gf[ks], dp[kb]);
                }
            }
            // register r of block kb holds key t0 + 32*kb + 8*(r/4) + 4*hi + r%4
            bf16x8 dsop[4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) {
                        const int r = 8 * m2 + jj;
                        const int key = t0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
                        bool vis = true;
                        if (need_mask) vis = key <= mylim && key < p.Lsub && (p.weff == 0 || mylim - key < p.weff);
                        const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c2, -lse2));
                        const float pr = vis ? e : 0.f;  // a select, not a branch
                        dsop[kb * 2 + m2][jj] = (bf16)(pr * (dp[kb][r] - Dq));
                    }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                    for (int db = 0; db < D / 32; ++db)
                        dq[db] = mfma32(read_rows_tr<D>(ks_, 32 * kb + 16 * m2, 32 * db, hi, l16, g2),
                                        dsop[kb * 2 + m2], dq[db]);
        }
    }
    if (qvalid) store_rows<D>(static_cast<bf16 *>(p.dq) + pos * qrs + (int64_t)h * D, dq, p.scale, hi);
}

// 3'. dQ at head dim 128 on the forward's d=128 structure: a workgroup is 8
// waves (HG heads of one GQA group x 8/HG blocks of 32 queries) sharing 64-key
// K/V tiles brought in by direct-to-LDS 16-byte copies (global_load_lds),
// double-buffered, one barrier per tile.  K and V rows are 256 B with the
// 16-byte chunk index XOR-swizzled by swzv(row): conflict-free both for the
// row reads of S^T = K Q^T and dP^T = V dO^T (A operands: 16 rows, one chunk)
// and for the transposed K reads of dQ^T += K^T dS^T (4 rows x 4 chunks per
// 32 lanes).  Per tile and wave (lane = query, registers = keys):
//   S^T, dP^T [64 keys x 32 queries]
//   P^T = exp2(scale*log2e * S^T - lse*log2e),  dS^T = P^T (dP^T - D)
//   dQ^T += K^T dS^T, the dS^T accumulators serving directly as B operand.
constexpr int DQ_NW = 8;  // waves per workgroup of the head-dim-128 dQ kernel

template <bool GQ>
__global__ __launch_bounds__(64 * DQ_NW, 1) void bwd_dq_d128_kernel(BwdArgs p, int HG, int TB, int nqblk) {
    constexpr int D = 128, KT = 64, QW = 32;
    constexpr int TILE = KT * D * 2;  // 16 KB per K or V tile
    __shared__ __attribute__((aligned(1024))) char buf0[2 * TILE];  // K | V, even tiles
    __shared__ __attribute__((aligned(1024))) char buf1[2 * TILE];  // K | V, odd tiles

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5, l16 = lane & 15, g2 = (lane >> 4) & 1;
    const int g = p.Hq / p.Hkv, ngrp = g / HG;

    // workgroup -> (query block, group), longest blocks first, balanced over
    // the 8 XCDs as in the forward
    const int nrest = p.B * p.Hkv * ngrp * p.nsub;
    const int nwg = nrest * nqblk;
    const int bid = blockIdx.x;
    int lid = bid;
    if (nwg % 8 == 0) {
        const int x = bid % 8, j = bid / 8;
        if (nrest % 8 == 0) {
            // the XCD's nrest/8 groups interleaved, longest blocks first
            const int gpx = nrest / 8;
            lid = (x * gpx + j % gpx) * nqblk + j / gpx;
        } else if (8 % nrest == 0 && nqblk % (8 / nrest) == 0) {
            const int r = 8 / nrest;
            lid = (x / r) * nqblk + j * r + x % r;
        }
    }
    const int qblk = nqblk - 1 - lid % nqblk;
    int rest = lid / nqblk;
    const int sub = rest % p.nsub; rest /= p.nsub;
    const int hgrp = rest % ngrp; rest /= ngrp;
    const int kvh = rest % p.Hkv;
    const int b = rest / p.Hkv;

    const int QB = QW * TB;
    const int q0 = qblk * QB;
    const int h = kvh * g + hgrp * HG + wave % HG;
    const int qw0 = q0 + (wave / HG) * QW;
    const int myq = qw0 + l32;
    const bool qvalid = myq < p.Lq;
    const int qmul = GQ ? p.qmul : 1, qadd = GQ ? p.qadd : 0;
    const int mylim = myq * qmul + qadd;            // last key this query may see
    const int lim0 = qw0 * qmul + qadd;             // ... for the wave's first query
    const int lim1 = (qw0 + QW - 1) * qmul + qadd;  // ... and its last

    const int64_t qrs = (int64_t)p.Hq * D, krs = (int64_t)p.Hkv * D;
    const int64_t bpos = (int64_t)b * p.nL + p.kbase + sub;  // key element 0
    const bf16 *kg = static_cast<const bf16 *>(p.k) + (int64_t)kvh * D;
    const bf16 *vg = static_cast<const bf16 *>(p.v) + (int64_t)kvh * D;

    const int kend = min((min(q0 + QB, p.Lq) - 1) * qmul + qadd + 1, p.Lsub);
    const int kbeg = p.weff ? max(0, q0 * qmul + qadd - p.weff + 1) : 0;
    const int tfirst = kbeg & ~(KT - 1);
    const int ntiles = (kend - tfirst + KT - 1) / KT;

    // copy-in: wave w moves rows (w*PER + i)*4 + lane/16 of each tile, lane l
    // filling physical chunk l%16 with logical chunk (l%16) ^ swzv(row); rows
    // past the end of the sub-sequence re-read its last row (masked later)
    const int rstride = p.stride * (int)krs;
    constexpr int PER = 16 / DQ_NW;
    int lrow[PER], lchunk[PER];
    unsigned boff[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        lrow[i] = (wave * PER + i) * 4 + (lane >> 4);
        lchunk[i] = ((lane & 15) ^ swzv(lrow[i])) * 8;
        boff[i] = (unsigned)(lrow[i] * rstride + lchunk[i]) * 2u;
    }
    auto issue = [&](int t0, char *dst) {
        const int64_t tbase = (bpos + (int64_t)t0 * p.stride) * krs;
        const bf16 *kt = kg + tbase, *vt = vg + tbase;
        const int rmax = p.Lsub - 1 - t0;
        unsigned bo[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i)
            bo[i] = (rmax < KT - 1) ? (unsigned)(min(lrow[i], rmax) * rstride + lchunk[i]) * 2u : boff[i];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int s0 = (wave * PER + i) * 64;
            lds_dma16_s(kt, bo[i], lds_addr(dst + s0 * 16));
            lds_dma16_s(vt, bo[i], lds_addr(dst + TILE + s0 * 16));
        }
    };
    if (ntiles > 0) issue(tfirst, buf0);

    // B operands Q^T and dO^T: lane = query, k-slots = dims 16*ks + 8*hi .. +7
    const int64_t qrow = (int64_t)b * p.qrows + (int64_t)sub * p.qsub + (int64_t)(qvalid ? myq : 0) * p.qstride;
    bf16x8 qf[D / 16], gf[D / 16];
    {
        const bf16 *qp = static_cast<const bf16 *>(p.q) + qrow * qrs + (int64_t)h * D + 8 * hi;
        const bf16 *gp = static_cast<const bf16 *>(p.dout) + qrow * qrs + (int64_t)h * D + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const bf16x8 x = *reinterpret_cast<const bf16x8 *>(qp + 16 * ks);
            const bf16x8 y = *reinterpret_cast<const bf16x8 *>(gp + 16 * ks);
            qf[ks] = qvalid ? x : bf16x8{};
            gf[ks] = qvalid ? y : bf16x8{};
        }
    }
    const float c2 = p.scale * kLog2e;
    const float lse2 = qvalid ? p.lse[row_stat(p, b, h, qrow)] * kLog2e : 0.f;
    const float Dq = qvalid ? p.drow[row_stat(p, b, h, qrow)] : 0.f;
    f32x16 dq[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dq[db] = f32x16{};

    const int rsw = swzv(l32);  // swzv(32*kb + l32) == swzv(l32)
    // Transposed K read jh of 32-dim block db at key rows r0 (a multiple of
    // 16): within each 16-lane group lane j addresses row r0 + 8jh + 4hi + j/4,
    // dims 32db + 16g2 + 4(j%4); with the swzv swizzle that is the lane base
    // below XOR-ed with (db, jh), plus r0*256 (an immediate offset).
    const unsigned tlane = (unsigned)((4 * hi + (l16 >> 2)) * 256 + ((l16 >> 2) << 6) + (g2 << 5) +
                                      ((((l16 & 3) >> 1) ^ hi) << 4) + ((l16 & 1) << 3));
    auto tile = [&](const char *cur, int t0) {
        const bool active = (t0 <= lim1) && (p.weff == 0 || t0 + KT - 1 > lim0 - p.weff);
        if (!active) return;
        const bool need_mask = (t0 + KT - 1 > lim0) || (t0 + KT > p.Lsub) || (p.weff != 0 && t0 <= lim1 - p.weff);
        const char *kbuf = cur, *vbuf = cur + TILE;
        f32x16 s[2], dp[2];
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] = dp[kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int off = (kb * 32 + l32) * 256 + (((2 * ks + hi) ^ rsw) << 4);
                s[kb] = mfma32(*reinterpret_cast<const bf16x8 *>(kbuf + off), qf[ks], s[kb]);
                dp[kb] = mfma32(*reinterpret_cast<const bf16x8 *>(vbuf + off), gf[ks], dp[kb]);
            }
        __builtin_amdgcn_s_setprio(0);
        if (need_mask) {  // visible <=> lo <= key <= hi_key, one unsigned compare
            const int lo = p.weff ? mylim - p.weff + 1 : 0;
            const unsigned span = (unsigned)(min(mylim, p.Lsub - 1) - lo);
            const int base = t0 + 4 * hi - lo;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const unsigned u = (unsigned)(base + kb * 32 + 8 * (r >> 2) + (r & 3));
                    s[kb][r] = (u <= span) ? s[kb][r] : -INFINITY;
                }
        }
        // register r of block kb holds key t0 + 32*kb + 8*(r/4) + 4*hi + r%4
        bf16x8 dsall[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int r = 8 * m2 + j;
                    const float pr = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c2, -lse2));
                    dsall[kb * 2 + m2][j] = (bf16)(pr * (dp[kb][r] - Dq));
                }
        __builtin_amdgcn_sched_barrier(0);
        unsigned tl = tlane;  // derived per tile, not held across the loop
        asm volatile("" : "+v"(tl));
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2) {
                const bf16x8 dsop = dsall[kb * 2 + m2];
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    s16x4 half[2];
#pragma unroll
                    for (int jh = 0; jh < 2; ++jh) {
                        const unsigned a = (tl ^ (unsigned)((db << 6) | (jh << 5))) + (kb * 32 + 16 * m2 + 8 * jh) * 256;
                        half[jh] = lds_read_tr16(kbuf + a);
                    }
                    const s16x8 both = __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
                    dq[db] = mfma32(__builtin_bit_cast(bf16x8, both), dsop, dq[db]);
                }
            }
        // the 32 transposed K reads run eight ahead of the 16 dQ MFMAs, two
        // per MFMA after that (sched_group_barrier masks: 0x100 LDS reads,
        // 0x008 MFMA)
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int i = 0; i < 12; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    for (int it = 0; it < ntiles; it += 2) {
        const int t0 = tfirst + it * KT;
        __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of tile it have landed
        __syncthreads();                // ... and every wave's; tile it-1 fully consumed
        if (it + 1 < ntiles) issue(t0 + KT, buf1);
        tile(buf0, t0);
        if (it + 1 < ntiles) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (it + 2 < ntiles) issue(t0 + 2 * KT, buf0);
            tile(buf1, t0 + KT);
        }
    }
    if (qvalid) store_rows<D>(static_cast<bf16 *>(p.dq) + qrow * qrs + (int64_t)h * D, dq, p.scale, hi);
}

// dK, dV for d = 128: the workgroup of the generic kernel above (8 waves x 32
// keys, K^T and V^T held as B operands in registers), with each round's
// query tiles (Q and dO rows of up to four heads, 64 KB) and their lse / D
// values copied direct to LDS and double-buffered, so the next round's copy
// is in flight while this round is computed.  Tiles are stored unpadded with
// row r's 16-byte chunks XOR-swizzled by swzv(r): conflict-free for the row
// reads of S = Q K^T and dP = dO V^T (32 rows, one chunk) and for the
// transposed reads of dV^T += dO^T P and dK^T += Q^T dS.
constexpr int DKV_NW = 8;  // waves (32 keys each) per workgroup
constexpr int DKV_HS = 4;  // heads of the group per round

template <bool GQ>
__global__ __launch_bounds__(64 * DKV_NW, 1) void bwd_dkdv_d128_kernel(BwdArgs p, int nseg, int segq) {
    constexpr int D = 128, QT = 32;
    constexpr int QTILE = QT * D * 2;          // 8 KB: 32 rows of one head
    constexpr int RB = 2 * DKV_HS * QTILE;     // Q tiles | dO tiles of a round
    __shared__ __attribute__((aligned(4096))) char tb0[RB];
    __shared__ __attribute__((aligned(4096))) char tb1[RB];
    __shared__ __attribute__((aligned(256))) float sb0[2][DKV_HS][QT];  // lse | D of the rows
    __shared__ __attribute__((aligned(256))) float sb1[2][DKV_HS][QT];
    // Per-lane constants read back each round (ds_read, counted by lgkmcnt)
    // instead of being held in registers across the loop: the kernel is at
    // its register limit, and a spilled value's reload from scratch would wait
    // (vmcnt counts in order) for the next round's copies issued before it.
    __shared__ unsigned lane_tab[6][64 * DKV_NW];  // aoff, toff, copy offsets 0..3

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5, l16 = lane & 15, g2 = (lane >> 4) & 1;
    const int g = p.Hq / p.Hkv;

    const int ngroups = p.B * p.Hkv * p.nsub;
    const int kseg = (int)(blockIdx.x / ngroups);
    const int kblk = kseg / nseg, seg = kseg % nseg;
    int rest = (int)(blockIdx.x % ngroups);
    const int sub = rest % p.nsub; rest /= p.nsub;
    const int kvh = rest % p.Hkv;
    const int b = rest / p.Hkv;
    const int j0 = kblk * BKW;
    const int jw0 = j0 + 32 * wave;
    const int myk = jw0 + l32;
    const bool kvalid = myk < p.Lsub;

    const int qend = nseg > 1 ? min(p.Lq, (seg + 1) * segq) : p.Lq;
    const int ibeg = max(first_query(p, j0), seg * segq);
    const int iend = min(query_end(p, min(j0 + BKW, p.Lsub) - 1), qend);
    if (nseg > 1 && ibeg >= iend) return;  // empty segment: the reduction skips it

    const int64_t qrs = (int64_t)p.Hq * D, krs = (int64_t)p.Hkv * D;
    const int64_t kpos = sub_pos(p, b, sub, kvalid ? myk : 0);
    bf16x8 kf[D / 16], vf[D / 16];
    {
        const bf16 *kr = static_cast<const bf16 *>(p.k) + kpos * krs + (int64_t)kvh * D + 8 * hi;
        const bf16 *vr = static_cast<const bf16 *>(p.v) + kpos * krs + (int64_t)kvh * D + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            kf[ks] = kvalid ? *reinterpret_cast<const bf16x8 *>(kr + 16 * ks) : bf16x8{};
            vf[ks] = kvalid ? *reinterpret_cast<const bf16x8 *>(vr + 16 * ks) : bf16x8{};
        }
    }
    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dk[db] = dv[db] = f32x16{};

    const float c2 = p.scale * kLog2e;
    const int qmul = GQ ? p.qmul : 1, qadd = GQ ? p.qadd : 0;
    const int ntq = iend > ibeg ? (iend - ibeg + QT - 1) / QT : 0;
    const int nrounds = ntq * ((g + DKV_HS - 1) / DKV_HS);

    // copy-in: wave w moves the 32 rows of tensor w / 4 (Q, dO) of head w % 4,
    // 4 rows per instruction; lane l fills physical chunk l % 16 of row
    // 4i + l/16 with logical chunk (l % 16) ^ swzv(row), and swzv(4i + l/16) =
    // 4*(l/16) + i%4, so four per-lane offsets serve all eight instructions
    const int ct = wave / DKV_HS, chh = wave % DKV_HS;
    const int rs = p.qstride * (int)qrs;  // elements between consecutive query rows
    auto issue = [&](int k, char *tb, float (*sb)[DKV_HS][QT]) {
        const int h0 = (k / ntq) * DKV_HS, i0 = ibeg + (k % ntq) * QT;
        const int nh = min(DKV_HS, g - h0);
        const int nvalid = min(QT, qend - i0);
        const int64_t qpos0 = q_row(p, b, sub, i0);
        unsigned voff[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) voff[m] = lane_tab[2 + m][tid];
        if (chh < nh) {
            const bf16 *src = static_cast<const bf16 *>(ct ? p.dout : p.q) + qpos0 * qrs + (int64_t)(kvh * g + h0 + chh) * D;
            char *dst = tb + (ct * DKV_HS + chh) * QTILE;
            if (nvalid == QT) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    lds_dma16_s(src + (int64_t)i * 4 * rs, voff[i & 3], lds_addr(dst + i * 1024));
            } else {  // tail: rows past the segment re-read its last row (masked later)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = 4 * i + (lane >> 4);
                    const unsigned vo = (unsigned)(min(r, nvalid - 1) * rs + (((lane & 15) ^ swzv(r)) * 8)) * 2u;
                    lds_dma16_s(src, vo, lds_addr(dst + i * 1024));
                }
            }
        }
        if (wave == 0) {  // lse and D of the round's rows: 2 heads x 32 rows per instruction
#pragma unroll
            for (int j = 0; j < DKV_HS / 2; ++j) {
                const int hh = min(2 * j + (lane >> 5), nh - 1);
                const int64_t qr = qpos0 + (int64_t)min(l32, nvalid - 1) * p.qstride;
                const unsigned so = (unsigned)row_stat(p, b, kvh * g + h0 + hh, qr) * 4u;
                lds_dma4_s(p.lse, so, lds_addr(reinterpret_cast<char *>(&sb[0][2 * j][0])));
                lds_dma4_s(p.drow, so, lds_addr(reinterpret_cast<char *>(&sb[1][2 * j][0])));
            }
        }
    };

    // LDS read addresses: the lane's offset within a tile for k-step 0 (row
    // reads) and for (m2, db, jh) = 0 (transposed reads); the others follow by
    // XOR with a constant (the swizzle only permutes bits 4..7 of a row, and
    // tiles are 4 KB aligned), so each read costs one v_xor, not a register
    const int rsw = swzv(l32);
    const unsigned aoff = (unsigned)(l32 * 256 + ((hi ^ rsw) << 4));  // ks -> aoff ^ (ks << 5)
    unsigned toff;  // (m2, db, jh) -> (toff ^ (64*db + 2080*jh)) + 4096*m2
    {
        const int row = 4 * hi + (l16 >> 2), dim = 16 * g2 + 4 * (l16 & 3);
        toff = (unsigned)(row * 256 + (((dim >> 3) ^ swzv(row)) << 4) + ((dim >> 2) & 1) * 8);
    }
    lane_tab[0][tid] = aoff;
    lane_tab[1][tid] = toff;
#pragma unroll
    for (int m = 0; m < 4; ++m)
        lane_tab[2 + m][tid] = (unsigned)((lane >> 4) * rs + (((lane & 15) ^ (4 * (lane >> 4) + m)) * 8)) * 2u;
    __syncthreads();
    auto round = [&](int k, const char *tb, const float (*sb)[DKV_HS][QT]) {
        const int h0 = (k / ntq) * DKV_HS, i0 = ibeg + (k % ntq) * QT;
        const int nh = min(DKV_HS, g - h0);
        const int lim_first = i0 * qmul + qadd, lim_last = (i0 + QT - 1) * qmul + qadd;
        const bool active = (lim_last >= jw0) && (p.weff == 0 || lim_first < jw0 + 31 + p.weff) && jw0 < p.Lsub;
        if (!active) return;
        const bool need_mask = (lim_first < jw0 + 31) || (i0 + QT > qend) || (jw0 + 32 > p.Lsub) ||
                               (p.weff != 0 && lim_last - jw0 >= p.weff);
        const unsigned ao = lane_tab[0][tid], to = lane_tab[1][tid];
        int hr = hi;  // the lse / D reads' lane part, derived per round (see lane_tab)
        asm volatile("" : "+v"(hr));
        for (int hh = 0; hh < nh; ++hh) {
            unsigned qa = lds_addr(tb + hh * QTILE) + ao, qt = lds_addr(tb + hh * QTILE) + to;
            asm volatile("" : "+v"(qa), "+v"(qt));  // keep the derived addresses per use
            constexpr unsigned GOFF = DKV_HS * QTILE;  // dO tile of the same head
            f32x16 s = f32x16{}, dp = f32x16{};
            __builtin_amdgcn_s_setprio(1);  // MFMA phases win issue arbitration over the other wave's VALU
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const unsigned a = qa ^ (unsigned)(ks << 5);
                s = mfma32(*reinterpret_cast<__attribute__((address_space(3))) const bf16x8 *>((size_t)a), kf[ks], s);
                dp = mfma32(*reinterpret_cast<__attribute__((address_space(3))) const bf16x8 *>((size_t)(a + GOFF)),
                            vf[ks], dp);
            }
            __builtin_amdgcn_s_setprio(0);
            // register r = 8*m2 + jj holds query 16*m2 + 8*(jj/4) + 4*hi + jj%4
            bf16x8 pop[2], dsop[2];
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int r = 8 * m2 + jj;
                    const int qi = 16 * m2 + 8 * (jj >> 2) + 4 * hi + (jj & 3);
                    const int qr = 16 * m2 + 8 * (jj >> 2) + 4 * hr + (jj & 3);  // == qi
                    const int i = i0 + qi, li = i * qmul + qadd;
                    bool vis = true;
                    if (need_mask) vis = kvalid && i < qend && li >= myk && (p.weff == 0 || li - myk < p.weff);
                    const float e = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -sb[0][hh][qr] * kLog2e));
                    const float pr = vis ? e : 0.f;  // a select, not a branch
                    pop[m2][jj] = (bf16)pr;
                    dsop[m2][jj] = (bf16)(pr * (dp[r] - sb[1][hh][qr]));
                }
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    s16x4 hg[2], hq[2];
#pragma unroll
                    for (int jh = 0; jh < 2; ++jh) {
                        const unsigned a = (qt ^ (unsigned)(64 * db + 2080 * jh)) + 4096u * m2;
                        hq[jh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            reinterpret_cast<__attribute__((address_space(3))) s16x4 *>((size_t)a));
                        hg[jh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            reinterpret_cast<__attribute__((address_space(3))) s16x4 *>((size_t)(a + GOFF)));
                    }
                    const s16x8 bg = __builtin_shufflevector(hg[0], hg[1], 0, 1, 2, 3, 4, 5, 6, 7);
                    const s16x8 bq = __builtin_shufflevector(hq[0], hq[1], 0, 1, 2, 3, 4, 5, 6, 7);
                    dv[db] = mfma32(__builtin_bit_cast(bf16x8, bg), pop[m2], dv[db]);
                    dk[db] = mfma32(__builtin_bit_cast(bf16x8, bq), dsop[m2], dk[db]);
                }
            // the 32 transposed reads run eight ahead of the 16 dV/dK MFMAs,
            // two per MFMA after that
            __builtin_amdgcn_s_setprio(1);
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
            for (int i = 0; i < 12; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
        }
    };

    if (nrounds > 0) issue(0, tb0, sb0);
    for (int k = 0; k < nrounds; k += 2) {
        __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of round k have landed
        __syncthreads();                // ... and every wave's; round k-1 fully consumed
        if (k + 1 < nrounds) issue(k + 1, tb1, sb1);
        round(k, tb0, sb0);
        if (k + 1 < nrounds) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (k + 2 < nrounds) issue(k + 2, tb0, sb0);
            round(k + 1, tb1, sb1);
        }
    }

    if (kvalid && nseg > 1) {
        float *pr = p.part + (((((int64_t)seg * p.B + b) * p.nsub + sub) * p.Hkv + kvh) * p.Lsub + myk) * (2 * D);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int c = db * 32 + 8 * r4 + 4 * hi;
                *reinterpret_cast<float4 *>(pr + c) =
                    float4{dk[db][4 * r4], dk[db][4 * r4 + 1], dk[db][4 * r4 + 2], dk[db][4 * r4 + 3]};
                *reinterpret_cast<float4 *>(pr + D + c) =
                    float4{dv[db][4 * r4], dv[db][4 * r4 + 1], dv[db][4 * r4 + 2], dv[db][4 * r4 + 3]};
            }
    } else if (kvalid) {
        const int64_t off = kpos * krs + (int64_t)kvh * D;
        store_rows<D>(static_cast<bf16 *>(p.dk) + off, dk, p.scale, hi);
        store_rows<D>(static_cast<bf16 *>(p.dv) + off, dv, 1.f, hi);
    }
}

// dK and dV rows that no key sub-sequence covers (the other streams of a
// final-stream intra layer: position t is covered iff (t - kbase) mod stride
// < nsub) receive no gradient: write zeros, 16 bytes per thread.
__global__ __launch_bounds__(256) void bwd_zero_uncovered_kernel(BwdArgs p, int chunks_per_row, int64_t nchunks) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= nchunks) return;
    const int64_t t = (c / chunks_per_row / p.Hkv) % p.nL;  // position within the batch row
    const int64_t rel = ((t - p.kbase) % p.stride + p.stride) % p.stride;
    if (rel < p.nsub) return;
    reinterpret_cast<uint4 *>(p.dk)[c] = uint4{0, 0, 0, 0};
    reinterpret_cast<uint4 *>(p.dv)[c] = uint4{0, 0, 0, 0};
}

hipError_t launch_zero_uncovered(const BwdArgs &a, int elem_bytes, hipStream_t st) {
    if (a.nsub == a.stride) return hipSuccess;  // every position is some sub-sequence's key
    const int chunks_per_row = a.d * elem_bytes / 16;
    const int64_t nchunks = (int64_t)a.B * a.nL * a.Hkv * chunks_per_row;
    const int64_t grid = (nchunks + 255) / 256;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bwd_zero_uncovered_kernel, dim3((unsigned)grid), dim3(256), 0, st, a, chunks_per_row,
                       nchunks);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_drow(const BwdArgs &a, hipStream_t st) {
    const int64_t rows = (int64_t)a.B * a.qrows * a.Hq;
    const int64_t grid = (rows + 15) / 16;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    switch (a.d) {
        case 32: hipLaunchKernelGGL((bwd_drow_kernel<T, 32>), dim3((unsigned)grid), dim3(256), 0, st, a); break;
        case 64: hipLaunchKernelGGL((bwd_drow_kernel<T, 64>), dim3((unsigned)grid), dim3(256), 0, st, a); break;
        case 128: hipLaunchKernelGGL((bwd_drow_kernel<T, 128>), dim3((unsigned)grid), dim3(256), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int D, bool GQ>
hipError_t launch_bf16_d(const BwdArgs &a, hipStream_t st) {
    const int g = a.Hq / a.Hkv;
    const int nkblk = (a.Lsub + BKW - 1) / BKW;
    const int64_t kgrid = (int64_t)nkblk * a.B * a.Hkv * a.nsub;
    const int HG = (g % 4 == 0) ? 4 : (g % 2 == 0) ? 2 : 1;
    const int TB = 4 / HG;
    const int nqblk = (a.Lq + 32 * TB - 1) / (32 * TB);
    const int64_t qgrid = (int64_t)nqblk * a.B * a.Hkv * (g / HG) * a.nsub;
    if (kgrid > 0x7fffffff || qgrid > 0x7fffffff) return hipErrorInvalidConfiguration;
    const BwdSplit sp = bwd_split(a);
    if (kgrid * sp.nseg > 0x7fffffff) return hipErrorInvalidConfiguration;
    // the d=128 kernel's per-lane copy offsets are 32-bit: 31 query rows +
    // 256 B, and the lse / D index of any row, in bytes
    if (D == 128 && (int64_t)31 * a.qstride * a.Hq * D * 2 + 256 < ((int64_t)1 << 32) &&
        (int64_t)a.B * a.Hq * a.qrows * 4 < ((int64_t)1 << 32)) {
        hipLaunchKernelGGL((bwd_dkdv_d128_kernel<GQ>), dim3((unsigned)(kgrid * sp.nseg)), dim3(64 * DKV_NW), 0, st,
                           a, sp.nseg, sp.segq);
    } else {
        hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, GQ>), dim3((unsigned)(kgrid * sp.nseg)), dim3(512), 0, st, a,
                           sp.nseg, sp.segq);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (sp.nseg > 1) {
        const int64_t n4 = (int64_t)a.B * a.nsub * a.Hkv * a.Lsub * (2 * D / 4);
        if ((n4 + 255) / 256 > 0x7fffffff) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(bwd_dkdv_reduce_kernel<D>, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, a,
                           sp.nseg, sp.segq);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // 32-bit per-lane copy offsets of the d=128 dQ kernel: rows 0..63 of a tile
    if (D == 128 && (int64_t)64 * a.stride * a.Hkv * D * 2 < ((int64_t)1 << 32)) {
        const int TB2 = DQ_NW / HG;
        const int nqblk2 = (a.Lq + 32 * TB2 - 1) / (32 * TB2);
        const int64_t grid2 = (int64_t)nqblk2 * a.B * a.Hkv * (g / HG) * a.nsub;
        if (grid2 > 0x7fffffff) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((bwd_dq_d128_kernel<GQ>), dim3((unsigned)grid2), dim3(64 * DQ_NW), 0, st, a, HG, TB2,
                           nqblk2);
    } else {
        hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, GQ>), dim3((unsigned)qgrid), dim3(256), 0, st, a, HG, TB, nqblk);
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_bf16_map(const BwdArgs &a, hipStream_t st) {
    return (a.qmul != 1 || a.qadd != 0) ? launch_bf16_d<D, true>(a, st) : launch_bf16_d<D, false>(a, st);
}

template <int D>
hipError_t launch_f32_d(const BwdArgs &a, hipStream_t st) {
    const int64_t qrows = (int64_t)a.B * a.nsub * a.Lq * a.Hq;
    const int64_t krows = (int64_t)a.B * a.nsub * a.Lsub * a.Hkv;
    if ((qrows + 63) / 64 > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bwd_dq_f32_kernel<D>, dim3((unsigned)((qrows + 63) / 64)), dim3(64), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dkdv_f32_kernel<D>, dim3((unsigned)((krows + 63) / 64)), dim3(64), 0, st, a);
    return hipGetLastError();
}

}  // namespace

BwdSplit bwd_split(const BwdArgs &a) {
    // key waves (32 keys each) of the dK/dV kernel; below four per SIMD of
    // the chip the query range is cut into segments of >= 128 queries, about
    // 8192 / waves of them (at most 8)
    const int64_t waves = (int64_t)a.B * a.Hkv * a.nsub * ((a.Lsub + 31) / 32);
    BwdSplit s{1, a.Lq};
    if (waves >= 4096 || a.Lq < 256) return s;
    const int want = (int)std::min<int64_t>(8, (8192 + waves - 1) / waves);
    int segq = (a.Lq + want - 1) / want;
    segq = std::max(128, (segq + BQT - 1) / BQT * BQT);
    const int nseg = (a.Lq + segq - 1) / segq;
    if (nseg > 1) s = BwdSplit{nseg, segq};
    return s;
}

size_t bwd_workspace_bytes(const BwdArgs &a, bool bf16_path) {
    size_t bytes = ((size_t)a.B * a.Hq * a.qrows * sizeof(float) + 255) / 256 * 256;
    const BwdSplit sp = bf16_path ? bwd_split(a) : BwdSplit{1, a.Lq};
    if (sp.nseg > 1) bytes += (size_t)sp.nseg * a.B * a.nsub * a.Hkv * a.Lsub * 2 * a.d * sizeof(float);
    return bytes;
}

hipError_t launch_sfa_bwd_bf16(const BwdArgs &a, hipStream_t st) {
    hipError_t e = launch_zero_uncovered(a, 2, st);
    if (e != hipSuccess) return e;
    e = launch_drow<bf16>(a, st);
    if (e != hipSuccess) return e;
    switch (a.d) {
        case 32: return launch_bf16_map<32>(a, st);
        case 64: return launch_bf16_map<64>(a, st);
        case 128: return launch_bf16_map<128>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_sfa_bwd_f32(const BwdArgs &a, hipStream_t st) {
    hipError_t e = launch_zero_uncovered(a, 4, st);
    if (e != hipSuccess) return e;
    e = launch_drow<float>(a, st);
    if (e != hipSuccess) return e;
    switch (a.d) {
        case 32: return launch_f32_d<32>(a, st);
        case 64: return launch_f32_d<64>(a, st);
        case 128: return launch_f32_d<128>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace hd
