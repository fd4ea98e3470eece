// sfa_decode_bf16.hip -- one decode step of Stream-Factorized Attention over
// the retained per-stream KV cache, bf16 in / fp32 accumulate.
//
// Method ("Hidden Decoding at Scale"): one KV cache per stream is kept
// ("Persistent KV and the KV-mirror Saving") and the n streams of the new
// token are processed together in one pass ("Inference Throughput").  The new
// token's query of stream s sits at expanded position len*n + s and attends
// under the layer's mask (Figure 2) over tokens 0..len.
//
// The step is HBM-bound: the cache is read once.  It runs as split-KV:
//   kernel 1  grid (split, b*Hkv): a workgroup streams `chunk` tokens x n
//             streams of one kv head's cache and scores them against all
//             n*g queries of that head group (g = Hq/Hkv) at once -- 16-row
//             query blocks on v_mfma_f32_16x16x32_bf16 -- then merges its four
//             waves and writes one fp32 partial (max, sum, acc[d]) per query.
//             The split holding token len also appends the new K/V rows to
//             the cache; no split reads cache row len (the new row is read
//             from k_new / v_new), so the append races with nothing.
//   kernel 2  one wavefront per output row merges the partials of the splits
//             that ran, in split order (log-sum-exp), and rounds to bf16.
// Intra-stream layers use only the stream-diagonal entries of each score
// block; the masked lanes cost matrix-core cycles, not bytes.
//
// 16x16x32 bf16 operand layout: lane l supplies row (l % 16) of A / column of
// B and k-slots 8*(l/16) .. +7; the accumulator holds C[4*(l/16) + i][l % 16].
#include <algorithm>

#include "attn_common.h"

namespace hd {

namespace {

// Workgroups the d=128 split aims for (one per CU at a time; 512-1024 measured
// best at B=64, ctx 8192: fewer leave HBM idle, more pay start-up latency).
constexpr int kDecodeTargetWgs = 1024;

constexpr int NW = 4;    // waves per workgroup
constexpr int RB = 32;   // cache rows per wave block

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct Split {
    int chunk;   // tokens per split
    int nsplit;  // splits per (b, kv head)
};

bool use_d128_path(int n, int d) { return d == 128 && 64 % n == 0; }

Split choose_split_d128(int B, int Hkv, int T_cap, int target = kDecodeTargetWgs) {
    // One workgroup per CU (128 KB LDS): aim for ~target workgroups, chunks
    // of >= 64 tokens in multiples of 16.
    const int64_t bh = (int64_t)B * Hkv;
    const int64_t want = (target + bh - 1) / bh;
    int64_t chunk = ((int64_t)T_cap + want - 1) / want;
    chunk = ((chunk + 15) / 16) * 16;
    if (chunk < 64) chunk = 64;
    Split s;
    s.chunk = (int)chunk;
    s.nsplit = (int)(((int64_t)T_cap + chunk - 1) / chunk);
    return s;
}

Split choose_split(int B, int Hkv, int T_cap) {
    // Aim for at least ~2048 workgroups (8 per CU) so enough cache bytes are in
    // flight, with chunks of >= 64 tokens and a multiple of 16 tokens.
    const int64_t bh = (int64_t)B * Hkv;
    int64_t want = (2048 + bh - 1) / bh;
    int64_t chunk = ((int64_t)T_cap + want - 1) / want;
    chunk = ((chunk + 15) / 16) * 16;
    if (chunk < 64) chunk = 64;
    Split s;
    s.chunk = (int)chunk;
    s.nsplit = (int)(((int64_t)T_cap + chunk - 1) / chunk);
    return s;
}

template <int D, int NQB>
__global__ __launch_bounds__(256) void decode_partial_kernel(DecArgs p, Split sp, float scale_log2) {
    constexpr int VP = D + 8;  // LDS pitch of the staged V rows
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, grp = lane >> 4;
    const int split = blockIdx.x;
    const int bh = blockIdx.y;
    const int b = bh / p.Hkv, kvh = bh - b * p.Hkv;
    const int n = p.n, g = p.Hq / p.Hkv, QR = p.nqs * g;
    const int len = p.cache_len[b];
    const int c0 = split * sp.chunk;
    // a length outside [0, T_cap) breaks the caller's contract: no append, no
    // scan (the combine writes NaN rows for that sequence)
    if (len < 0 || len >= p.T_cap) return;
    if (c0 > len) return;  // nothing cached here yet; the combine skips it
    const int c1 = min(c0 + sp.chunk, len + 1);

    const bf16 *kn = static_cast<const bf16 *>(p.k_new);
    const bf16 *vn = static_cast<const bf16 *>(p.v_new);
    bf16 *kc = static_cast<bf16 *>(p.k_cache);
    bf16 *vc = static_cast<bf16 *>(p.v_cache);
    const int64_t cache_tok = (int64_t)n * p.Hkv * D;  // elements per cached token
    const int64_t cache_b = (int64_t)b * p.T_cap * cache_tok + (int64_t)kvh * D;
    const int64_t new_b = (int64_t)b * n * p.Hkv * D + (int64_t)kvh * D;

    // Append the new token's rows of this kv head (row len is read by nobody).
    if (len < c1) {
        for (int c = tid; c < n * (D / 8); c += 256) {
            const int s = c / (D / 8), cc = c - s * (D / 8);
            const int64_t src = new_b + (int64_t)s * p.Hkv * D + cc * 8;
            const int64_t dst = cache_b + (int64_t)len * cache_tok + (int64_t)s * p.Hkv * D + cc * 8;
            *reinterpret_cast<uint4 *>(kc + dst) = *reinterpret_cast<const uint4 *>(kn + src);
            *reinterpret_cast<uint4 *>(vc + dst) = *reinterpret_cast<const uint4 *>(vn + src);
        }
    }

    // Tokens older than len - window are invisible to every query.
    const int tlo = p.window ? max(c0, len - p.window) : c0;
    const int64_t row_lo = (int64_t)tlo * n, row_hi = (int64_t)c1 * n;
    const int nrow = row_hi > row_lo ? (int)(row_hi - row_lo) : 0;
    const int nblk = (nrow + RB - 1) / RB;
    const int iters = (nblk + NW - 1) / NW;

    // Query operands: block qb, lane column l16 is query row c = qb*16 + l16
    // (row c <-> stream qs0 + c / g, head kvh*g + c % g); slots grp hold dims
    // ks*32 + 8*grp .. +7.
    const bf16 *qg = static_cast<const bf16 *>(p.q);
    bf16x8 qop[NQB][D / 32];
    int qstream[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int c = qb * 16 + l16;
        const bool ok = c < QR;
        const int sr = ok ? c / g : 0, hh = ok ? c - sr * g : 0;  // query stream qs0 + sr
        qstream[qb] = p.qs0 + sr;
        const bf16 *qp = qg + (((int64_t)b * p.nqs + sr) * p.Hq + kvh * g + hh) * D + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            bf16x8 x = *reinterpret_cast<const bf16x8 *>(qp + ks * 32);
            qop[qb][ks] = ok ? x : bf16x8{};
        }
    }

    f32x4 oacc[NQB][D / 16];
    float m_run[NQB], l_run[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        m_run[qb] = -INFINITY;
        l_run[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) oacc[qb][db] = f32x4{};
    }

    bf16 *Vw = reinterpret_cast<bf16 *>(smem) + wave * RB * VP;
    const int64_t tq_base = (int64_t)len * n;

    for (int it = 0; it < iters; ++it) {
        const int blk = it * NW + wave;
        const int64_t rbase = row_lo + (int64_t)blk * RB;

        // Source address of cache row r (token r/n, stream r%n); -1 if absent.
        auto row_src = [&](int64_t r, const bf16 *&kp, const bf16 *&vp) -> bool {
            if (blk >= nblk || r >= row_hi) return false;
            const int64_t tok = r / n;
            const int s = (int)(r - tok * n);
            if (tok < len) {
                const int64_t off = cache_b + tok * cache_tok + (int64_t)s * p.Hkv * D;
                kp = kc + off; vp = vc + off;
            } else {
                const int64_t off = new_b + (int64_t)s * p.Hkv * D;
                kp = kn + off; vp = vn + off;
            }
            return true;
        };

        // K operands straight from global memory, V rows into this wave's LDS.
        bf16x8 kop[2][D / 32];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            const bf16 *kp = nullptr, *vp = nullptr;
            const bool ok = row_src(rbase + kh * 16 + l16, kp, vp);
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks)
                kop[kh][ks] = ok ? *reinterpret_cast<const bf16x8 *>(kp + ks * 32 + 8 * grp) : bf16x8{};
        }
#pragma unroll
        for (int c = lane; c < RB * (D / 8); c += 64) {
            const int r = c / (D / 8), cc = c - r * (D / 8);
            const bf16 *kp = nullptr, *vp = nullptr;
            uint4 x = {0, 0, 0, 0};
            if (row_src(rbase + r, kp, vp)) x = *reinterpret_cast<const uint4 *>(vp + cc * 8);
            *reinterpret_cast<uint4 *>(Vw + r * VP + cc * 8) = x;
        }
        __syncthreads();

        if (blk < nblk) {
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                f32x4 sacc[2];
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) {
                    sacc[kh] = f32x4{};
#pragma unroll
                    for (int ks = 0; ks < D / 32; ++ks) sacc[kh] = mfma16(kop[kh][ks], qop[qb][ks], sacc[kh]);
                }
                const int sq = qstream[qb];
                const int64_t tq = tq_base + sq;
                float mx = -INFINITY;
#pragma unroll
                for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t r = rbase + kh * 16 + 4 * grp + i;
                        const int64_t tok = r / n;
                        const int sk = (int)(r - tok * n);
                        bool vis = r < row_hi;
                        if (p.mode == 0) vis = vis && sk == sq && (p.window == 0 || len - tok < p.window);
                        else vis = vis && r <= tq && (p.window == 0 || tq - r < (int64_t)n * p.window);
                        const float x = vis ? sacc[kh][i] * scale_log2 : -INFINITY;
                        sacc[kh][i] = x;
                        mx = fmaxf(mx, x);
                    }
                mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                const float m_new = fmaxf(m_run[qb], mx);
                const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_use);
                bf16x8 pop;
                float lsum = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float pv = __builtin_amdgcn_exp2f(sacc[j >> 2][j & 3] - m_use);
                    lsum += pv;
                    pop[j] = (bf16)pv;
                }
                l_run[qb] = l_run[qb] * alpha + lsum;
                m_run[qb] = m_new;
#pragma unroll
                for (int db = 0; db < D / 16; ++db) oacc[qb][db] *= alpha;
                // slot j <-> key row 16*(j/4) + 4*grp + (j%4) of the block
#pragma unroll
                for (int db = 0; db < D / 16; ++db) {
                    bf16x8 vop;
                    const bf16 *vcol = Vw + 4 * grp * VP + db * 16 + l16;
#pragma unroll
                    for (int j = 0; j < 8; ++j) vop[j] = vcol[(16 * (j >> 2) + (j & 3)) * VP];
                    oacc[qb][db] = mfma16(vop, pop, oacc[qb][db]);
                }
            }
        }
        __syncthreads();
    }

    // Merge the four waves, then write this split's partial per query row.
    float *ml = reinterpret_cast<float *>(smem);            // [NW][NQB*16][2]
    float *ow = ml + NW * NQB * 16 * 2;                     // [NW][NQB*16][D]
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        float lt = l_run[qb];
        lt += __shfl_xor(lt, 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        const int c = qb * 16 + l16;
        if (grp == 0) {
            ml[(wave * NQB * 16 + c) * 2 + 0] = m_run[qb];
            ml[(wave * NQB * 16 + c) * 2 + 1] = lt;
        }
#pragma unroll
        for (int db = 0; db < D / 16; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ow[(wave * NQB * 16 + c) * D + db * 16 + 4 * grp + i] = oacc[qb][db][i];
    }
    __syncthreads();
    const int64_t part = ((int64_t)bh * sp.nsplit + split) * QR;
    float *ws_acc = p.ws;
    float *ws_ml = p.ws + (int64_t)p.B * p.Hkv * sp.nsplit * QR * D;
    for (int e = tid; e < QR * D; e += 256) {
        const int c = e / D, dim = e - c * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, ml[(w * NQB * 16 + c) * 2]);
        const float Mu = (M == -INFINITY) ? 0.f : M;
        float acc = 0.f, L = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float wt = __builtin_amdgcn_exp2f(ml[(w * NQB * 16 + c) * 2] - Mu);
            acc += wt * ow[(w * NQB * 16 + c) * D + dim];
            L += wt * ml[(w * NQB * 16 + c) * 2 + 1];
        }
        ws_acc[(part + c) * D + dim] = acc;
        if (dim == 0) {
            ws_ml[(part + c) * 2 + 0] = M;
            ws_ml[(part + c) * 2 + 1] = L;
        }
    }
}

// ---------------------------------------------------------------------------
// Head dim 128, n dividing 64: bandwidth-oriented partial kernel.
//   * the workgroup streams its chunk in tiles of 64 cache rows (64/n tokens x
//     n streams) of K and V, 32 KB per tile, copied straight into LDS with
//     direct-to-LDS loads and kept three tiles ahead (4 buffers, 96 KB in
//     flight per CU): the copy engine, not the waves, carries the bytes;
//   * rows of token len come from k_new / v_new (selected per lane, no
//     branches); rows past the chunk re-read its last row and are masked;
//   * wave w scores rows 16w .. 16w+15 of every tile against all n*g query
//     rows (16-row blocks): S^T with v_mfma_f32_16x16x32_bf16, whose
//     accumulator layout is exactly the B operand of v_mfma_f32_16x16x16_bf16
//     for PV (lane l: query l%16, keys 4*(l/16) .. +3), and the V^T operand is
//     one ds_read_b64_tr_b16 (a 16-lane group reads 4 rows x 16 dims).
//   LDS rows are 256 B with the chunk swizzle sw(r) used by the prefill.
constexpr int DT_ROWS = 64;                    // cache rows per tile
constexpr int DT_TILE = DT_ROWS * 128 * 2;     // bytes of one K (or V) tile
constexpr int DT_NBUF = 4;                   // tile buffers: copies run three tiles ahead
static_assert(DT_NBUF >= 2 && DT_NBUF <= 5, "tile buffers");

typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16(bf16x4v a, bf16x4v b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

template <int NQB>
__global__ __launch_bounds__(256, 1) void decode_partial_d128_kernel(DecArgs p, Split sp, float scale_log2) {
    constexpr int D = 128;
    constexpr int TILES_BYTES = DT_NBUF * 2 * DT_TILE;
    constexpr int MERGE_BYTES = NW * NQB * 16 * (2 + D) * 4;
    __shared__ __attribute__((aligned(1024))) char smem[TILES_BYTES > MERGE_BYTES ? TILES_BYTES : MERGE_BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, grp = lane >> 4;
    const int split = blockIdx.x, bh = blockIdx.y;
    const int b = bh / p.Hkv, kvh = bh - b * p.Hkv;
    const int n = p.n, g = p.Hq / p.Hkv, QR = p.nqs * g;
    const int len = p.cache_len[b];
    const int c0 = split * sp.chunk;
    // a length outside [0, T_cap) breaks the caller's contract: no append, no
    // scan (the combine writes NaN rows for that sequence)
    if (len < 0 || len >= p.T_cap) return;
    if (c0 > len) return;  // nothing cached here yet; the combine skips it
    const int c1 = min(c0 + sp.chunk, len + 1);

    const bf16 *kn = static_cast<const bf16 *>(p.k_new);
    const bf16 *vn = static_cast<const bf16 *>(p.v_new);
    bf16 *kc = static_cast<bf16 *>(p.k_cache);
    bf16 *vc = static_cast<bf16 *>(p.v_cache);
    const int64_t hstride = (int64_t)p.Hkv * D;       // elements between streams of one token
    const int64_t cache_tok = (int64_t)n * hstride;   // elements per cached token
    const int64_t cache_b = (int64_t)b * p.T_cap * cache_tok + (int64_t)kvh * D;
    const int64_t new_b = (int64_t)b * n * hstride + (int64_t)kvh * D;

    // Append the new token's rows of this kv head (row len is read by nobody).
    if (len < c1) {
        for (int c = tid; c < n * (D / 8); c += 256) {
            const int s = c / (D / 8), cc = c - s * (D / 8);
            const int64_t src = new_b + (int64_t)s * hstride + cc * 8;
            const int64_t dst = cache_b + (int64_t)len * cache_tok + (int64_t)s * hstride + cc * 8;
            *reinterpret_cast<uint4 *>(kc + dst) = *reinterpret_cast<const uint4 *>(kn + src);
            *reinterpret_cast<uint4 *>(vc + dst) = *reinterpret_cast<const uint4 *>(vn + src);
        }
    }

    // Rows of this chunk inside the window: flat token*n + stream, or (rpt = 1)
    // one row per token, of stream qs0 only.
    const int rpt = p.rpt;
    const int sbase = (rpt == 1) ? p.qs0 : 0;  // stream of a token's first scanned row
    const int tlo = p.window ? max(c0, len - p.window) : c0;
    const int row_lo = tlo * rpt, row_hi = c1 * rpt;
    const int ntiles = row_hi > row_lo ? (row_hi - row_lo + DT_ROWS - 1) / DT_ROWS : 0;

    // Copy-in mapping: wave w, instruction i covers slots (4w+i)*64 .. +63 of
    // the tile (slot = row*16 + physical chunk); rpt divides 64, so the row's
    // token offset and stream are fixed per lane.
    int ltok[4], lstream[4], lchunk[4], lrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (wave * 4 + i) * 4 + (lane >> 4);
        lrow[i] = r;
        ltok[i] = r / rpt;
        lstream[i] = sbase + r - ltok[i] * rpt;
        lchunk[i] = ((lane & 15) ^ swz128(r)) * 8;
    }
    const int tok_per_tile = DT_ROWS / rpt;
    auto issue = [&](int t) {
        char *dst = smem + (t % DT_NBUF) * 2 * DT_TILE;
        const int tok0 = tlo + t * tok_per_tile;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int tok = tok0 + ltok[i];
            const int last = (row_hi - 1) / rpt;  // rows past the chunk re-read its last row
            const bool past = (tok - tlo) * rpt + (lstream[i] - sbase) >= row_hi - row_lo;
            tok = past ? last : tok;
            const int s = past ? sbase + (row_hi - 1) - last * rpt : lstream[i];
            const int64_t coff = cache_b + (int64_t)tok * cache_tok + (int64_t)s * hstride + lchunk[i];
            const int64_t noff = new_b + (int64_t)s * hstride + lchunk[i];
            const bool is_new = tok >= len;
            const bf16 *ksrc = is_new ? kn + noff : kc + coff;
            const bf16 *vsrc = is_new ? vn + noff : vc + coff;
            const int s0 = (wave * 4 + i) * 64;
            lds_dma16(ksrc, lds_addr(dst + s0 * 16));
            lds_dma16(vsrc, lds_addr(dst + DT_TILE + s0 * 16));
        }
    };
    // Query operands: block qb, lane column l16 is query row c = qb*16 + l16
    // (row c <-> stream qs0 + c / g, head kvh*g + c % g); slots grp hold dims
    // ks*32 + 8*grp .. +7.
    const bf16 *qg = static_cast<const bf16 *>(p.q);
    bf16x8 qop[NQB][D / 32];
    int qstream[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int c = qb * 16 + l16;
        const bool ok = c < QR;
        const int sr = ok ? c / g : 0, hh = ok ? c - sr * g : 0;  // query stream qs0 + sr
        qstream[qb] = p.qs0 + sr;
        const bf16 *qp = qg + (((int64_t)b * p.nqs + sr) * p.Hq + kvh * g + hh) * D + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            const bf16x8 x = *reinterpret_cast<const bf16x8 *>(qp + ks * 32);
            qop[qb][ks] = ok ? x : bf16x8{};
        }
    }

    // The append stores and query loads complete before any copy is issued,
    // so the explicit vmcnt waits below count only this wave's tile copies.
    __builtin_amdgcn_s_waitcnt(0);
    for (int t = 0; t < DT_NBUF - 1 && t < ntiles; ++t) issue(t);

    f32x4 oacc[NQB][D / 16];
    float m_run[NQB], l_run[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        m_run[qb] = -INFINITY;
        l_run[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) oacc[qb][db] = f32x4{};
    }

    // This lane's K operand row (16w + l16) and transposed-V row (16w + 4*grp + l16/4).
    const int krow = 16 * wave + l16;
    const int kx = swz128(krow);
    const int vrow = 16 * wave + 4 * grp + (l16 >> 2);
    const int vsw = swz128(vrow);
    const int vhalf = (l16 & 1) * 8;
    const int vc_lo = (l16 & 3) >> 1;
    const int64_t tq_base = (int64_t)len * n;

    for (int t = 0; t < ntiles; ++t) {
        // Tile t has landed; the newer tiles already issued (8 copies each)
        // may stay in flight (gfx9 s_waitcnt immediates).
        const int newer = min(ntiles - 1 - t, DT_NBUF - 2);
        if (newer >= 3) __builtin_amdgcn_s_waitcnt(0x4F78);       // vmcnt(24)
        else if (newer == 2) __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16)
        else if (newer == 1) __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8)
        else __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // ... for every wave; tile t-1 fully consumed
        if (t + DT_NBUF - 1 < ntiles) issue(t + DT_NBUF - 1);
        const char *kbuf = smem + (t % DT_NBUF) * 2 * DT_TILE;
        const char *vbuf = kbuf + DT_TILE;

        bf16x8 kop[D / 32];
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
            kop[ks] = *reinterpret_cast<const bf16x8 *>(kbuf + krow * 256 + (((4 * ks + grp) ^ kx) << 4));
        bf16x4v vop[D / 16];
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
            const s16x4 x = lds_read_tr16(vbuf + vrow * 256 + (((2 * db + vc_lo) ^ vsw) << 4) + vhalf);
            vop[db] = __builtin_bit_cast(bf16x4v, x);
        }

        const int rtile = row_lo + t * DT_ROWS + 16 * wave + 4 * grp;  // this lane's first key row
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            f32x4 sacc = {};
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) sacc = mfma16(kop[ks], qop[qb][ks], sacc);
            const int sq = qstream[qb];
            const int64_t tq = tq_base + sq;
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = rtile + i;
                const int tok = r / rpt;
                const int sk = sbase + r - tok * rpt;
                bool vis = r < row_hi;
                if (p.mode == 0) vis = vis && sk == sq && (p.window == 0 || len - tok < p.window);
                else vis = vis && r <= tq && (p.window == 0 || tq - r < (int64_t)n * p.window);
                sacc[i] = vis ? sacc[i] : -INFINITY;
                mx = fmaxf(mx, sacc[i]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_tile = mx * scale_log2;
            const float m_new = (m_tile > m_run[qb] + 8.f) ? m_tile : m_run[qb];
            const float alpha = (m_new == m_run[qb]) ? 1.f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
            const float neg_m = (m_new == -INFINITY) ? 0.f : -m_new;
            bf16x4v pop;
            float lsum = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[i], scale_log2, neg_m));
                lsum += pv;
                pop[i] = (bf16)pv;
            }
            if (__ballot(alpha != 1.f)) {
#pragma unroll
                for (int db = 0; db < D / 16; ++db) oacc[qb][db] *= alpha;
            }
            l_run[qb] = l_run[qb] * alpha + lsum;
            m_run[qb] = m_new;
#pragma unroll
            for (int db = 0; db < D / 16; ++db) oacc[qb][db] = mfma16x16(vop[db], pop, oacc[qb][db]);
        }
    }
    __syncthreads();  // tile buffers are reused for the merge below

    float *ml = reinterpret_cast<float *>(smem);  // [4][NQB*16][2]
    float *ow = ml + NW * NQB * 16 * 2;           // [4][NQB*16][D]
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        float lt = l_run[qb];
        lt += __shfl_xor(lt, 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        const int c = qb * 16 + l16;
        if (grp == 0) {
            ml[(wave * NQB * 16 + c) * 2 + 0] = m_run[qb];
            ml[(wave * NQB * 16 + c) * 2 + 1] = lt;
        }
#pragma unroll
        for (int db = 0; db < D / 16; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) ow[(wave * NQB * 16 + c) * D + db * 16 + 4 * grp + i] = oacc[qb][db][i];
    }
    __syncthreads();
    const int64_t part = ((int64_t)bh * sp.nsplit + split) * QR;
    float *ws_acc = p.ws;
    float *ws_ml = p.ws + (int64_t)p.B * p.Hkv * sp.nsplit * QR * D;
    for (int e = tid; e < QR * D; e += 256) {
        const int c = e / D, dim = e - c * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, ml[(w * NQB * 16 + c) * 2]);
        const float Mu = (M == -INFINITY) ? 0.f : M;
        float acc = 0.f, L = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float wt = __builtin_amdgcn_exp2f(ml[(w * NQB * 16 + c) * 2] - Mu);
            acc += wt * ow[(w * NQB * 16 + c) * D + dim];
            L += wt * ml[(w * NQB * 16 + c) * 2 + 1];
        }
        ws_acc[(part + c) * D + dim] = acc;
        if (dim == 0) {
            ws_ml[(part + c) * 2 + 0] = M;
            ws_ml[(part + c) * 2 + 1] = L;
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecArgs p, Split sp) {
    const int lane = threadIdx.x & 63;
    const int g = p.Hq / p.Hkv, QR = p.nqs * g;
    const int64_t row = (int64_t)blockIdx.x * NW + (threadIdx.x >> 6);  // (bh, c)
    if (row >= (int64_t)p.B * p.Hkv * QR) return;
    const int c = (int)(row % QR);
    const int bh = (int)(row / QR);
    const int b = bh / p.Hkv, kvh = bh - b * p.Hkv;
    const int len = p.cache_len[b];
    const int sr = c / g, hh = c - sr * g;  // query stream qs0 + sr
    bf16 *op = static_cast<bf16 *>(p.o) + (((int64_t)b * p.nqs + sr) * p.Hq + kvh * g + hh) * D;
    constexpr int PER = (D + 63) / 64;
    if (len < 0 || len >= p.T_cap) {  // contract violation: no partial was written
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int dim = lane + 64 * e;
            if (dim < D) reinterpret_cast<unsigned short *>(op)[dim] = 0x7fc0;  // bf16 quiet NaN
        }
        return;
    }
    const int ns = min(sp.nsplit, len / sp.chunk + 1);  // splits with c0 <= len
    const float *ws_acc = p.ws;
    const float *ws_ml = p.ws + (int64_t)p.B * p.Hkv * sp.nsplit * QR * D;
    const int64_t part0 = (int64_t)bh * sp.nsplit * QR + c;

    float M = -INFINITY;
    for (int k = 0; k < ns; ++k) M = fmaxf(M, ws_ml[(part0 + (int64_t)k * QR) * 2]);
    float acc[PER] = {};
    float L = 0.f;
    for (int k = 0; k < ns; ++k) {
        const int64_t pk = part0 + (int64_t)k * QR;
        const float wt = __builtin_amdgcn_exp2f(ws_ml[pk * 2] - M);
        L += wt * ws_ml[pk * 2 + 1];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int dim = lane + 64 * e;
            if (dim < D) acc[e] += wt * ws_acc[pk * D + dim];
        }
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int dim = lane + 64 * e;
        if (dim < D) op[dim] = (bf16)(acc[e] * inv);
    }
}

template <int D, int NQB>
hipError_t launch_partial(const DecArgs &a, Split sp, float sl2, hipStream_t st) {
    constexpr int VP = D + 8;
    const size_t stage = (size_t)NW * RB * VP * sizeof(bf16);
    const size_t merge = (size_t)NW * NQB * 16 * (2 + D) * sizeof(float);
    const size_t lds = stage > merge ? stage : merge;
    if (lds > 65536) {  // above the default dynamic-LDS limit: opt in once
        static bool raised = false;
        if (!raised) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&decode_partial_kernel<D, NQB>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            raised = true;
        }
    }
    hipLaunchKernelGGL((decode_partial_kernel<D, NQB>), dim3(sp.nsplit, a.B * a.Hkv), dim3(256), lds, st, a,
                       sp, sl2);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecArgs &a, Split sp, float sl2, hipStream_t st) {
    const int QR = a.nqs * (a.Hq / a.Hkv);
    hipError_t e;
    switch ((QR + 15) / 16) {
        case 1: e = launch_partial<D, 1>(a, sp, sl2, st); break;
        case 2: e = launch_partial<D, 2>(a, sp, sl2, st); break;
        case 3: e = launch_partial<D, 3>(a, sp, sl2, st); break;
        case 4: e = launch_partial<D, 4>(a, sp, sl2, st); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)a.B * a.Hkv * QR;
    hipLaunchKernelGGL(decode_combine_kernel<D>, dim3((unsigned)((rows + NW - 1) / NW)), dim3(256), 0, st, a, sp);
    return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int B, int n, int Hq, int Hkv, int d, int T_cap) {
    const Split sp = use_d128_path(n, d) ? choose_split_d128(B, Hkv, T_cap) : choose_split(B, Hkv, T_cap);
    return (size_t)B * n * Hq * sp.nsplit * (size_t)(d + 2) * sizeof(float);
}

template <int NQB>
hipError_t launch_partial_d128(const DecArgs &a, Split sp, float sl2, hipStream_t st) {
    hipLaunchKernelGGL((decode_partial_d128_kernel<NQB>), dim3(sp.nsplit, a.B * a.Hkv), dim3(256), 0, st, a, sp,
                       sl2);
    return hipGetLastError();
}

hipError_t launch_sfa_decode_bf16(const DecArgs &a, hipStream_t st) {
    const float sl2 = a.scale * kLog2e;
    if (use_d128_path(a.n, a.d)) {
        // a scan of one stream's rows (rpt = 1 of n) reads 1/n of the bytes
        // per token: fewer, longer chunks (sweep: B=64, ctx 8192, final-stream
        // intra decode 0.371 ms at 1024 workgroups, 0.357 ms at 512)
        const Split sp = choose_split_d128(a.B, a.Hkv, a.T_cap, std::max(1, kDecodeTargetWgs * a.rpt / a.n));
        const int QR = a.nqs * (a.Hq / a.Hkv);
        hipError_t e;
        switch ((QR + 15) / 16) {
            case 1: e = launch_partial_d128<1>(a, sp, sl2, st); break;
            case 2: e = launch_partial_d128<2>(a, sp, sl2, st); break;
            case 3: e = launch_partial_d128<3>(a, sp, sl2, st); break;
            case 4: e = launch_partial_d128<4>(a, sp, sl2, st); break;
            default: return hipErrorInvalidValue;
        }
        if (e != hipSuccess) return e;
        const int64_t rows = (int64_t)a.B * a.Hkv * QR;
        hipLaunchKernelGGL(decode_combine_kernel<128>, dim3((unsigned)((rows + NW - 1) / NW)), dim3(256), 0, st, a,
                           sp);
        return hipGetLastError();
    }
    const Split sp = choose_split(a.B, a.Hkv, a.T_cap);
    switch (a.d) {
        case 32: return launch_d<32>(a, sp, sl2, st);
        case 64: return launch_d<64>(a, sp, sl2, st);
        case 128: return launch_d<128>(a, sp, sl2, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace hd
