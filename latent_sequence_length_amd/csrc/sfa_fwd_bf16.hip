// sfa_fwd_bf16.hip -- Stream-Factorized Attention prefill, bf16 in / fp32
// accumulate, on gfx950 matrix cores.
//
// The method ("Hidden Decoding at Scale", "Stream-Factorized Attention",
// Figure 2): intra-stream layers attend causally within a stream only, cross-
// stream layers causally over the whole expanded sequence, each optionally in
// a sliding window.  Both are run here as causal attention over a strided
// sub-sequence (see FwdArgs): for intra, the keys of stream s are rows
// s, s+n, s+2n, ... of K/V, gathered by address arithmetic into LDS tiles, so
// no mask tensor exists and no tile of another stream is ever loaded.
//
// Work decomposition
//   workgroup = 4 wavefronts = one kv head, HG query heads of its GQA group x
//               TB blocks of 32 consecutive sub-sequence queries (HG*TB = 4);
//               the K/V tile in LDS is shared by all four waves.
//   wave      = 32 queries of one head.
//   tile      = 64 keys.
// Per tile each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (two
// 32-key blocks), so lane l owns query (l % 32) and 16 keys of each block: the
// online-softmax row state (max, sum) lives in one lane pair (l, l^32).  Then
// O^T += V^T P^T with the same instruction; P^T comes straight out of the S^T
// accumulator registers (no LDS round trip) and O^T keeps every accumulator
// of a lane on that lane's own query, so the rescale is one scalar per lane.
//
// Operand layouts of the 32x32x16 bf16 instruction used below: lane l supplies
// row (l % 32) of A (column of B) and eight consecutive k-slots of half
// (l / 32); A and B pair k-slots identically, so any consistent assignment of
// real k indices to slots is a valid contraction.  The accumulator holds
// C[8*(r/4) + 4*(l/32) + (r%4)][l % 32] in register r.
#include "attn_common.h"

namespace hd {

namespace {

constexpr int KT = 64;   // keys per tile
constexpr int QW = 32;   // queries per wave
constexpr int NWAVE = 4;

__device__ __forceinline__ float wave_xor32(float x) {
    return __shfl_xor(x, 32, 64);
}

template <int D>
__global__ __launch_bounds__(256) void sfa_fwd_bf16_kernel(FwdArgs p, int HG, int TB, int nqblk,
                                                           float scale_log2) {
    constexpr int KP = D + 8;  // LDS row pitch (elements): 16-byte pad per row
    __shared__ __attribute__((aligned(16))) bf16 Ks[KT * KP];
    __shared__ __attribute__((aligned(16))) bf16 Vs[KT * KP];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int g = p.Hq / p.Hkv, ngrp = g / HG;

    // Workgroup -> (q block, b, kv head, head group, sub-sequence).  The last
    // (longest) query blocks are dispatched first.
    const int nrest = p.B * p.Hkv * ngrp * p.nsub;
    const int qblk = nqblk - 1 - (int)(blockIdx.x / nrest);
    int rest = (int)(blockIdx.x % nrest);
    const int sub = rest % p.nsub; rest /= p.nsub;
    const int hgrp = rest % ngrp; rest /= ngrp;
    const int kvh = rest % p.Hkv;
    const int b = rest / p.Hkv;

    const int QB = QW * TB;
    const int q0 = qblk * QB;
    const int hw = wave % HG, tb = wave / HG;
    const int h = kvh * g + hgrp * HG + hw;
    const int qw0 = q0 + tb * QW;       // first query of this wave
    const int myq = qw0 + l32;          // this lane's query (sub-sequence index)
    const bool qvalid = myq < p.Lq;
    const int mylim = myq * p.qmul + p.qadd;                      // last key this query may see
    const int lim0 = qw0 * p.qmul + p.qadd;                       // ... for the wave's first query
    const int lim1 = (qw0 + QW - 1) * p.qmul + p.qadd;            // ... and its last

    const int64_t qrs = (int64_t)p.Hq * D;   // elements between positions (Q, O)
    const int64_t krs = (int64_t)p.Hkv * D;  // elements between positions (K, V)
    const int64_t bpos = (int64_t)b * p.nL + p.kbase + sub;       // key element 0
    const int64_t qbase = (int64_t)b * p.qrows + (int64_t)sub * p.qsub;  // query 0's Q row
    const bf16 *qg = static_cast<const bf16 *>(p.q);
    const bf16 *kg = static_cast<const bf16 *>(p.k);
    const bf16 *vg = static_cast<const bf16 *>(p.v);

    // Q^T operand, resident for the whole loop: slot half hi of k-step ks
    // holds dims ks*16 + 8*hi .. +7 of this lane's query.
    bf16x8 qop[D / 16];
    {
        const bf16 *qp = qg + (qbase + (int64_t)(qvalid ? myq : 0) * p.qstride) * qrs + (int64_t)h * D;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            bf16x8 x = *reinterpret_cast<const bf16x8 *>(qp + ks * 16 + 8 * hi);
            qop[ks] = qvalid ? x : bf16x8{};
        }
        if (p.rope) rope_rotate_q<D>(qop, p.kbase + sub + (int64_t)mylim * p.stride, p.rope_ft, hi);
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    const int kend = min((min(q0 + QB, p.Lq) - 1) * p.qmul + p.qadd + 1, p.Lsub);
    const int kbeg = p.weff ? max(0, q0 * p.qmul + p.qadd - p.weff + 1) : 0;
    constexpr int CH = D / 8;  // 16-byte chunks per row

    for (int t0 = kbeg & ~(KT - 1); t0 < kend; t0 += KT) {
        __syncthreads();  // previous tile fully consumed
        for (int c = tid; c < KT * CH; c += 256) {
            const int r = c / CH, cc = c - r * CH;
            const int j = t0 + r;
            uint4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
            if (j < p.Lsub) {
                const int64_t off = (bpos + (int64_t)j * p.stride) * krs + (int64_t)kvh * D + cc * 8;
                kx = *reinterpret_cast<const uint4 *>(kg + off);
                vx = *reinterpret_cast<const uint4 *>(vg + off);
            }
            *reinterpret_cast<uint4 *>(&Ks[r * KP + cc * 8]) = kx;
            *reinterpret_cast<uint4 *>(&Vs[r * KP + cc * 8]) = vx;
        }
        __syncthreads();

        // Skip tiles wholly outside this wave's causal / window band.
        const bool active = (t0 <= lim1) && (p.weff == 0 || t0 + KT - 1 > lim0 - p.weff);
        if (!active) continue;
        const bool need_mask = (t0 + KT - 1 > lim0) || (t0 + KT > p.Lsub) ||
                               (p.weff != 0 && t0 <= lim1 - p.weff);

        // S^T = K Q^T for two 32-key blocks.
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sacc[kb] = f32x16{};
            const bf16 *kr = &Ks[(kb * 32 + l32) * KP + 8 * hi];
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks)
                sacc[kb] = mfma32(*reinterpret_cast<const bf16x8 *>(kr + ks * 16), qop[ks], sacc[kb]);
        }

        // Scale to log2 units, mask (visible <=> lo <= key <= hi_key, one
        // unsigned compare and a select per score), tile max.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][r] *= scale_log2;
        if (need_mask) {  // uniform: only tiles on the band edges
            const int lo = p.weff ? mylim - p.weff + 1 : 0;
            const unsigned span = (unsigned)(min(mylim, p.Lsub - 1) - lo);
            const int base = t0 + 4 * hi - lo;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const unsigned u = (unsigned)(base + kb * 32 + 8 * (r >> 2) + (r & 3));
                    sacc[kb][r] = (u <= span) ? sacc[kb][r] : -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
        mx = fmaxf(mx, wave_xor32(mx));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pv = __builtin_amdgcn_exp2f(sacc[kb][r] - m_use);
                sacc[kb][r] = pv;
                lsum += pv;
            }
        l_run = l_run * alpha + lsum;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;

        // O^T += V^T P^T.  PV step (kb, m2) contracts the 16 keys held in
        // registers 8*m2 .. 8*m2+7 of block kb: slot j <-> key
        // kb*32 + 16*m2 + 8*(j/4) + 4*hi + (j%4).
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2) {
                bf16x8 pop;
#pragma unroll
                for (int j = 0; j < 8; ++j) pop[j] = (bf16)sacc[kb][8 * m2 + j];
                const int kbase = kb * 32 + 16 * m2 + 4 * hi;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    bf16x8 vop;
                    const bf16 *vc = &Vs[db * 32 + l32];
#pragma unroll
                    for (int j = 0; j < 8; ++j) vop[j] = vc[(kbase + 8 * (j >> 2) + (j & 3)) * KP];
                    oacc[db] = mfma32(vop, pop, oacc[db]);
                }
            }
    }

    // Epilogue: combine the lane pair's partial sums, normalise, store.
    const float l_tot = l_run + wave_xor32(l_run);
    if (qvalid) {
        const float inv = 1.f / l_tot;
        const int64_t qrow = qbase + (int64_t)myq * p.qstride;
        bf16 *op = static_cast<bf16 *>(p.o) + qrow * qrs + (int64_t)h * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                bf16x4 y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = (bf16)(oacc[db][4 * r4 + e] * inv);
                *reinterpret_cast<bf16x4 *>(op + db * 32 + 8 * r4 + 4 * hi) = y;
            }
        if (p.lse != nullptr && hi == 0)
            p.lse[((int64_t)b * p.Hq + h) * p.qrows + (qrow - (int64_t)b * p.qrows)] =
                m_run * kLn2 + __logf(l_tot);
    }
}


// ---------------------------------------------------------------------------
// Head dim 128 fast path.  Same math as above, with these changes:
//   * a workgroup is 8 waves (HG heads x 8/HG blocks of 32 positions), two
//     per SIMD and one workgroup per CU, so every K/V tile copied into LDS
//     serves 256 query rows (half the L2-to-LDS traffic of 4-wave groups);
//   * each wave raises its issue priority while it issues the QK^T MFMAs, so
//     the other wave of its SIMD fills the matrix core's gaps with its own
//     softmax and PV rather than competing for it;
//   * K and V tiles are fetched with direct-to-LDS 16-byte loads
//     (global_load_lds), double-buffered: tile t+1 is in flight while tile t
//     is computed, with no VGRPs spent on staging and one barrier per tile;
//     the tile base is a scalar and each lane's offset is fixed, so issuing a
//     copy costs no vector ALU work;
//   * the QK^T MFMAs run as two interleaved accumulator chains with the K
//     operand reads scheduled eight ahead;
//   * LDS rows are 256 B with the 16-byte chunk index XOR-swizzled by the row
//     (sw(r) = 2*(r%8) + (r/8)%2), so the K-operand reads (16 rows, one chunk)
//     and the transposed V reads (8 rows, four chunks) are bank-conflict free;
//   * the V^T operand comes from two ds_read_b64_tr_b16 per MFMA: within each
//     16-lane group that instruction returns out[i][e] = in[4e + i/4][i%4],
//     so lane j of the group addresses key row r0 + j/4, dims d0 + 4*(j%4);
//   * softmax: the scale is folded into one fma before exp2; a tile's
//     probabilities are taken against the running max as it stands and kept
//     when every lane's share of its row sum stays <= 2^32 (no probability
//     exceeds 2^32: harmless for fp32 sums and for bf16 P, whose relative
//     precision does not depend on magnitude); otherwise, and on the first
//     tile, the wave takes the tile max, rescales O and l and recomputes.
//     The common tile needs no max, no rescale test and no O rescale; the
//     final normalisation is unchanged;
//   * workgroups are ordered so each XCD (round-robin dispatch) walks whole
//     (batch, kv head, stream) groups, keeping that group's K/V in its L2.
constexpr int D128_NW = 8;  // waves per workgroup of the head-dim-128 kernel


// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgMfma = 0x008, kSgDsRead = 0x100;

// One tile of the d=128 loop: wait for tile `it` (in buffer `cur`), start
// the DMA of tile it+1 into `nxt`, then compute tile `it`.  `cur` and `nxt`
// are distinct __shared__ arrays known at compile time, so the compiler can
// tell the in-flight DMA and this tile's LDS reads apart.
struct D128State {
    f32x16 oacc[4];
    float m_run, l_run;
};

template <typename Issue>
__device__ __forceinline__ void d128_tile(const char *__restrict__ cur, Issue &&issue_next, bool has_next,
                                          int t0, const FwdArgs &p, int lim0, int lim1, int mylim, int hi, int l32,
                                          int l16, int g2, const bf16x8 (&qop)[8], float scale_log2,
                                          D128State &st) {
    constexpr int D = 128;
    constexpr int TILE = KT * D * 2;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the tile have landed
    __syncthreads();                // ... and every wave's; the previous tile is fully consumed
    if (has_next) issue_next();

    const bool active = (t0 <= lim1) && (p.weff == 0 || t0 + KT - 1 > lim0 - p.weff);
    if (!active) return;
    const bool need_mask = (t0 + KT - 1 > lim0) || (t0 + KT > p.Lsub) || (p.weff != 0 && t0 <= lim1 - p.weff);
    const char *kbuf = cur;
    const char *vbuf = cur + TILE;

    f32x16 sacc[2];
    __builtin_amdgcn_s_setprio(1);  // the wave issuing MFMAs wins arbitration on its SIMD
    // two independent 32-key accumulator chains, interleaved; the K-operand
    // reads are scheduled eight ahead of the MFMAs that consume them
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sacc[kb] = f32x16{};
    const int ksw = swz128(l32) ^ hi;  // swz128(32*kb + l32) == swz128(l32); 2*ks + hi == (2*ks) ^ hi
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kbuf + (kb * 32 + l32) * 256 + (((2 * ks) ^ ksw) << 4));
            sacc[kb] = mfma32(a, qop[ks], sacc[kb]);
        }
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 8, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 8, 0);
    __builtin_amdgcn_sched_barrier(0);

    __builtin_amdgcn_s_setprio(0);
    if (need_mask) {
        // visible <=> lo <= key <= hi, checked as one unsigned compare
        const int lo = p.weff ? mylim - p.weff + 1 : 0;
        const int hi_key = min(mylim, p.Lsub - 1);
        const unsigned span = (unsigned)(hi_key - lo);
        const int base = t0 + 4 * hi - lo;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const unsigned u = (unsigned)(base + kb * 32 + 8 * (r >> 2) + (r & 3));
                sacc[kb][r] = (u <= span) ? sacc[kb][r] : -INFINITY;
            }
    }
    // Probabilities against the running max; the tile is accepted as is when
    // every lane's share of its row sum stays <= 2^32 (so no probability
    // exceeds it), else -- and while some row has no max yet -- the wave
    // raises every row's max to the tile's, rescales and recomputes.
    bf16x8 pop[4];
    float lsum = 0.f;
    auto probs = [&](float neg_m) {
        lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2) {
                bf16x8 pp;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    pp[j] = (bf16)__builtin_amdgcn_exp2f(fmaf(sacc[kb][8 * m2 + j], scale_log2, neg_m));
                lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pp, pp, 0, 1), kOnes2, lsum, false);
                lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pp, pp, 2, 3), kOnes2, lsum, false);
                lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pp, pp, 4, 5), kOnes2, lsum, false);
                lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pp, pp, 6, 7), kOnes2, lsum, false);
                pop[kb * 2 + m2] = pp;
            }
    };
    bool slow = true;
    if (!__ballot(st.m_run == -INFINITY)) {
        probs(-st.m_run);
        slow = __ballot(!(lsum <= 4294967296.f)) != 0;  // also catches inf / NaN
    }
    if (slow) {
        float m0 = fmaxf(sacc[0][0], sacc[0][1]), m1 = fmaxf(sacc[1][0], sacc[1][1]);
#pragma unroll
        for (int r = 2; r < 16; r += 2) {
            m0 = fmaxf(m0, fmaxf(sacc[0][r], sacc[0][r + 1]));
            m1 = fmaxf(m1, fmaxf(sacc[1][r], sacc[1][r + 1]));
        }
        const float m_tile = pair_max(fmaxf(m0, m1)) * scale_log2;
        const float m_new = fmaxf(st.m_run, m_tile);
        const float alpha = (m_new == st.m_run) ? 1.f : __builtin_amdgcn_exp2f(st.m_run - m_new);
        if (__ballot(alpha != 1.f)) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db) st.oacc[db] *= alpha;
        }
        st.l_run *= alpha;
        st.m_run = m_new;
        probs((m_new == -INFINITY) ? 0.f : -m_new);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                s16x4 half[2];
#pragma unroll
                for (int jh = 0; jh < 2; ++jh) {
                    const int row = kb * 32 + 16 * m2 + 8 * jh + 4 * hi + (l16 >> 2);
                    const int dim = db * 32 + 16 * g2 + 4 * (l16 & 3);
                    const char *addr = vbuf + row * 256 + (((dim >> 3) ^ swzv(row)) << 4) + ((dim >> 2) & 1) * 8;
                    half[jh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4 *)(addr));
                }
                const s16x8 both = __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
                st.oacc[db] = mfma32(__builtin_bit_cast(bf16x8, both), pop[kb * 2 + m2], st.oacc[db]);
            }
        }
    // the 32 transposed V reads run eight ahead of the 16 PV MFMAs, two per
    // MFMA after that (measured best of 4..16 ahead: -2% on every layer)
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 8, 0);
#pragma unroll
    for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
    st.l_run += lsum;
}

// GQ: the query map is not the identity (qmul, qadd) != (1, 0); a full layer
// runs the GQ = false instance, whose band tests are the plain p <= j ones.
// ROPE: q is rotated at its expanded position right after the load.
template <bool GQ, bool ROPE>
__global__ __launch_bounds__(64 * D128_NW, 1) void sfa_fwd_bf16_d128_kernel(FwdArgs p, int HG, int TB, int nqblk,
                                                                  float scale_log2) {
    constexpr int D = 128;
    constexpr int TILE = KT * D * 2;  // 16 KB per K or V tile
    __shared__ __attribute__((aligned(1024))) char buf0[2 * TILE];  // K | V, even tiles
    __shared__ __attribute__((aligned(1024))) char buf1[2 * TILE];  // K | V, odd tiles

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5, l16 = lane & 15, g2 = (lane >> 4) & 1;
    const int g = p.Hq / p.Hkv, ngrp = g / HG;

    // Workgroup -> (query block, group).  Dispatch is round-robin over the 8
    // XCDs (XCD bid % 8 runs its workgroups in bid order); the map keeps each
    // XCD's share balanced (longest blocks first) and its groups few:
    // whole groups per XCD when the group count is a multiple of 8 (the
    // XCD's groups interleaved, so its longest blocks of every group run
    // first), each group spread over 8/G XCDs when G divides 8, else
    // round-robin.
    const int nrest = p.B * p.Hkv * ngrp * p.nsub;
    const int nwg = nrest * nqblk;
    const int bid = blockIdx.x;
    int lid = bid;
    if (nwg % 8 == 0) {
        const int x = bid % 8, j = bid / 8;
        if (nrest % 8 == 0) {
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
    const int hw = wave % HG, tb = wave / HG;
    const int h = kvh * g + hgrp * HG + hw;
    const int qw0 = q0 + tb * QW;
    const int myq = qw0 + l32;
    const bool qvalid = myq < p.Lq;
    const int qmul = GQ ? p.qmul : 1, qadd = GQ ? p.qadd : 0;
    const int mylim = myq * qmul + qadd;            // last key this query may see
    const int lim0 = qw0 * qmul + qadd;             // ... for the wave's first query
    const int lim1 = (qw0 + QW - 1) * qmul + qadd;  // ... and its last

    const int64_t qrs = (int64_t)p.Hq * D;
    const int64_t krs = (int64_t)p.Hkv * D;
    const int64_t bpos = (int64_t)b * p.nL + p.kbase + sub;              // key element 0
    const int64_t qbase = (int64_t)b * p.qrows + (int64_t)sub * p.qsub;  // query 0's Q row
    const bf16 *qg = static_cast<const bf16 *>(p.q);
    const bf16 *kg = static_cast<const bf16 *>(p.k) + (int64_t)kvh * D;
    const bf16 *vg = static_cast<const bf16 *>(p.v) + (int64_t)kvh * D;

    const int kend = min((min(q0 + QB, p.Lq) - 1) * qmul + qadd + 1, p.Lsub);
    const int kbeg = p.weff ? max(0, q0 * qmul + qadd - p.weff + 1) : 0;
    const int tfirst = kbeg & ~(KT - 1);
    const int ntiles = (kend - tfirst + KT - 1) / KT;

    // Each wave moves 4 x 1 KB of K and of V per tile: slots w*256 .. +255,
    // slot s = row*16 + physical chunk; lane l of instruction i fills slot
    // (w*4+i)*64 + l with logical chunk (s%16) ^ sw(row).  Rows past the end
    // of the sub-sequence re-read its last row (finite data, masked later).
    const int rstride = p.stride * (int)krs;  // elements between sub-sequence rows
    constexpr int PER = 16 / D128_NW;  // 1 KB copies of K (and of V) per wave per tile
    int lrow[PER], lchunk[PER], lchunkv[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        lrow[i] = (wave * PER + i) * 4 + (lane >> 4);
        lchunk[i] = ((lane & 15) ^ swz128(lrow[i])) * 8;
        lchunkv[i] = ((lane & 15) ^ swzv(lrow[i])) * 8;
    }
    unsigned boff[PER], boffv[PER];  // per-lane byte offsets of K / V within a tile (rows unclamped)
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        boff[i] = (unsigned)(lrow[i] * rstride + lchunk[i]) * 2u;
        boffv[i] = (unsigned)(lrow[i] * rstride + lchunkv[i]) * 2u;
    }
    auto issue = [&](int t0, char *dst) {
        const int64_t tbase = (bpos + (int64_t)t0 * p.stride) * krs;
        const bf16 *kt = kg + tbase, *vt = vg + tbase;
        const int rmax = p.Lsub - 1 - t0;
        unsigned bo[PER], bv[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) { bo[i] = boff[i]; bv[i] = boffv[i]; }
        if (rmax < KT - 1) {  // tail tile: rows past the end re-read the last row
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                bo[i] = (unsigned)(min(lrow[i], rmax) * rstride + lchunk[i]) * 2u;
                bv[i] = (unsigned)(min(lrow[i], rmax) * rstride + lchunkv[i]) * 2u;
            }
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int s0 = (wave * PER + i) * 64;
            lds_dma16_s(kt, bo[i], lds_addr(dst + s0 * 16));
            lds_dma16_s(vt, bv[i], lds_addr(dst + TILE + s0 * 16));
        }
    };
    if (ntiles > 0) issue(tfirst, buf0);

    bf16x8 qop[D / 16];
    {
        const bf16 *qp = qg + (qbase + (int64_t)(qvalid ? myq : 0) * p.qstride) * qrs + (int64_t)h * D;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            bf16x8 x = *reinterpret_cast<const bf16x8 *>(qp + ks * 16 + 8 * hi);
            qop[ks] = qvalid ? x : bf16x8{};
        }
        // expanded position of the query: key element lim(p) of this sub-sequence
        if (ROPE) rope_rotate_q<D>(qop, p.kbase + sub + (int64_t)mylim * p.stride, p.rope_ft, hi);
    }

    D128State st;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) st.oacc[db] = f32x16{};
    st.m_run = -INFINITY;
    st.l_run = 0.f;

    for (int it = 0; it < ntiles; it += 2) {
        const int t0 = tfirst + it * KT;
        d128_tile(buf0, [&] { issue(t0 + KT, buf1); }, it + 1 < ntiles, t0, p, lim0, lim1, mylim, hi, l32, l16, g2,
                  qop, scale_log2, st);
        if (it + 1 < ntiles)
            d128_tile(buf1, [&] { issue(t0 + 2 * KT, buf0); }, it + 2 < ntiles, t0 + KT, p, lim0, lim1, mylim, hi,
                      l32, l16, g2, qop, scale_log2, st);
    }

    const float l_tot = pair_sum(st.l_run);
    if (qvalid) {
        const float inv = 1.f / l_tot;
        const int64_t qrow = qbase + (int64_t)myq * p.qstride;
        bf16 *op = static_cast<bf16 *>(p.o) + qrow * qrs + (int64_t)h * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                bf16x4 y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = (bf16)(st.oacc[db][4 * r4 + e] * inv);
                *reinterpret_cast<bf16x4 *>(op + db * 32 + 8 * r4 + 4 * hi) = y;
            }
        if (p.lse != nullptr && hi == 0)
            p.lse[((int64_t)b * p.Hq + h) * p.qrows + (qrow - (int64_t)b * p.qrows)] =
                st.m_run * kLn2 + __logf(l_tot);
    }
}

}  // namespace

hipError_t launch_sfa_fwd_bf16(const FwdArgs &a, hipStream_t st) {
    const int g = a.Hq / a.Hkv;
    const int HG = (g % 4 == 0) ? 4 : (g % 2 == 0) ? 2 : 1;
    const int TB = NWAVE / HG;
    const int nqblk = (a.Lq + QW * TB - 1) / (QW * TB);
    const int64_t grid = (int64_t)nqblk * a.B * a.Hkv * (g / HG) * a.nsub;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    const float sl2 = a.scale * kLog2e;
    switch (a.d) {
        case 32:
            hipLaunchKernelGGL(sfa_fwd_bf16_kernel<32>, dim3((unsigned)grid), dim3(256), 0, st, a, HG, TB, nqblk, sl2);
            break;
        case 64:
            hipLaunchKernelGGL(sfa_fwd_bf16_kernel<64>, dim3((unsigned)grid), dim3(256), 0, st, a, HG, TB, nqblk, sl2);
            break;
        case 128:
            if ((int64_t)KT * a.stride * a.Hkv * 128 >= (int64_t)1 << 31) {  // 32-bit copy offsets
                hipLaunchKernelGGL(sfa_fwd_bf16_kernel<128>, dim3((unsigned)grid), dim3(256), 0, st, a, HG, TB, nqblk,
                                   sl2);
                break;
            }
            {
                const int TB2 = D128_NW / HG;
                const int nqblk2 = (a.Lq + QW * TB2 - 1) / (QW * TB2);
                const int64_t grid2 = (int64_t)nqblk2 * a.B * a.Hkv * (g / HG) * a.nsub;
                if (grid2 > 0x7fffffff) return hipErrorInvalidConfiguration;
                const bool gq = a.qmul != 1 || a.qadd != 0;
                auto kern = gq ? (a.rope ? sfa_fwd_bf16_d128_kernel<true, true> : sfa_fwd_bf16_d128_kernel<true, false>)
                               : (a.rope ? sfa_fwd_bf16_d128_kernel<false, true> : sfa_fwd_bf16_d128_kernel<false, false>);
                hipLaunchKernelGGL(kern, dim3((unsigned)grid2), dim3(64 * D128_NW), 0, st, a, HG, TB2, nqblk2, sl2);
            }
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace hd
