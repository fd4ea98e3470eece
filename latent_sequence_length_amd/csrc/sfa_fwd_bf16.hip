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
#include "sfa_fwd_d128_loop.inc"

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
//   * a workgroup is 4 waves, one per SIMD and one workgroup per CU; a wave
//     holds 64 queries of one head (two 32-query halves), the workgroup HG
//     heads x 4/HG blocks of 64 positions, so every K/V tile copied into LDS
//     serves 256 query rows, and every K or V^T fragment a wave reads from
//     LDS feeds two MFMAs (one per half): half the LDS operand traffic of
//     32-query waves.  O^T of both halves (128 accumulators) lives in AGPRs,
//     the scores, probabilities and Q in VGPRs (an MFMA whose A or B operand
//     is an AGPR gains nothing here, and accumulators in AGPRs cost nothing);
//   * the key loop is one hand-ordered instruction stream (see
//     gen_fwd_d128_loop.py): per 32-key sub-tile i, the QK^T MFMAs of i, the
//     softmax of i-1 and the PV MFMAs of i-2, the softmax's vector ops placed
//     one by one between the MFMAs so that the vector ALU and the matrix core
//     of the SIMD work at the same time inside the one wave;
//   * K and V tiles are fetched with direct-to-LDS 16-byte loads
//     (global_load_lds) into three-deep rings, one barrier per tile: K of
//     tile t+2 and V of tile t+1 are copied while tile t is computed, so a
//     tile's first operand reads can be issued before its barrier; no VGPRs
//     are spent on staging, and each lane's copy offset is fixed;
//   * LDS rows are 256 B with the 16-byte chunk index XOR-swizzled by the row
//     (K: sw(r) = 2*(r%8) + (r/8)%2, V: 4*(r%4) + (r/4)%4), so the K-operand
//     reads (16 rows, one chunk) and the transposed V reads are bank-conflict
//     free; the per-lane LDS addresses are a table of 16 registers, the ring
//     buffer and row block are immediate offsets;
//   * the V^T operand comes from two ds_read_b64_tr_b16 per MFMA: within each
//     16-lane group that instruction returns out[i][e] = in[4e + i/4][i%4],
//     so lane j of the group addresses key row r0 + j/4, dims d0 + 4*(j%4);
//   * softmax: the scale is folded into one fma before exp2; a sub-tile's
//     probabilities are taken against the running max as it stands and kept
//     when every lane's share of its row sum stays <= 2^32 (no probability
//     exceeds 2^32: harmless for fp32 sums and for bf16 P, whose relative
//     precision does not depend on magnitude); otherwise, and on the first
//     sub-tile, the wave takes the tile max, rescales O and l and recomputes.
//     The row sum l adds the fp32 probabilities (v_add_f32: the packed bf16
//     dot instruction would stall the matrix core);
//   * the loop's last step scales O by 1/l and writes the bf16 rows to LDS,
//     so that every global store writes 16-byte pieces of whole rows;
//   * items (query block x group) are ordered so each XCD (round-robin
//     dispatch) walks whole (batch, kv head, stream) groups, keeping that
//     group's K/V in its L2; with more items than CUs the launch is
//     persistent (one workgroup per CU walking its share of the XCD's items,
//     see the kernel below).
constexpr int D128_NW = 4;  // waves per workgroup of the head-dim-128 kernel (one per SIMD)
constexpr int D128_QW = 64; // queries per wave (two 32-query halves)


// A wave-uniform pointer, marked so for the compiler.
__device__ __forceinline__ const char *uniform_ptr(const char *p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return (const char *)(((uint64_t)hi << 32) | lo);
}

// GQ: the query map is not the identity (qmul, qadd) != (1, 0); a full layer
// runs the GQ = false instance (compile-time identity map).
// ROPE: q is rotated at its expanded position right after the load.
//
// Persistent: a launch has at most one workgroup per CU, and each walks a
// list of items (query block of one group).  The items of an XCD are those
// the non-persistent order would dispatch to it; a CU takes every
// (32 CUs)-th of them in a snake order (c, 63-c, 64+c, ...), so that the
// longest-first sequence gives each CU about the same number of tiles.
// Between two items the next item's first K/V copies and its Q loads are
// issued before the current item's output rows are stored, so the memory
// latency that starts an item overlaps the end of the previous one and no
// workgroup launch separates them.
//
// This function does the work-item map, loads Q, builds the per-lane LDS
// address tables and copy offsets the key loop (sfa_fwd_d128_loop.inc) uses,
// binds them to the registers the loop expects, and stores the output rows
// the loop leaves in LDS.
template <bool GQ, bool ROPE>
__global__ __launch_bounds__(64 * D128_NW, 1) void sfa_fwd_bf16_d128_kernel(FwdArgs p, int HG, int TB, int nqblk,
                                                                  float scale_log2) {
    constexpr int D = 128;
    constexpr int TILE = KT * D * 2;  // 16 KB per K or V tile
    constexpr int OPITCH = 272;       // bytes per staged output row (16-byte aligned, spreads the banks)
    // K ring (3 tiles) | V ring (3 tiles).  The output rows a wave leaves at
    // the end of an item are staged from byte 4*TILE on (V ring buffers 1-2
    // and beyond), clear of the buffers the next item's first copies fill
    // (K 0, K 1, V 0); the next item's loop copies into V buffer 1 only
    // after its first barrier, which every wave reaches once its own staged
    // rows are read.
    constexpr int STG = 4 * TILE;
    __shared__ __attribute__((aligned(1024))) char lds[STG + D128_NW * D128_QW * OPITCH];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5, l16 = lane & 15, g2 = (lane >> 4) & 1;
    const int g = p.Hq / p.Hkv, ngrp = g / HG;
    const int nrest = p.B * p.Hkv * ngrp * p.nsub;
    const int nwg = nrest * nqblk;
    const int hw = wave % HG, tb = wave / HG;
    const int qmul = GQ ? p.qmul : 1, qadd = GQ ? p.qadd : 0;
    const int64_t qrs = (int64_t)p.Hq * D;
    const int64_t krs = (int64_t)p.Hkv * D;
    const int QB = D128_QW * TB;

    // Item r of this workgroup, as the index of the non-persistent launch
    // (nwg when there is none).  The launch has either one workgroup per
    // item or a multiple of 8 workgroups, one per CU.
    const int G = (int)gridDim.x;
    auto item_bid = [&](int r) -> int {
        if (G >= nwg) return r == 0 ? (int)blockIdx.x : nwg;
        const int x = (int)blockIdx.x % 8, c = (int)blockIdx.x / 8, ncx = G / 8;
        const int j = r * ncx + ((r & 1) ? ncx - 1 - c : c);
        return min(x + 8 * j, nwg);
    };
    // Workgroup index -> (query block, group).  Dispatch is round-robin over
    // the 8 XCDs (XCD bid % 8 runs its workgroups in bid order); the map
    // keeps each XCD's share balanced (longest blocks first) and its groups
    // few: whole groups per XCD when the group count is a multiple of 8 (the
    // XCD's groups taken two at a time, their blocks interleaved longest
    // first: one group at a time leaves a tail of short blocks, all of them
    // at once a K/V working set larger than the XCD's L2), each group spread
    // over 8/G XCDs when G divides 8, else round-robin.
    auto item_lid = [&](int bid) -> int {
        int lid = bid;
        if (nwg % 8 == 0) {
            const int x = bid % 8, j = bid / 8;
            if (nrest % 8 == 0) {
                const int gpx = nrest / 8;
                const int iw = gpx % 2 == 0 ? 2 : gpx;  // groups interleaved at a time
                const int ph = j / (iw * nqblk), jj = j % (iw * nqblk);
                lid = (x * gpx + ph * iw + jj % iw) * nqblk + jj / iw;
            } else if (8 % nrest == 0 && nqblk % (8 / nrest) == 0) {
                const int r = 8 / nrest;
                lid = (x / r) * nqblk + j * r + x % r;
            }
        }
        return lid;
    };

    // LDS address tables.  K operand of k-step ks (keys 0-31 of ring buffer
    // 0): row l32, 16-byte chunk (2ks + hi) ^ sw(row).  V^T half-operand
    // (db, jh) (keys 0-15 of V buffer 0): ds_read_b64_tr_b16 lane j of a
    // 16-lane group addresses key 8jh + 4hi + j/4, dims 32db + 16g2 + 4(j%4);
    // with the V swizzle 4*(r%4) + (r/4)%4 the chunk index splits into
    // 4*(db ^ r4) + ((2g2 + c1) ^ (2jh + hi)).  The loop adds ring buffer,
    // 32-key half and 16-key row block as immediate offsets.
    const unsigned ldsk = lds_addr(lds), ldsv = ldsk + 3 * TILE;
    unsigned kaddr[8], vaddr[8];
    {
        const int ksw = swz128(l32) ^ hi;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) kaddr[ks] = ldsk + l32 * 256 + (((2 * ks) ^ ksw) << 4);
        const int r4 = l16 >> 2, c1 = (l16 & 3) >> 1, c0 = l16 & 1;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int jh = 0; jh < 2; ++jh)
                vaddr[db * 2 + jh] = ldsv + (8 * jh + 4 * hi + r4) * 256 +
                                     16 * (4 * (db ^ r4) + ((2 * g2 + c1) ^ (2 * jh + hi))) + 8 * c0;
    }

    // Copies: each wave moves 4 x 1 KB of K and of V per tile: slots
    // w*256 .. +255, slot s = row*16 + physical chunk; lane l of copy i fills
    // slot (w*4+i)*64 + l with logical chunk (s%16) ^ sw(row).  A tile with
    // rows past the end of the sub-sequence re-reads its last row there
    // (finite data, masked in the loop).
    const int rstride = p.stride * (int)krs;  // elements between sub-sequence rows
    const unsigned tbytes = (unsigned)(KT * rstride) * 2u;
    const unsigned ldsw = ldsk + (unsigned)wave * 4096u;  // this wave's copy slots in a ring buffer
    unsigned boff[4], boffv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int lrow = (wave * 4 + i) * 4 + (lane >> 4);
        const int lc = ((lane & 15) ^ swz128(lrow)) * 8, lcv = ((lane & 15) ^ swzv(lrow)) * 8;
        boff[i] = (unsigned)(lrow * rstride + lc) * 2u;
        boffv[i] = (unsigned)(lrow * rstride + lcv) * 2u;
    }

    // The 64 output rows of this wave are staged in LDS so that each store
    // writes 16-byte pieces of whole 256-byte rows.
    char *ost = lds + STG + wave * D128_QW * OPITCH;
    const unsigned stg = lds_addr(ost) + l32 * OPITCH + 8 * hi;

    // One item's work map: query block, head, first key tile and tile count,
    // the tile whose rows run past the sub-sequence's end, K/V of tile 0.
    struct Item {
        int qw0, h, ntiles, tfirst, tailt, rmax, b, sub;
        int64_t qbase;
        const char *kptr, *vptr;
    };
    auto decode = [&](int lid) -> Item {
        Item it;
        const int qblk = nqblk - 1 - lid % nqblk;
        int rest = lid / nqblk;
        const int sub = rest % p.nsub; rest /= p.nsub;
        const int hgrp = rest % ngrp; rest /= ngrp;
        const int kvh = rest % p.Hkv;
        const int b = rest / p.Hkv;
        const int q0 = qblk * QB;
        it.b = b;
        it.sub = sub;
        it.h = kvh * g + hgrp * HG + hw;
        it.qw0 = q0 + tb * D128_QW;  // first query of this wave; half hf holds qw0 + 32 hf + l32
        it.qbase = (int64_t)b * p.qrows + (int64_t)sub * p.qsub;  // query 0's Q row
        const int64_t bpos = (int64_t)b * p.nL + p.kbase + sub;  // key element 0
        const int kend = min((min(q0 + QB, p.Lq) - 1) * qmul + qadd + 1, p.Lsub);
        const int kbeg = p.weff ? max(0, q0 * qmul + qadd - p.weff + 1) : 0;
        it.tfirst = kbeg & ~(KT - 1);
        it.ntiles = (kend - it.tfirst + KT - 1) / KT;
        const int tlast = it.tfirst + (it.ntiles - 1) * KT;
        it.rmax = p.Lsub - 1 - tlast;
        it.tailt = it.rmax < KT - 1 ? it.ntiles - 1 : -1;
        const int64_t tile0 = (bpos + (int64_t)it.tfirst * p.stride) * krs + (int64_t)kvh * D;  // elements
        it.kptr = reinterpret_cast<const char *>(static_cast<const bf16 *>(p.k) + tile0);
        it.vptr = reinterpret_cast<const char *>(static_cast<const bf16 *>(p.v) + tile0);
        return it;
    };
    // Per-lane copy offsets of a tile whose rows run past the end.
    auto tail_offsets = [&](const Item &it, unsigned *toff, unsigned *toffv) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int lrow = (wave * 4 + i) * 4 + (lane >> 4);
            const int lc = ((lane & 15) ^ swz128(lrow)) * 8, lcv = ((lane & 15) ^ swzv(lrow)) * 8;
            toff[i] = (unsigned)(min(lrow, it.rmax) * rstride + lc) * 2u;
            toffv[i] = (unsigned)(min(lrow, it.rmax) * rstride + lcv) * 2u;
        }
    };
    // Copies of K(0), K(1) and V(0) of an item; its loop copies K(T+2) and
    // V(T+1) at the start of tile T.
    // (The item's fields are wave-uniform; readfirstlane says so to the
    // compiler, which must pass them in scalar registers.)
    auto first_copies = [&](const Item &it) {
        if (it.ntiles <= 0) return;
        unsigned toff[4], toffv[4];
        tail_offsets(it, toff, toffv);
        const char *kp = uniform_ptr(it.kptr), *vp = uniform_ptr(it.vptr);
        const unsigned lw = (unsigned)__builtin_amdgcn_readfirstlane((int)ldsw);
#pragma unroll
        for (int i = 0; i < 4; ++i) lds_dma16_s(kp, it.tailt == 0 ? toff[i] : boff[i], lw + i * 1024);
        if (it.ntiles > 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                lds_dma16_s(kp + tbytes, it.tailt == 1 ? toff[i] : boff[i], lw + TILE + i * 1024);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            lds_dma16_s(vp, it.tailt == 0 ? toffv[i] : boffv[i], lw + 3 * TILE + i * 1024);
    };
    // Q of both halves; a row past the end loads row 0 and is zeroed
    // before use (so that all 16 loads can be in flight together).
    auto load_q = [&](const Item &it, bf16x8 (&qop)[2][D / 16]) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int myq = it.qw0 + 32 * hf + l32;
            const bf16 *qp = static_cast<const bf16 *>(p.q) +
                             (it.qbase + (int64_t)(myq < p.Lq ? myq : 0) * p.qstride) * qrs + (int64_t)it.h * D;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) qop[hf][ks] = *reinterpret_cast<const bf16x8 *>(qp + ks * 16 + 8 * hi);
        }
    };

    int r = 0;
    const int bid0 = item_bid(0);
    if (bid0 >= nwg) return;
    Item cur = decode(item_lid(bid0));
    bf16x8 qop[2][D / 16];
    first_copies(cur);
    load_q(cur, qop);
    for (;;) {
        // Each half's band: key k visible <=> k - lo <= span (unsigned).
        int maskbase[2], span[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int myq = cur.qw0 + 32 * hf + l32;
            const int mylim = myq * qmul + qadd;
            if (myq >= p.Lq) {
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) qop[hf][ks] = bf16x8{};
            }
            if (ROPE) rope_rotate_q<D>(qop[hf], p.kbase + cur.sub + (int64_t)mylim * p.stride, p.rope_ft, hi);
            const int lo = p.weff ? mylim - p.weff + 1 : 0;
            span[hf] = min(mylim, p.Lsub - 1) - lo;
            maskbase[hf] = 4 * hi - lo;
        }
        // The wave's 32-key sub-tiles that need the mask: j < jw (window
        // start) or j >= jm (the diagonal or the end of the sub-sequence).
        const int lim0 = cur.qw0 * qmul + qadd;                    // last key the wave's first query may see
        const int lim1 = (cur.qw0 + D128_QW - 1) * qmul + qadd;    // ... and its last
        const int mfull = min(lim0, p.Lsub - 1) - 31 - cur.tfirst;
        const int jm = mfull >= 0 ? mfull / 32 + 1 : 0;
        const int wfull = lim1 - p.weff - cur.tfirst;
        const int jw = (p.weff && wfull >= 0) ? wfull / 32 + 1 : 0;

        float m0 = -INFINITY, m1 = -INFINITY, l0 = 0.f, l1 = 0.f;
        if (cur.ntiles > 0) {
            unsigned toff[4], toffv[4];
            tail_offsets(cur, toff, toffv);
            const void *kptr2 = cur.kptr + 2 * (size_t)tbytes;
            const void *vptr1 = cur.vptr + tbytes;
            const int ntiles = cur.ntiles, tfirst = cur.tfirst, tailt = cur.tailt;
            asm volatile(HD_FWD_D128_LOOP
                         : "+{v160}"(m0), "+{v161}"(m1), "+{v162}"(l0), "+{v163}"(l1)
                         : "{v[96:99]}"(qop[0][0]), "{v[100:103]}"(qop[0][1]), "{v[104:107]}"(qop[0][2]),
                           "{v[108:111]}"(qop[0][3]), "{v[112:115]}"(qop[0][4]), "{v[116:119]}"(qop[0][5]),
                           "{v[120:123]}"(qop[0][6]), "{v[124:127]}"(qop[0][7]), "{v[128:131]}"(qop[1][0]),
                           "{v[132:135]}"(qop[1][1]), "{v[136:139]}"(qop[1][2]), "{v[140:143]}"(qop[1][3]),
                           "{v[144:147]}"(qop[1][4]), "{v[148:151]}"(qop[1][5]), "{v[152:155]}"(qop[1][6]),
                           "{v[156:159]}"(qop[1][7]),
                           "{v164}"(kaddr[0]), "{v165}"(kaddr[1]), "{v166}"(kaddr[2]), "{v167}"(kaddr[3]),
                           "{v168}"(kaddr[4]), "{v169}"(kaddr[5]), "{v170}"(kaddr[6]), "{v171}"(kaddr[7]),
                           "{v172}"(vaddr[0]), "{v173}"(vaddr[1]), "{v174}"(vaddr[2]), "{v175}"(vaddr[3]),
                           "{v176}"(vaddr[4]), "{v177}"(vaddr[5]), "{v178}"(vaddr[6]), "{v179}"(vaddr[7]),
                           "{v180}"(boff[0]), "{v181}"(boff[1]), "{v182}"(boff[2]), "{v183}"(boff[3]),
                           "{v184}"(boffv[0]), "{v185}"(boffv[1]), "{v186}"(boffv[2]), "{v187}"(boffv[3]),
                           "{v188}"(toff[0]), "{v189}"(toff[1]), "{v190}"(toff[2]), "{v191}"(toff[3]),
                           "{v192}"(toffv[0]), "{v193}"(toffv[1]), "{v194}"(toffv[2]), "{v195}"(toffv[3]),
                           "{v196}"(maskbase[0]), "{v197}"(maskbase[1]), "{v198}"(span[0]), "{v199}"(span[1]),
                           "{v249}"(stg), [nt] "s"(ntiles), [kt0] "s"(tfirst), [kptr2] "s"(kptr2),
                           [vptr1] "s"(vptr1), [tbytes] "s"(tbytes), [tailt] "s"(tailt), [jw] "s"(jw),
                           [jm] "s"(jm), [sc] "s"(scale_log2), [ldsw] "s"(ldsw)
                         : HD_FWD_D128_CLOBBERS);
        } else {
            // no key tile (an empty key range): zero rows
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    *reinterpret_cast<uint2 *>(ost + (hf * 32 + l32) * OPITCH + 8 * hi + 16 * i) = uint2{0, 0};
            __builtin_amdgcn_s_waitcnt(0xc07f);
        }

        // The next item's first copies and Q loads go out before this item's
        // rows are stored (the loop above has passed its last barrier, so the
        // ring buffers they fill are free).
        const int bidn = item_bid(++r);
        const bool more = bidn < nwg;
        Item nxt = cur;
        if (more) {
            nxt = decode(item_lid(bidn));
            first_copies(nxt);
            load_q(nxt, qop);
        }

        // All staged rows are read first, then stored (without a per-row
        // branch when every row of the wave is in range), so the reads and
        // the stores each go out back to back.
        {
            // (one asm block with its own wait: the compiler, short of
            // registers here, would otherwise wait for each read in turn)
            static_assert(D128_QW / 4 == 16 && 15 * 4 * OPITCH < 65536, "staged-row reads below");
            u32x4 x[D128_QW / 4];
            const unsigned ra = lds_addr(ost) + (lane >> 4) * OPITCH + (lane & 15) * 16;
            asm volatile(
                "ds_read_b128 %0, %16\n\tds_read_b128 %1, %16 offset:1088\n\t"
                "ds_read_b128 %2, %16 offset:2176\n\tds_read_b128 %3, %16 offset:3264\n\t"
                "ds_read_b128 %4, %16 offset:4352\n\tds_read_b128 %5, %16 offset:5440\n\t"
                "ds_read_b128 %6, %16 offset:6528\n\tds_read_b128 %7, %16 offset:7616\n\t"
                "ds_read_b128 %8, %16 offset:8704\n\tds_read_b128 %9, %16 offset:9792\n\t"
                "ds_read_b128 %10, %16 offset:10880\n\tds_read_b128 %11, %16 offset:11968\n\t"
                "ds_read_b128 %12, %16 offset:13056\n\tds_read_b128 %13, %16 offset:14144\n\t"
                "ds_read_b128 %14, %16 offset:15232\n\tds_read_b128 %15, %16 offset:16320\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=v"(x[0]), "=v"(x[1]), "=v"(x[2]), "=v"(x[3]), "=v"(x[4]), "=v"(x[5]), "=v"(x[6]), "=v"(x[7]),
                  "=v"(x[8]), "=v"(x[9]), "=v"(x[10]), "=v"(x[11]), "=v"(x[12]), "=v"(x[13]), "=v"(x[14]),
                  "=v"(x[15])
                : "v"(ra)
                : "memory");
            char *orow = reinterpret_cast<char *>(p.o) +
                         ((cur.qbase + (int64_t)(cur.qw0 + (lane >> 4)) * p.qstride) * qrs + (int64_t)cur.h * D) * 2 +
                         (lane & 15) * 16;
            const int64_t step = 4 * (int64_t)p.qstride * qrs * 2;  // bytes between rows 4 apart
            if (cur.qw0 + D128_QW <= p.Lq) {
#pragma unroll
                for (int i = 0; i < D128_QW / 4; ++i) *reinterpret_cast<u32x4 *>(orow + i * step) = x[i];
            } else {
#pragma unroll
                for (int i = 0; i < D128_QW / 4; ++i)
                    if (cur.qw0 + 4 * i + (lane >> 4) < p.Lq) *reinterpret_cast<u32x4 *>(orow + i * step) = x[i];
            }
        }
        if (p.lse != nullptr && hi == 0) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int myq = cur.qw0 + 32 * hf + l32;
                if (myq < p.Lq) {
                    const int64_t qrow = cur.qbase + (int64_t)myq * p.qstride;
                    p.lse[((int64_t)cur.b * p.Hq + cur.h) * p.qrows + (qrow - (int64_t)cur.b * p.qrows)] =
                        (hf ? m1 : m0) * kLn2 + __logf(hf ? l1 : l0);
                }
            }
        }
        if (!more) break;
        cur = nxt;
    }
}

}  // namespace

// Compute units of the current device (read once per device).
static int device_cu_count() {
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cached[dev] = n;
    }
    return cached[dev];
}

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
                const int nqblk2 = (a.Lq + D128_QW * TB2 - 1) / (D128_QW * TB2);
                const int64_t grid2 = (int64_t)nqblk2 * a.B * a.Hkv * (g / HG) * a.nsub;
                if (grid2 > 0x7fffffff) return hipErrorInvalidConfiguration;
                const bool gq = a.qmul != 1 || a.qadd != 0;
                auto kern = gq ? (a.rope ? sfa_fwd_bf16_d128_kernel<true, true> : sfa_fwd_bf16_d128_kernel<true, false>)
                               : (a.rope ? sfa_fwd_bf16_d128_kernel<false, true> : sfa_fwd_bf16_d128_kernel<false, false>);
                // one workgroup per CU (a multiple of 8, one per XCD in turn) when
                // there are more items than CUs
                const int ncu = device_cu_count() & ~7;
                const int64_t grid3 = (ncu >= 8 && grid2 > ncu) ? ncu : grid2;
                hipLaunchKernelGGL(kern, dim3((unsigned)grid3), dim3(64 * D128_NW), 0, st, a, HG, TB2, nqblk2, sl2);
            }
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace hd
