// hd_internal.h -- types and launcher declarations shared by the HIP sources
// of libhd.so.  Not part of the public ABI (that is include/hd.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hd {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Expansion: out[b][i*n+s][:] = tables[s][ids[b][i]][:]
struct EmbedArgs {
    const int32_t *ids;
    const char *tables[16];
    char *out;
    int B, L, n;
    int64_t V;          // rows per table (ids are clamped to [0, V))
    int64_t row_bytes;
};
hipError_t launch_expand_embed(const EmbedArgs &a, hipStream_t st);

// ---------------------------------------------------------------------------
// Prefill.  Both masks are run as causal attention over a strided
// "sub-sequence" of the expanded sequence:
//   intra: one sub-sequence per stream s, element j at position j*n + s,
//          length L, window W tokens;
//   cross: one sub-sequence (the whole expanded sequence), element j at
//          position j, length n*L, window n*W positions.
// Query p of a sub-sequence sees key element j iff
//   j <= lim(p) = p*qmul + qadd  and  (weff == 0 || lim(p) - j < weff).
// A full layer has one query per key element (qmul = 1, qadd = 0, Q rows laid
// out like K rows).  The final-stream queries of a KV-mirror layer are the
// rows t = p*n + n-1 only, stored compactly: intra runs stream n-1's
// sub-sequence (kbase = n-1) with lim(p) = p; cross runs the whole sequence
// with lim(p) = p*n + n-1.
struct FwdArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;   // [B][Hq][qrows]
    int B, nL, Hq, Hkv, d;
    int Lsub;     // key elements per sub-sequence
    int nsub;     // sub-sequences per batch row (n for intra, 1 for cross)
    int stride;   // expanded positions between consecutive key elements
    int kbase;    // expanded position of element 0 of sub-sequence 0
    int weff;     // window in sub-sequence elements, 0 = none
    float scale;  // softmax scale (already resolved, > 0)
    int Lq;       // queries per sub-sequence
    int qrows;    // Q / O / lse rows per batch row
    int qsub;     // Q rows between the first queries of consecutive sub-sequences
    int qstride;  // Q rows between consecutive queries
    int qmul, qadd;
    // rotary embedding of q at its expanded position, applied after the load
    // (0 = q is used as given); rope_ft[c] = theta^(-2c/d) / (2 pi), c < d/2
    int rope;
    double rope_ft[64];
};
hipError_t launch_sfa_fwd_bf16(const FwdArgs &a, hipStream_t st);
hipError_t launch_sfa_fwd_f32(const FwdArgs &a, hipStream_t st);

// ---------------------------------------------------------------------------
// Backward of the prefill, in the same sub-sequence form as FwdArgs.
// The query side follows the same map as FwdArgs (full layer: identity;
// final-stream queries of a KV-mirror layer: compact rows, lim(p) = p*qmul + qadd).
struct BwdArgs {
    const void *q, *k, *v, *o, *dout;  // q, o, dout [B][qrows][Hq][d]
    const float *lse;  // [B][Hq][qrows], natural log, from the forward
    void *dq, *dk, *dv;
    float *drow;       // workspace [B][Hq][qrows]: D = dO . O per query row
    float *part;       // workspace after drow: dK/dV partial sums of query segments (or unused)
    int B, nL, Hq, Hkv, d;
    int Lsub, nsub, stride, kbase, weff;
    float scale;
    int Lq, qrows, qsub, qstride, qmul, qadd;
};
// Query segments of the dK/dV pass (nseg = 1: one workgroup per key block).
struct BwdSplit {
    int nseg, segq;
};
BwdSplit bwd_split(const BwdArgs &a);
// Workspace of one backward call on the mapped layer a: drow, then (bf16
// path, nseg > 1) the segments' fp32 partial dK/dV rows.
size_t bwd_workspace_bytes(const BwdArgs &a, bool bf16_path);
hipError_t launch_sfa_bwd_bf16(const BwdArgs &a, hipStream_t st);
hipError_t launch_sfa_bwd_f32(const BwdArgs &a, hipStream_t st);

// ---------------------------------------------------------------------------
// Rotary embedding of x [B][T][H][d] at positions
// t*t_mul + t_add + pos_mul * pos_base[b].
struct RopeArgs {
    const void *x;
    void *out;                // may equal x
    const int32_t *pos_base;  // device [B] or NULL
    int64_t pos_mul, t_mul, t_add;
    int B, T, H, d;
    double freq_turns[64];    // theta^(-2c/d) / (2 pi), c < d/2
};
hipError_t launch_rope(const RopeArgs &a, bool bf16_data, hipStream_t st);

// ---------------------------------------------------------------------------
// Decode over the per-stream cache [B][T_cap][n][Hkv][d].
struct DecArgs {
    const void *q, *k_new, *v_new;
    void *k_cache, *v_cache;
    const int32_t *cache_len;
    void *o;
    float *ws;          // split-KV partials (bf16 path)
    int B, n, Hq, Hkv, d, T_cap;
    int mode;           // 0 intra, 1 cross
    int window;         // tokens, 0 = none
    float scale;
    // queries: streams qs0 .. qs0+nqs-1 of the new token (all n, or only the
    // final stream of a KV-mirror layer); q, o are [B][nqs][Hq][d]
    int qs0, nqs;
    // cache rows scanned per token: n, or 1 when only stream qs0's keys can be
    // visible (an intra layer's final-stream query)
    int rpt;
};
size_t decode_workspace_bytes(int B, int n, int Hq, int Hkv, int d, int T_cap);
hipError_t launch_sfa_decode_bf16(const DecArgs &a, hipStream_t st);
hipError_t launch_sfa_decode_f32(const DecArgs &a, hipStream_t st);

}  // namespace hd
