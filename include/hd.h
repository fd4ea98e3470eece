/*
 * hd.h -- C ABI of the Stream-Factorized Attention library (libhd.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (WeLM blog "Hidden Decoding at Scale", section "Method Recap and
 * New Designs"): every token x_i is expanded into n stream embeddings taken from
 * n independent tables and interleaved along the sequence; attention over the
 * n*L-long expanded sequence is either intra-stream (causal inside a stream,
 * streams invisible to one another) or cross-stream (causal over all
 * positions), optionally inside a sliding window; decoding keeps one KV cache
 * per stream and processes the n streams of a new token in one pass.
 *
 * Conventions shared by every entry point
 *   - Indices are 0-based: expanded position t = i*n + s for token i in [0,L)
 *     and stream s in [0,n) (the pages' 1-based t = (i-1)n + k).
 *   - Every tensor pointer is DEVICE memory owned by the caller, row-major and
 *     dense, 16-byte aligned.  The library allocates no memory, keeps no
 *     pointer after a call returns and holds no state between calls except a
 *     thread-local error string (and the static scratch array of
 *     hd_sfa_decode_noalloc).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on that stream and returns without synchronising; results
 *     are deterministic (no atomics, fixed reduction orders).
 *   - dtype HD_BF16: inputs and outputs bfloat16, products accumulated in
 *     float32, softmax in float32, outputs rounded to nearest even once.
 *     dtype HD_F32: float32 end to end.
 *   - GQA: query head h reads kv head h / (Hq/Hkv).
 *   - Softmax scale: `scale` if > 0, else 1/sqrt(d).
 *
 * Error behaviour: arguments are validated on the host before anything is
 * enqueued.  HD_ERR_INVALID: a size < 1 (where >= 1 is required), Hq not a
 * multiple of Hkv, window < 0, n above HD_MAX_STREAMS, a NULL or misaligned
 * pointer, or a too-small workspace.  HD_ERR_UNSUPPORTED: a head dim other than
 * 32, 64 or 128, an unknown dtype or mode, or a shape past a documented limit.
 * HD_ERR_DEVICE: the HIP runtime reported an error at launch.  On any non-OK
 * return nothing was launched by that call (except HD_ERR_DEVICE, where an
 * earlier kernel of the same call may have been enqueued) and hd_last_error()
 * describes the problem.  Token ids outside [0,V) and cache_len[b] outside
 * [0, T_cap) are caller contract violations: the host cannot see device
 * values without synchronising, so they are not validated here (the Python
 * binding checks both when HD_DEBUG=1).  On the device, a decode step skips a
 * sequence whose cache_len is out of range (no append, no cache read) and
 * writes NaN to its outputs; an out-of-range id reads row min(max(id,0),V-1).
 */
#ifndef HD_H
#define HD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HD_OK = 0,
    HD_ERR_INVALID = 1,
    HD_ERR_UNSUPPORTED = 2,
    HD_ERR_DEVICE = 3
} hd_status;

typedef enum { HD_MODE_INTRA = 0, HD_MODE_CROSS = 1 } hd_mode;
typedef enum { HD_BF16 = 0, HD_F32 = 1 } hd_dtype;

#define HD_MAX_STREAMS 16

/*
 * Multi-stream expansion ("Multi-Stream Expansion and Training Objective",
 * equation S_t = E_k(x_i) at t = (i-1)n + k):
 *     out[b][i*n + s][:] = tables[s][ids[b][i]][:]
 * a bit-exact row copy.
 *   ids     device int32 [B][L], each in [0, V)
 *   tables  HOST array of n device pointers, table s is [V][D] of dtype dt
 *   out     device [B][n*L][D] of dtype dt
 * Requires B, L >= 1, 1 <= n <= HD_MAX_STREAMS, V >= 1, D >= 1.
 */
hd_status hd_expand_embed(const int32_t *ids, int B, int L, int n,
                          const void *const *tables, int64_t V, int D, hd_dtype dt,
                          void *out, void *stream);

/*
 * Prefill with the rotary embedding of the expanded positions fused in
 * ("Multi-Stream Expansion and Training Objective": contiguous RoPE positions
 * over the expanded sequence): k is rotated into k_rot (exactly hd_rope with
 * pos_base = NULL), q is rotated inside the attention kernel right after it
 * is loaded (no rotated q is written), then attention runs as hd_sfa_fwd on
 * the rotated q and k_rot.  Same arguments as hd_sfa_fwd plus
 *   k_rot  [B][n*L][Hkv][d] (dtype dt): output, the rotated keys (the rows a
 *          decode cache holds); may equal k (k is then rotated in place)
 *   theta  RoPE base (> 0), as in hd_rope
 * The in-kernel rotation of q reduces the angle in double and uses the
 * hardware sine / cosine; it agrees with hd_rope to the bf16 rounding of q.
 */
hd_status hd_sfa_fwd_rope(const void *q, const void *k, const void *v, void *o, float *lse, void *k_rot,
                          int B, int L, int n, int Hq, int Hkv, int d, hd_mode mode, int window, float scale,
                          float theta, hd_dtype dt, void *stream);

/*
 * Rotary position embedding at the expanded positions ("Multi-Stream
 * Expansion and Training Objective": the expanded sequence is fed to the
 * Transformer with contiguous RoPE positions, so S_t is rotated by its
 * expanded position t = i*n + s, not by its token index).  Rotate-half form,
 * h = d/2, f_c = theta^(-2c/d):
 *   out[..][c]     = x[c] cos(p f_c) - x[c+h] sin(p f_c)
 *   out[..][c + h] = x[c+h] cos(p f_c) + x[c] sin(p f_c)
 * with position p = t*t_mul + t_add + pos_mul * pos_base[b] for row (b, t).
 *   x, out    [B][T][H][d] (dtype dt); out may equal x (in place)
 *   pos_base  device int32 [B] or NULL (0)
 * The rows the library's entry points take:
 *   prefill q, k [B][n*L][H][d]:           pos_base NULL, t_mul 1, t_add 0 (p = t)
 *   final-stream q [B][L][H][d] (KV-mirror): pos_base NULL, t_mul n, t_add n-1
 *                                           (row i is position i*n + n-1)
 *   decode q, k_new [B][n][H][d]:          pos_base = cache_len, pos_mul n,
 *                                           t_mul 1, t_add 0 (p = len*n + s)
 *   final-stream decode q [B][1][H][d]:     pos_base = cache_len, pos_mul n,
 *                                           t_add n-1 (p = len*n + n-1)
 * Apply it to q and k before the attention call.  Requires B, T, H >= 1,
 * d in {32, 64, 128}, theta > 0, pos_mul, t_mul, t_add >= 0.
 */
hd_status hd_rope(const void *x, void *out, int B, int T, int H, int d, const int32_t *pos_base, int64_t pos_mul,
                  int64_t t_mul, int64_t t_add, float theta, hd_dtype dt, void *stream);

/*
 * Stream-Factorized Attention prefill ("Stream-Factorized Attention", index
 * maps i(t) = ceil(t/n), s(t) = (t-1) mod n + 1, and Figure 2).  For every
 * query row (b, t_q, h) with i_q = t_q/n, s_q = t_q%n:
 *   mode HD_MODE_INTRA (mask c): keys t_k = j*n + s_q with j <= i_q, and
 *        i_q - j < window when window > 0 (window counts tokens, incl. self);
 *   mode HD_MODE_CROSS (mask a; mask b when window > 0): keys t_k <= t_q, and
 *        t_q - t_k < n*window when window > 0;
 *   o = softmax(scale * q.k over the visible keys) . v
 *   q, o  [B][n*L][Hq][d]         k, v  [B][n*L][Hkv][d]     (dtype dt)
 *   lse   optional float32 [B][Hq][n*L]: natural log of the softmax
 *         denominator sum_k exp(scale*q.k) over the visible keys (NULL = skip)
 * Requires B, L, n, Hq, Hkv >= 1, Hq % Hkv == 0, d in {32, 64, 128},
 * window >= 0, n <= HD_MAX_STREAMS, n*L <= 2^30.
 */
hd_status hd_sfa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                     int B, int L, int n, int Hq, int Hkv, int d,
                     hd_mode mode, int window, float scale, hd_dtype dt, void *stream);

/*
 * Final-stream queries of a KV-mirror layer ("Persistent KV and the KV-mirror
 * Saving": a mirrored layer takes its K/V from an earlier layer, where all n
 * streams were processed, and only the supervised last stream is run through
 * it).  Query i of q is the row of stream n-1 of token i, expanded position
 * t = i*n + n-1; it attends over k/v of all n*L positions exactly as that row
 * of hd_sfa_fwd would:
 *   mode HD_MODE_INTRA: keys t_k = j*n + n-1, j <= i, i - j < window if > 0;
 *   mode HD_MODE_CROSS: keys t_k <= t, t - t_k < n*window if window > 0.
 *   q, o  [B][L][Hq][d] (final-stream rows only)   k, v  [B][n*L][Hkv][d]
 *   lse   optional float32 [B][Hq][L] (NULL = skip)
 * Same requirements and errors as hd_sfa_fwd.
 */
hd_status hd_sfa_fwd_final(const void *q, const void *k, const void *v, void *o, float *lse,
                           int B, int L, int n, int Hq, int Hkv, int d,
                           hd_mode mode, int window, float scale, hd_dtype dt, void *stream);

/*
 * Bytes of device workspace hd_sfa_bwd needs for these sizes (0 if the sizes
 * are invalid), the larger of the intra and cross layers of the shape (the
 * window does not change it): one float32 per query row (B*Hq*n*L*4, rounded
 * up to 256 bytes), then, for bf16 layers whose dK/dV pass would have fewer
 * than 4096 key waves (B*Hkv*(sub-sequences)*ceil(keys per sub-sequence/32))
 * and at least 256 queries per sub-sequence, float32 partial dK and dV rows
 * for nseg segments of the query range: segments of
 * max(128, ceil(ceil(Lq/want)/32)*32) queries, want = min(8, ceil(8192/waves)),
 * nseg*B*(sub-sequences)*Hkv*(keys per sub-sequence)*2*d*4 bytes.  For the
 * n = 1 control at L = 4096, 32/8 heads, d = 128 that is 268 MB.
 */
size_t hd_sfa_bwd_workspace_bytes(int B, int L, int n, int Hq, int Hkv, int d, hd_dtype dt);

/*
 * Backward of hd_sfa_fwd: the gradients of the scalar sum(dout * o) with
 * respect to q, k and v, for the same mask, window and scale.  The pages
 * define the forward ("Stream-Factorized Attention", Figure 2) and state the
 * method's cost in training step time ("Near-Linear Training Cost", Figure 3);
 * this is the standard derivative of that forward.  With P the softmax
 * weights over the visible keys (recomputed from lse) and D = dout . o per
 * query row:
 *   dP = dout . v,  dS = P * (dP - D)
 *   dq = scale * dS k,   dk = scale * dS^T q,   dv = P^T dout
 * where dk and dv sum over the query heads of each kv head's GQA group.
 *   q, o, dout, dq  [B][n*L][Hq][d]      k, v, dk, dv  [B][n*L][Hkv][d]  (dtype dt)
 *   lse        float32 [B][Hq][n*L] as written by hd_sfa_fwd for these inputs
 *   workspace  device, >= hd_sfa_bwd_workspace_bytes(...) bytes; contents on
 *              entry do not matter; two calls that may run concurrently need
 *              separate workspaces
 * Every output element is written exactly once (no atomics); results are
 * deterministic.  Size rules as for hd_sfa_fwd; all pointers must be non-NULL
 * and 16-byte aligned.
 */
hd_status hd_sfa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                     const float *lse, void *dq, void *dk, void *dv,
                     int B, int L, int n, int Hq, int Hkv, int d,
                     hd_mode mode, int window, float scale, hd_dtype dt,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace hd_sfa_bwd_final needs (0 if the sizes are
 * invalid): one float32 per final-stream query row (B*Hq*L*4, rounded up to
 * 256 bytes), plus the partial dK/dV rows of the same rule as
 * hd_sfa_bwd_workspace_bytes with one sub-sequence of L keys (intra) or n*L
 * keys (cross) and L queries.
 */
size_t hd_sfa_bwd_final_workspace_bytes(int B, int L, int n, int Hq, int Hkv, int d, hd_dtype dt);

/*
 * Backward of hd_sfa_fwd_final (training through a KV-mirror layer, where only
 * the final stream is run; "Persistent KV and the KV-mirror Saving"): the
 * gradients of sum(dout * o) over the final-stream rows with respect to q (the
 * final rows), k and v (every position, of every stream: a key row receives
 * gradient from the final-stream queries that see it, zero if none does).
 * Same formulas as hd_sfa_bwd, with
 *   q, o, dout, dq  [B][L][Hq][d]      k, v, dk, dv  [B][n*L][Hkv][d]  (dtype dt)
 *   lse        float32 [B][Hq][L] as written by hd_sfa_fwd_final for these inputs
 *   workspace  device memory of at least hd_sfa_bwd_final_workspace_bytes bytes
 * Same requirements and errors as hd_sfa_bwd.
 */
hd_status hd_sfa_bwd_final(const void *q, const void *k, const void *v, const void *o, const void *dout,
                           const float *lse, void *dq, void *dk, void *dv, int B, int L, int n, int Hq, int Hkv,
                           int d, hd_mode mode, int window, float scale, hd_dtype dt, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace hd_sfa_decode needs for these sizes (0 if the
 * sizes are invalid).  The workspace holds float32 split-KV partial results.
 */
size_t hd_sfa_decode_workspace_bytes(int B, int n, int Hq, int Hkv, int d, int T_cap);

/*
 * One decode step over the retained per-stream KV cache ("Persistent KV and
 * the KV-mirror Saving": a separate KV cache per stream; "Inference
 * Throughput": the n streams of the new token are processed in one pass).
 * For sequence b with len = cache_len[b] tokens already cached:
 *   1. the new token's keys/values are appended at token len:
 *        k_cache[b][len][s][h][:] = k_new[b][s][h][:]   (same for v)
 *   2. the query of stream s sits at expanded position t_q = len*n + s and
 *      attends, under the layer's mask (see hd_sfa_fwd), over the keys of
 *      tokens 0..len (the appended row included):
 *        o[b][s][h][:] = softmax(scale * q.k) . v
 *   q, o         [B][n][Hq][d]
 *   k_new, v_new [B][n][Hkv][d]
 *   k_cache, v_cache [B][T_cap][n][Hkv][d], rows >= len are never read
 *   cache_len    DEVICE int32 [B], each in [0, T_cap); not modified (the
 *                caller advances it after the step)
 *   workspace    device, >= hd_sfa_decode_workspace_bytes(B, n, Hq, Hkv, d, T_cap)
 *                bytes (HD_BF16; the HD_F32 path uses none and accepts NULL);
 *                its contents on entry do not matter
 * Requires the prefill size rules plus T_cap >= 1, n*(Hq/Hkv) <= 64.
 */
hd_status hd_sfa_decode(const void *q, const void *k_new, const void *v_new,
                        void *k_cache, void *v_cache, const int32_t *cache_len, int T_cap,
                        void *o, int B, int n, int Hq, int Hkv, int d,
                        hd_mode mode, int window, float scale, hd_dtype dt,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode step of a KV-mirror layer ("Persistent KV and the KV-mirror
 * Saving": only the supervised final stream is run through a mirrored layer;
 * its K/V, of every stream, come from the paired early layer).  As
 * hd_sfa_decode, with only the final stream's query:
 *   q, o   [B][1][Hq][d]: the query / output of stream n-1 of the new token,
 *          at expanded position len*n + n-1
 *   k_new, v_new  [B][n][Hkv][d]: all n streams' rows, appended as in
 *          hd_sfa_decode (the cache layout is shared)
 * Intra layers read only stream n-1's cache rows (1/n of the cache bytes);
 * cross layers read every row.  The workspace is the one hd_sfa_decode
 * needs for the same sizes (hd_sfa_decode_workspace_bytes).  Same
 * requirements and errors, with Hq/Hkv <= 64.
 */
hd_status hd_sfa_decode_final(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                              const int32_t *cache_len, int T_cap, void *o, int B, int n, int Hq, int Hkv, int d,
                              hd_mode mode, int window, float scale, hd_dtype dt, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * hd_sfa_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, semantics and errors as hd_sfa_decode, without the
 * workspace: the split-KV partials go to a scratch array of
 * HD_NOALLOC_SCRATCH_BYTES that the library holds in device memory, one copy
 * per GPU, from the first call on that GPU until the process ends.  Sizes
 * whose partials need more (hd_sfa_decode_workspace_bytes above the limit)
 * return HD_ERR_INVALID.  The call allocates nothing.  Calls that overlap on
 * one GPU (enqueued on different streams without ordering between them) race
 * on the shared scratch; calls ordered on one stream do not.
 */
#define HD_NOALLOC_SCRATCH_BYTES (32u << 20)
hd_status hd_sfa_decode_noalloc(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                                const int32_t *cache_len, int T_cap, void *o, int B, int n, int Hq, int Hkv, int d,
                                hd_mode mode, int window, float scale, hd_dtype dt, void *stream);

/* Static name of a status code. */
const char *hd_status_string(hd_status s);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char *hd_last_error(void);

/* Library ABI version (major*10000 + minor*100 + patch). */
int hd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HD_H */
