// api.hip -- the C ABI of libhd.so (declared in include/hd.h): argument
// validation on the host, then dispatch to the HIP kernels on the caller's
// stream.  No allocation, no synchronisation; the only state is a
// thread-local error string and, for the allocation-free decode entry point,
// the per-device address of its static scratch array.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "hd.h"
#include "hd_internal.h"

namespace {

thread_local char g_err[512] = "";

hd_status fail(hd_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

hd_status ok() {
    g_err[0] = '\0';
    return HD_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hd_status check_ptr(const void *p, const char *name) {
    if (p == nullptr) return fail(HD_ERR_INVALID, "%s is NULL", name);
    if (!aligned16(p)) return fail(HD_ERR_INVALID, "%s is not 16-byte aligned", name);
    return HD_OK;
}

hd_status device_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(HD_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

#define HD_TRY(expr)                         \
    do {                                     \
        hd_status _s = (expr);               \
        if (_s != HD_OK) return _s;          \
    } while (0)

// The raw value of an enum a C caller passed (it may lie outside the
// enumerators, and loading such a value as the enum type is undefined in C++).
template <typename E>
int raw_int(const E &e) {
    static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
    int v;
    std::memcpy(&v, &e, sizeof v);
    return v;
}

// Shared validation of the attention sizes (mode and dtype as raw values).
hd_status check_attn(int B, int n, int Hq, int Hkv, int d, int mode, int window, int dt) {
    if (B < 1 || n < 1 || Hq < 1 || Hkv < 1)
        return fail(HD_ERR_INVALID, "sizes must be >= 1 (B=%d n=%d Hq=%d Hkv=%d)", B, n, Hq, Hkv);
    if (n > HD_MAX_STREAMS) return fail(HD_ERR_INVALID, "n=%d above HD_MAX_STREAMS=%d", n, HD_MAX_STREAMS);
    if (Hq % Hkv) return fail(HD_ERR_INVALID, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (window < 0) return fail(HD_ERR_INVALID, "window=%d < 0", window);
    if (d != 32 && d != 64 && d != 128) return fail(HD_ERR_UNSUPPORTED, "head dim %d not in {32, 64, 128}", d);
    if (dt != HD_BF16 && dt != HD_F32) return fail(HD_ERR_UNSUPPORTED, "unknown dtype %d", dt);
    if (mode != HD_MODE_INTRA && mode != HD_MODE_CROSS) return fail(HD_ERR_UNSUPPORTED, "unknown mode %d", mode);
    return HD_OK;
}

float resolve_scale(float scale, int d) {
    return (scale > 0.f && std::isfinite(scale)) ? scale : 1.0f / std::sqrt((float)d);
}

// Scratch of hd_sfa_decode_noalloc: the split-KV partials of one decode step
// live here instead of in a caller workspace.  One copy per GPU the library
// runs on, held until the process ends; every call on a GPU shares it.
static __device__ __align__(256) char scratch[HD_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` per device, looked up once per device (with it
// current) on the first allocation-free call there.  Host code never uses the
// array's own name as an address: on the host it is only a stand-in symbol.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

hd_status scratch_for_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(HD_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(HD_ERR_UNSUPPORTED, "device %d above %d", dev, kMaxDevices - 1);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr)
            return fail(HD_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return HD_OK;
}

}  // namespace

extern "C" {

const char *hd_status_string(hd_status s) {
    // C callers may pass any int: read the raw value (loading an enum outside
    // its enumerators is undefined in C++)
    int v;
    std::memcpy(&v, &s, sizeof v);
    switch (v) {
        case HD_OK: return "HD_OK";
        case HD_ERR_INVALID: return "HD_ERR_INVALID";
        case HD_ERR_UNSUPPORTED: return "HD_ERR_UNSUPPORTED";
        case HD_ERR_DEVICE: return "HD_ERR_DEVICE";
    }
    return "HD_ERR_UNKNOWN";
}

const char *hd_last_error(void) { return g_err; }

int hd_version(void) { return 100; }

hd_status hd_expand_embed(const int32_t *ids, int B, int L, int n, const void *const *tables, int64_t V,
                          int D, hd_dtype dt, void *out, void *stream) {
    if (B < 1 || L < 1 || n < 1 || V < 1 || D < 1)
        return fail(HD_ERR_INVALID, "sizes must be >= 1 (B=%d L=%d n=%d V=%lld D=%d)", B, L, n, (long long)V, D);
    if (n > HD_MAX_STREAMS) return fail(HD_ERR_INVALID, "n=%d above HD_MAX_STREAMS=%d", n, HD_MAX_STREAMS);
    if (raw_int(dt) != HD_BF16 && raw_int(dt) != HD_F32)
        return fail(HD_ERR_UNSUPPORTED, "unknown dtype %d", raw_int(dt));
    if (tables == nullptr) return fail(HD_ERR_INVALID, "tables is NULL");
    HD_TRY(check_ptr(ids, "ids"));
    HD_TRY(check_ptr(out, "out"));
    hd::EmbedArgs a{};
    for (int s = 0; s < n; ++s) {
        HD_TRY(check_ptr(tables[s], "tables[s]"));
        a.tables[s] = static_cast<const char *>(tables[s]);
    }
    a.ids = ids;
    a.out = static_cast<char *>(out);
    a.B = B;
    a.L = L;
    a.n = n;
    a.V = V;
    a.row_bytes = (int64_t)D * (dt == HD_BF16 ? 2 : 4);
    return device_status(hd::launch_expand_embed(a, static_cast<hipStream_t>(stream)), "expand_embed launch");
}

// Sub-sequence form and query map of one attention layer (FwdArgs, BwdArgs):
// every position a query (final_only = false), or only the rows of stream
// n-1, stored compactly, over K/V of every position (final_only = true).
extern "C++" {
template <typename A>
static void layer_map(A &a, int L, int n, hd_mode mode, int window, bool final_only) {
    a.nL = n * L;
    const int64_t wx = (int64_t)n * window;  // cross window in positions
    const int wcross = (window == 0 || wx >= (int64_t)n * L) ? 0 : (int)wx;
    const int wintra = window >= L ? 0 : window;
    if (!final_only) {
        if (mode == HD_MODE_INTRA) { a.Lsub = L; a.nsub = n; a.stride = n; a.weff = wintra; }
        else { a.Lsub = n * L; a.nsub = 1; a.stride = 1; a.weff = wcross; }
        a.kbase = 0;
        a.Lq = a.Lsub; a.qrows = n * L; a.qsub = 1; a.qstride = a.stride;  // Q rows laid out like K rows
        a.qmul = 1; a.qadd = 0;
        return;
    }
    a.nsub = 1;
    a.Lq = L; a.qrows = L; a.qsub = 0; a.qstride = 1;  // query i is row i of the compact q
    if (mode == HD_MODE_INTRA) {
        // stream n-1's own sub-sequence: key j at position j*n + n-1
        a.Lsub = L; a.stride = n; a.kbase = n - 1;
        a.qmul = 1; a.qadd = 0;
        a.weff = wintra;
    } else {
        // the whole expanded sequence; query i sits at position i*n + n-1
        a.Lsub = n * L; a.stride = 1; a.kbase = 0;
        a.qmul = n; a.qadd = n - 1;
        a.weff = wcross;
    }
}

// Rotary frequencies in turns: ft[c] = theta^(-2c/d) / (2 pi), c < d/2.
static void rope_freqs(double *ft, int d, float theta) {
    for (int c = 0; c < d / 2; ++c) ft[c] = std::pow((double)theta, -2.0 * c / d) / (2.0 * 3.14159265358979323846);
}
}  // extern "C++"

hd_status hd_sfa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int L, int n,
                     int Hq, int Hkv, int d, hd_mode mode, int window, float scale, hd_dtype dt, void *stream) {
    if (L < 1) return fail(HD_ERR_INVALID, "L=%d < 1", L);
    HD_TRY(check_attn(B, n, Hq, Hkv, d, raw_int(mode), window, raw_int(dt)));
    if ((int64_t)n * L > (1 << 30)) return fail(HD_ERR_UNSUPPORTED, "n*L=%lld above 2^30", (long long)n * L);
    HD_TRY(check_ptr(q, "q"));
    HD_TRY(check_ptr(k, "k"));
    HD_TRY(check_ptr(v, "v"));
    HD_TRY(check_ptr(o, "o"));
    if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u))
        return fail(HD_ERR_INVALID, "lse is not 4-byte aligned");
    hd::FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.d = d;
    layer_map(a, L, n, mode, window, false);
    a.scale = resolve_scale(scale, d);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = (dt == HD_BF16) ? hd::launch_sfa_fwd_bf16(a, st) : hd::launch_sfa_fwd_f32(a, st);
    return device_status(e, "sfa_fwd launch");
}

hd_status hd_sfa_fwd_final(const void *q, const void *k, const void *v, void *o, float *lse, int B, int L, int n,
                           int Hq, int Hkv, int d, hd_mode mode, int window, float scale, hd_dtype dt,
                           void *stream) {
    if (L < 1) return fail(HD_ERR_INVALID, "L=%d < 1", L);
    HD_TRY(check_attn(B, n, Hq, Hkv, d, raw_int(mode), window, raw_int(dt)));
    if ((int64_t)n * L > (1 << 30)) return fail(HD_ERR_UNSUPPORTED, "n*L=%lld above 2^30", (long long)n * L);
    HD_TRY(check_ptr(q, "q"));
    HD_TRY(check_ptr(k, "k"));
    HD_TRY(check_ptr(v, "v"));
    HD_TRY(check_ptr(o, "o"));
    if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u))
        return fail(HD_ERR_INVALID, "lse is not 4-byte aligned");
    hd::FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.d = d;
    layer_map(a, L, n, mode, window, true);
    a.scale = resolve_scale(scale, d);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = (dt == HD_BF16) ? hd::launch_sfa_fwd_bf16(a, st) : hd::launch_sfa_fwd_f32(a, st);
    return device_status(e, "sfa_fwd_final launch");
}

hd_status hd_sfa_fwd_rope(const void *q, const void *k, const void *v, void *o, float *lse, void *k_rot, int B,
                          int L, int n, int Hq, int Hkv, int d, hd_mode mode, int window, float scale, float theta,
                          hd_dtype dt, void *stream) {
    if (L < 1) return fail(HD_ERR_INVALID, "L=%d < 1", L);
    HD_TRY(check_attn(B, n, Hq, Hkv, d, raw_int(mode), window, raw_int(dt)));
    if ((int64_t)n * L > (1 << 30)) return fail(HD_ERR_UNSUPPORTED, "n*L=%lld above 2^30", (long long)n * L);
    if (!(theta > 0.f) || !std::isfinite(theta)) return fail(HD_ERR_INVALID, "theta=%g must be > 0", (double)theta);
    HD_TRY(check_ptr(q, "q"));
    HD_TRY(check_ptr(k, "k"));
    HD_TRY(check_ptr(v, "v"));
    HD_TRY(check_ptr(o, "o"));
    HD_TRY(check_ptr(k_rot, "k_rot"));
    if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u))
        return fail(HD_ERR_INVALID, "lse is not 4-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(stream);
    hd::RopeArgs ra{};  // k -> k_rot at positions 0 .. n*L-1
    ra.x = k; ra.out = k_rot; ra.pos_base = nullptr; ra.pos_mul = 0; ra.t_mul = 1; ra.t_add = 0;
    ra.B = B; ra.T = n * L; ra.H = Hkv; ra.d = d;
    rope_freqs(ra.freq_turns, d, theta);
    hipError_t e = hd::launch_rope(ra, dt == HD_BF16, st);
    if (e != hipSuccess) return device_status(e, "rope launch");
    hd::FwdArgs a{};
    a.q = q; a.k = k_rot; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.d = d;
    layer_map(a, L, n, mode, window, false);
    a.scale = resolve_scale(scale, d);
    a.rope = 1;
    rope_freqs(a.rope_ft, d, theta);
    e = (dt == HD_BF16) ? hd::launch_sfa_fwd_bf16(a, st) : hd::launch_sfa_fwd_f32(a, st);
    return device_status(e, "sfa_fwd_rope launch");
}

hd_status hd_rope(const void *x, void *out, int B, int T, int H, int d, const int32_t *pos_base, int64_t pos_mul,
                  int64_t t_mul, int64_t t_add, float theta, hd_dtype dt, void *stream) {
    if (B < 1 || T < 1 || H < 1) return fail(HD_ERR_INVALID, "sizes must be >= 1 (B=%d T=%d H=%d)", B, T, H);
    if (d != 32 && d != 64 && d != 128) return fail(HD_ERR_UNSUPPORTED, "head dim %d not in {32, 64, 128}", d);
    if (raw_int(dt) != HD_BF16 && raw_int(dt) != HD_F32)
        return fail(HD_ERR_UNSUPPORTED, "unknown dtype %d", raw_int(dt));
    if (!(theta > 0.f) || !std::isfinite(theta)) return fail(HD_ERR_INVALID, "theta=%g must be > 0", (double)theta);
    if (pos_mul < 0 || t_mul < 0 || t_add < 0)
        return fail(HD_ERR_INVALID, "pos_mul=%lld, t_mul=%lld, t_add=%lld must be >= 0", (long long)pos_mul,
                    (long long)t_mul, (long long)t_add);
    HD_TRY(check_ptr(x, "x"));
    HD_TRY(check_ptr(out, "out"));
    if (pos_base != nullptr && (reinterpret_cast<uintptr_t>(pos_base) & 3u))
        return fail(HD_ERR_INVALID, "pos_base is not 4-byte aligned");
    hd::RopeArgs a{};
    a.x = x; a.out = out; a.pos_base = pos_base; a.pos_mul = pos_mul; a.t_mul = t_mul; a.t_add = t_add;
    a.B = B; a.T = T; a.H = H; a.d = d;
    rope_freqs(a.freq_turns, d, theta);
    return device_status(hd::launch_rope(a, dt == HD_BF16, static_cast<hipStream_t>(stream)), "rope launch");
}

// Workspace of a backward call, the larger of the intra and cross layers of
// this shape (the window does not change it).
static size_t bwd_ws_bytes(int B, int L, int n, int Hq, int Hkv, int d, hd_dtype dt, bool final_only) {
    if (L < 1 || (int64_t)n * L > (1 << 30)) return 0;
    if (check_attn(B, n, Hq, Hkv, d, HD_MODE_INTRA, 0, raw_int(dt)) != HD_OK) return 0;
    size_t need = 0;
    for (hd_mode mode : {HD_MODE_INTRA, HD_MODE_CROSS}) {
        hd::BwdArgs a{};
        a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.d = d;
        layer_map(a, L, n, mode, 0, final_only);
        need = std::max(need, hd::bwd_workspace_bytes(a, dt == HD_BF16));
    }
    return need;
}

size_t hd_sfa_bwd_workspace_bytes(int B, int L, int n, int Hq, int Hkv, int d, hd_dtype dt) {
    return bwd_ws_bytes(B, L, n, Hq, Hkv, d, dt, false);
}

static hd_status sfa_bwd_common(const void *q, const void *k, const void *v, const void *o, const void *dout,
                                const float *lse, void *dq, void *dk, void *dv, int B, int L, int n, int Hq,
                                int Hkv, int d, hd_mode mode, int window, float scale, hd_dtype dt, void *workspace,
                                size_t workspace_bytes, void *stream, bool final_only) {
    if (L < 1) return fail(HD_ERR_INVALID, "L=%d < 1", L);
    HD_TRY(check_attn(B, n, Hq, Hkv, d, raw_int(mode), window, raw_int(dt)));
    if ((int64_t)n * L > (1 << 30)) return fail(HD_ERR_UNSUPPORTED, "n*L=%lld above 2^30", (long long)n * L);
    HD_TRY(check_ptr(q, "q"));
    HD_TRY(check_ptr(k, "k"));
    HD_TRY(check_ptr(v, "v"));
    HD_TRY(check_ptr(o, "o"));
    HD_TRY(check_ptr(dout, "dout"));
    HD_TRY(check_ptr(dq, "dq"));
    HD_TRY(check_ptr(dk, "dk"));
    HD_TRY(check_ptr(dv, "dv"));
    HD_TRY(check_ptr(lse, "lse"));
    HD_TRY(check_ptr(workspace, "workspace"));
    hd::BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.d = d;
    layer_map(a, L, n, mode, window, final_only);
    a.scale = resolve_scale(scale, d);
    const size_t need = hd::bwd_workspace_bytes(a, dt == HD_BF16);
    if (workspace_bytes < need)
        return fail(HD_ERR_INVALID, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    a.drow = static_cast<float *>(workspace);
    a.part = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                       ((size_t)B * Hq * a.qrows * sizeof(float) + 255) / 256 * 256);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = (dt == HD_BF16) ? hd::launch_sfa_bwd_bf16(a, st) : hd::launch_sfa_bwd_f32(a, st);
    return device_status(e, final_only ? "sfa_bwd_final launch" : "sfa_bwd launch");
}

hd_status hd_sfa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                     const float *lse, void *dq, void *dk, void *dv, int B, int L, int n, int Hq, int Hkv, int d,
                     hd_mode mode, int window, float scale, hd_dtype dt, void *workspace, size_t workspace_bytes,
                     void *stream) {
    return sfa_bwd_common(q, k, v, o, dout, lse, dq, dk, dv, B, L, n, Hq, Hkv, d, mode, window, scale, dt,
                          workspace, workspace_bytes, stream, false);
}

size_t hd_sfa_bwd_final_workspace_bytes(int B, int L, int n, int Hq, int Hkv, int d, hd_dtype dt) {
    return bwd_ws_bytes(B, L, n, Hq, Hkv, d, dt, true);
}

hd_status hd_sfa_bwd_final(const void *q, const void *k, const void *v, const void *o, const void *dout,
                           const float *lse, void *dq, void *dk, void *dv, int B, int L, int n, int Hq, int Hkv,
                           int d, hd_mode mode, int window, float scale, hd_dtype dt, void *workspace,
                           size_t workspace_bytes, void *stream) {
    return sfa_bwd_common(q, k, v, o, dout, lse, dq, dk, dv, B, L, n, Hq, Hkv, d, mode, window, scale, dt,
                          workspace, workspace_bytes, stream, true);
}

size_t hd_sfa_decode_workspace_bytes(int B, int n, int Hq, int Hkv, int d, int T_cap) {
    if (B < 1 || n < 1 || Hq < 1 || Hkv < 1 || d < 1 || T_cap < 1 || Hq % Hkv) return 0;
    return hd::decode_workspace_bytes(B, n, Hq, Hkv, d, T_cap);
}

static hd_status sfa_decode_common(const void *q, const void *k_new, const void *v_new, void *k_cache,
                                   void *v_cache, const int32_t *cache_len, int T_cap, void *o, int B, int n, int Hq,
                                   int Hkv, int d, hd_mode mode, int window, float scale, hd_dtype dt,
                                   void *workspace, size_t workspace_bytes, void *stream, bool final_only,
                                   bool noalloc = false) {
    HD_TRY(check_attn(B, n, Hq, Hkv, d, raw_int(mode), window, raw_int(dt)));
    if (T_cap < 1) return fail(HD_ERR_INVALID, "T_cap=%d < 1", T_cap);
    const int qrows = (final_only ? 1 : n) * (Hq / Hkv);
    if (qrows > 64) return fail(HD_ERR_UNSUPPORTED, "%d query rows per kv head above 64", qrows);
    HD_TRY(check_ptr(q, "q"));
    HD_TRY(check_ptr(k_new, "k_new"));
    HD_TRY(check_ptr(v_new, "v_new"));
    HD_TRY(check_ptr(k_cache, "k_cache"));
    HD_TRY(check_ptr(v_cache, "v_cache"));
    HD_TRY(check_ptr(cache_len, "cache_len"));
    HD_TRY(check_ptr(o, "o"));
    hd::DecArgs a{};
    a.q = q; a.k_new = k_new; a.v_new = v_new; a.k_cache = k_cache; a.v_cache = v_cache;
    a.cache_len = cache_len; a.o = o;
    a.B = B; a.n = n; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.T_cap = T_cap;
    a.mode = (int)mode; a.window = window;
    a.scale = resolve_scale(scale, d);
    if (final_only) {
        // the final stream's query only; an intra layer shows it stream n-1's keys alone
        a.qs0 = n - 1; a.nqs = 1; a.rpt = (mode == HD_MODE_INTRA) ? 1 : n;
    } else {
        a.qs0 = 0; a.nqs = n; a.rpt = n;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    const char *what = final_only ? "sfa_decode_final launch" : "sfa_decode launch";
    if (dt == HD_BF16) {
        const size_t need = hd::decode_workspace_bytes(B, n, Hq, Hkv, d, T_cap);
        if (noalloc) {  // the library's own scratch, looked up after every other check
            if (need > (size_t)HD_NOALLOC_SCRATCH_BYTES)
                return fail(HD_ERR_INVALID, "these sizes need %zu bytes of split-KV scratch, above the %zu bytes "
                            "hd_sfa_decode_noalloc holds (use hd_sfa_decode with a workspace)",
                            need, (size_t)HD_NOALLOC_SCRATCH_BYTES);
            HD_TRY(scratch_for_current_device(&workspace));
            workspace_bytes = (size_t)HD_NOALLOC_SCRATCH_BYTES;
        }
        if (workspace_bytes < need)
            return fail(HD_ERR_INVALID, "workspace of %zu bytes below the %zu required", workspace_bytes, need);
        HD_TRY(check_ptr(workspace, "workspace"));
        a.ws = static_cast<float *>(workspace);
        return device_status(hd::launch_sfa_decode_bf16(a, st), what);
    }
    return device_status(hd::launch_sfa_decode_f32(a, st), what);
}

hd_status hd_sfa_decode(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                        const int32_t *cache_len, int T_cap, void *o, int B, int n, int Hq, int Hkv, int d,
                        hd_mode mode, int window, float scale, hd_dtype dt, void *workspace,
                        size_t workspace_bytes, void *stream) {
    return sfa_decode_common(q, k_new, v_new, k_cache, v_cache, cache_len, T_cap, o, B, n, Hq, Hkv, d, mode, window,
                             scale, dt, workspace, workspace_bytes, stream, false);
}

hd_status hd_sfa_decode_noalloc(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                                const int32_t *cache_len, int T_cap, void *o, int B, int n, int Hq, int Hkv, int d,
                                hd_mode mode, int window, float scale, hd_dtype dt, void *stream) {
    return sfa_decode_common(q, k_new, v_new, k_cache, v_cache, cache_len, T_cap, o, B, n, Hq, Hkv, d, mode, window,
                             scale, dt, nullptr, 0, stream, false, true);
}

hd_status hd_sfa_decode_final(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                              const int32_t *cache_len, int T_cap, void *o, int B, int n, int Hq, int Hkv, int d,
                              hd_mode mode, int window, float scale, hd_dtype dt, void *workspace,
                              size_t workspace_bytes, void *stream) {
    return sfa_decode_common(q, k_new, v_new, k_cache, v_cache, cache_len, T_cap, o, B, n, Hq, Hkv, d, mode, window,
                             scale, dt, workspace, workspace_bytes, stream, true);
}

}  // extern "C"
