// Host-side driver for the sanitizer build of libhd's C ABI (test
// infrastructure).  Every entry point is called with arguments that fail
// validation, with extreme sizes (so that overflowing size arithmetic would
// be reported by UBSan), and -- only when no GPU is present -- with valid
// arguments, which then pass validation and fail at the launch.  Fake
// pointers are never dereferenced by host code.  Exit status 0 iff every
// call returned the expected status.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "hd.h"

static int g_fail = 0, g_calls = 0;

static void expect(const char *what, hd_status got, hd_status want) {
    ++g_calls;
    if (got != want) {
        std::printf("FAIL %s: got %s, want %s (%s)\n", what, hd_status_string(got), hd_status_string(want),
                    hd_last_error());
        ++g_fail;
    }
}

// With no device, a call that passes validation reports a launch failure.
static void expect_launch(const char *what, hd_status got, bool have_gpu) {
    if (have_gpu) return;
    expect(what, got, HD_ERR_DEVICE);
}

int main() {
    int ndev = 0;
    const bool have_gpu = hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0;
    void *F = reinterpret_cast<void *>(uintptr_t{0x10000});      // aligned, never dereferenced
    void *M = reinterpret_cast<void *>(uintptr_t{0x10008});      // misaligned
    float *Ff = static_cast<float *>(F);
    const int32_t *Fi = static_cast<const int32_t *>(F);
    const hd_mode I = HD_MODE_INTRA, C = HD_MODE_CROSS;

    for (int s = -1; s <= 4; ++s) (void)std::strlen(hd_status_string(static_cast<hd_status>(s)));
    (void)hd_version();

    // expansion
    const void *tabs[HD_MAX_STREAMS];
    for (auto &t : tabs) t = F;
    const void *bad_tabs[2] = {F, M};
    expect("embed B=0", hd_expand_embed(Fi, 0, 4, 2, tabs, 10, 8, HD_BF16, F, nullptr), HD_ERR_INVALID);
    expect("embed n=17", hd_expand_embed(Fi, 1, 4, 17, tabs, 10, 8, HD_BF16, F, nullptr), HD_ERR_INVALID);
    expect("embed tables", hd_expand_embed(Fi, 1, 4, 2, nullptr, 10, 8, HD_BF16, F, nullptr), HD_ERR_INVALID);
    expect("embed misaligned", hd_expand_embed(Fi, 1, 4, 2, bad_tabs, 10, 8, HD_BF16, F, nullptr), HD_ERR_INVALID);
    expect("embed dtype", hd_expand_embed(Fi, 1, 4, 2, tabs, 10, 8, (hd_dtype)7, F, nullptr), HD_ERR_UNSUPPORTED);
    expect("embed V=0", hd_expand_embed(Fi, 1, 4, 2, tabs, 0, 8, HD_BF16, F, nullptr), HD_ERR_INVALID);
    expect_launch("embed ok", hd_expand_embed(Fi, 64, 1, 4, tabs, 160000, 7168, HD_BF16, F, nullptr), have_gpu);
    expect_launch("embed 2-byte rows", hd_expand_embed(Fi, 3, 5, 16, tabs, 37, 7, HD_BF16, F, nullptr), have_gpu);

    // prefill (plain, final-stream, fused rotary)
    using Fwd = hd_status (*)(const void *, const void *, const void *, void *, float *, int, int, int, int, int,
                              int, hd_mode, int, float, hd_dtype, void *);
    const Fwd fwds[2] = {hd_sfa_fwd, hd_sfa_fwd_final};
    for (Fwd f : fwds) {
        expect("fwd B=0", f(F, F, F, F, nullptr, 0, 8, 2, 4, 2, 64, I, 0, 0.f, HD_BF16, nullptr), HD_ERR_INVALID);
        expect("fwd L=0", f(F, F, F, F, nullptr, 1, 0, 2, 4, 2, 64, I, 0, 0.f, HD_BF16, nullptr), HD_ERR_INVALID);
        expect("fwd Hq%Hkv", f(F, F, F, F, nullptr, 1, 8, 2, 3, 2, 64, I, 0, 0.f, HD_BF16, nullptr), HD_ERR_INVALID);
        expect("fwd window", f(F, F, F, F, nullptr, 1, 8, 2, 4, 2, 64, I, -1, 0.f, HD_BF16, nullptr), HD_ERR_INVALID);
        expect("fwd d", f(F, F, F, F, nullptr, 1, 8, 2, 4, 2, 96, I, 0, 0.f, HD_BF16, nullptr), HD_ERR_UNSUPPORTED);
        expect("fwd mode", f(F, F, F, F, nullptr, 1, 8, 2, 4, 2, 64, (hd_mode)3, 0, 0.f, HD_BF16, nullptr),
               HD_ERR_UNSUPPORTED);
        expect("fwd lse", f(F, F, F, F, reinterpret_cast<float *>(uintptr_t{0x10002}), 1, 8, 2, 4, 2, 64, I, 0, 0.f,
                            HD_BF16, nullptr), HD_ERR_INVALID);
        expect("fwd n*L", f(F, F, F, F, nullptr, 1, INT_MAX, 16, 4, 2, 64, C, 0, 0.f, HD_BF16, nullptr),
               HD_ERR_UNSUPPORTED);
        expect("fwd window huge", f(F, F, F, F, nullptr, 1, 8, 16, 4, 2, 64, C, INT_MAX, 0.f, HD_BF16, nullptr),
               have_gpu ? HD_OK : HD_ERR_DEVICE);
        for (int d : {32, 64, 128})
            for (hd_mode m : {I, C}) {
                expect_launch("fwd ok", f(F, F, F, F, Ff, 2, 4096, 4, 32, 8, d, m, 4096, 0.f, HD_BF16, nullptr), have_gpu);
                expect_launch("fwd f32", f(F, F, F, F, nullptr, 1, 64, 2, 4, 4, d, m, 0, 0.5f, HD_F32, nullptr), have_gpu);
            }
    }
    expect("rope theta", hd_sfa_fwd_rope(F, F, F, F, nullptr, F, 1, 8, 2, 4, 2, 64, I, 0, 0.f, 0.f, HD_BF16, nullptr),
           HD_ERR_INVALID);
    expect("rope k_rot", hd_sfa_fwd_rope(F, F, F, F, nullptr, M, 1, 8, 2, 4, 2, 64, I, 0, 0.f, 1e4f, HD_BF16, nullptr),
           HD_ERR_INVALID);
    expect_launch("fwd rope ok",
                  hd_sfa_fwd_rope(F, F, F, F, nullptr, F, 1, 4096, 4, 32, 8, 128, I, 0, 0.f, 1e4f, HD_BF16, nullptr),
                  have_gpu);
    expect("rope T=0", hd_rope(F, F, 1, 0, 2, 64, nullptr, 0, 1, 0, 1e4f, HD_BF16, nullptr), HD_ERR_INVALID);
    expect("rope mul", hd_rope(F, F, 1, 8, 2, 64, nullptr, -1, 1, 0, 1e4f, HD_BF16, nullptr), HD_ERR_INVALID);
    expect_launch("rope ok", hd_rope(F, F, 64, 1, 8, 128, Fi, 4, 1, 3, 1e4f, HD_BF16, nullptr), have_gpu);

    // decode (workspace, final-stream, allocation-free)
    const size_t ws = hd_sfa_decode_workspace_bytes(64, 4, 32, 8, 128, 8200);
    expect("decode ws nonzero", ws > 0 ? HD_OK : HD_ERR_INVALID, HD_OK);
    expect("decode ws bad", hd_sfa_decode_workspace_bytes(0, 4, 32, 8, 128, 8200) == 0 ? HD_OK : HD_ERR_INVALID,
           HD_OK);
    (void)hd_sfa_decode_workspace_bytes(INT_MAX, 16, 64 * 4, 4, 128, INT_MAX);
    (void)hd_sfa_decode_workspace_bytes(1, 1, 1, 1, 32, INT_MAX);
    using Dec = hd_status (*)(const void *, const void *, const void *, void *, void *, const int32_t *, int, void *,
                              int, int, int, int, int, hd_mode, int, float, hd_dtype, void *, size_t, void *);
    const Dec decs[2] = {hd_sfa_decode, hd_sfa_decode_final};
    for (Dec f : decs) {
        expect("decode T_cap", f(F, F, F, F, F, Fi, 0, F, 2, 4, 8, 2, 128, C, 0, 0.f, HD_BF16, F, ws, nullptr),
               HD_ERR_INVALID);
        expect("decode lens", f(F, F, F, F, F, nullptr, 16, F, 2, 4, 8, 2, 128, C, 0, 0.f, HD_BF16, F, ws, nullptr),
               HD_ERR_INVALID);
        expect("decode ws small", f(F, F, F, F, F, Fi, 8200, F, 64, 4, 32, 8, 128, C, 0, 0.f, HD_BF16, F, 16, nullptr),
               HD_ERR_INVALID);
        expect("decode rows", f(F, F, F, F, F, Fi, 16, F, 2, 8, 256, 2, 128, C, 0, 0.f, HD_BF16, F, ws, nullptr),
               HD_ERR_UNSUPPORTED);
        for (hd_mode m : {I, C}) {
            expect_launch("decode ok", f(F, F, F, F, F, Fi, 8200, F, 64, 4, 32, 8, 128, m, 0, 0.f, HD_BF16, F, ws, nullptr),
                          have_gpu);
            expect_launch("decode d64", f(F, F, F, F, F, Fi, 300, F, 2, 3, 12, 2, 64, m, 7, 0.f, HD_BF16, F,
                                          hd_sfa_decode_workspace_bytes(2, 3, 12, 2, 64, 300), nullptr), have_gpu);
            expect_launch("decode f32", f(F, F, F, F, F, Fi, 40, F, 2, 4, 8, 2, 32, m, 0, 0.f, HD_F32, nullptr, 0, nullptr),
                          have_gpu);
        }
    }
    expect("noalloc too big", hd_sfa_decode_noalloc(F, F, F, F, F, Fi, 64, F, 1024, 4, 32, 8, 128, C, 0, 0.f, HD_BF16,
                                                    nullptr), HD_ERR_INVALID);
    expect("noalloc lens", hd_sfa_decode_noalloc(F, F, F, F, F, nullptr, 64, F, 2, 4, 32, 8, 128, C, 0, 0.f, HD_BF16,
                                                 nullptr), HD_ERR_INVALID);
    if (!have_gpu)  // the scratch lookup itself fails without a device
        expect("noalloc no device", hd_sfa_decode_noalloc(F, F, F, F, F, Fi, 64, F, 2, 4, 32, 8, 128, C, 0, 0.f,
                                                          HD_BF16, nullptr), HD_ERR_DEVICE);

    // backward
    using Bwd = hd_status (*)(const void *, const void *, const void *, const void *, const void *, const float *,
                              void *, void *, void *, int, int, int, int, int, int, hd_mode, int, float, hd_dtype,
                              void *, size_t, void *);
    using BwdWs = size_t (*)(int, int, int, int, int, int, hd_dtype);
    const Bwd bwds[2] = {hd_sfa_bwd, hd_sfa_bwd_final};
    const BwdWs bwss[2] = {hd_sfa_bwd_workspace_bytes, hd_sfa_bwd_final_workspace_bytes};
    for (int e = 0; e < 2; ++e) {
        (void)bwss[e](INT_MAX, INT_MAX, 16, 64, 8, 128, HD_BF16);
        (void)bwss[e](64, 1 << 26, 16, 64, 1, 128, HD_BF16);
        (void)bwss[e](1, 1, 1, 1, 1, 32, HD_F32);
        const size_t need = bwss[e](1, 4096, 4, 32, 8, 128, HD_BF16);
        const size_t need1 = bwss[e](1, 4096, 1, 32, 8, 128, HD_BF16);
        expect("bwd dout", bwds[e](F, F, F, F, nullptr, Ff, F, F, F, 1, 8, 2, 4, 2, 64, I, 0, 0.f, HD_BF16, F, 1 << 20,
                                   nullptr), HD_ERR_INVALID);
        expect("bwd ws small", bwds[e](F, F, F, F, F, Ff, F, F, F, 1, 4096, 4, 32, 8, 128, I, 0, 0.f, HD_BF16, F,
                                       need - 1, nullptr), HD_ERR_INVALID);
        expect("bwd d", bwds[e](F, F, F, F, F, Ff, F, F, F, 1, 8, 2, 4, 2, 96, I, 0, 0.f, HD_BF16, F, 1 << 20, nullptr),
               HD_ERR_UNSUPPORTED);
        for (hd_mode m : {I, C}) {
            expect_launch("bwd ok", bwds[e](F, F, F, F, F, Ff, F, F, F, 1, 4096, 4, 32, 8, 128, m, 0, 0.f, HD_BF16, F,
                                            need, nullptr), have_gpu);
            expect_launch("bwd segments", bwds[e](F, F, F, F, F, Ff, F, F, F, 1, 4096, 1, 32, 8, 128, m, 64, 0.f, HD_BF16,
                                                  F, need1, nullptr), have_gpu);
            expect_launch("bwd f32", bwds[e](F, F, F, F, F, Ff, F, F, F, 1, 64, 2, 4, 2, 32, m, 0, 0.f, HD_F32, F,
                                             bwss[e](1, 64, 2, 4, 2, 32, HD_F32), nullptr), have_gpu);
        }
    }

    std::printf("%d calls, %d failures%s\n", g_calls, g_fail, have_gpu ? " (GPU present: launches skipped)" : "");
    return g_fail == 0 ? 0 : 1;
}
