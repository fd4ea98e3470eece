"""C-ABI checks that need no GPU: libhd.so loads, exports every symbol that
include/hd.h declares, and rejects bad arguments on the host before any HIP
call (every call below fails validation, so nothing is launched)."""
import ctypes
import os
import re

import pytest
import torch

from latent_sequence_length_amd import hd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hd.h")


@pytest.fixture(scope="module")
def lib():
    from latent_sequence_length_amd import build

    srcs = build.sources()
    if not os.path.exists(hd.LIB_PATH) or os.path.getmtime(hd.LIB_PATH) < max(
            os.path.getmtime(s) for s in srcs + [HEADER]):
        build.build()
    return hd.load()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hd_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_symbols() == sorted([
        "hd_expand_embed", "hd_rope", "hd_sfa_fwd", "hd_sfa_fwd_final", "hd_sfa_fwd_rope",
        "hd_sfa_bwd_workspace_bytes", "hd_sfa_bwd",
        "hd_sfa_bwd_final_workspace_bytes", "hd_sfa_bwd_final",
        "hd_sfa_decode_workspace_bytes", "hd_sfa_decode", "hd_sfa_decode_final", "hd_sfa_decode_noalloc",
        "hd_status_string", "hd_last_error", "hd_version"])


def test_every_declared_symbol_is_exported(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {hd.LIB_PATH}").read()
    for name in declared_symbols():
        assert re.search(rf"\bT {name}$", out, re.M), name


def test_status_strings(lib):
    assert [hd.status_string(s) for s in range(4)] == [
        "HD_OK", "HD_ERR_INVALID", "HD_ERR_UNSUPPORTED", "HD_ERR_DEVICE"]
    assert lib.hd_version() >= 100


FAKE = 0x10000  # aligned non-null address; never dereferenced (validation fails first)


def fwd(lib, entry="hd_sfa_fwd", **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, L=8, n=2, Hq=4, Hkv=2, d=64,
             mode=0, window=0, scale=0.0, dt=0, stream=None)
    a.update(kw)
    return getattr(lib, entry)(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), hd.HD_ERR_INVALID), (dict(L=0), hd.HD_ERR_INVALID), (dict(n=0), hd.HD_ERR_INVALID),
    (dict(n=17), hd.HD_ERR_INVALID), (dict(Hq=3), hd.HD_ERR_INVALID), (dict(Hkv=0), hd.HD_ERR_INVALID),
    (dict(window=-1), hd.HD_ERR_INVALID), (dict(q=None), hd.HD_ERR_INVALID),
    (dict(k=FAKE + 8), hd.HD_ERR_INVALID), (dict(o=None), hd.HD_ERR_INVALID),
    (dict(lse=FAKE + 2), hd.HD_ERR_INVALID),
    (dict(d=96), hd.HD_ERR_UNSUPPORTED), (dict(d=16), hd.HD_ERR_UNSUPPORTED),
    (dict(dt=7), hd.HD_ERR_UNSUPPORTED), (dict(mode=2), hd.HD_ERR_UNSUPPORTED),
    (dict(L=1 << 29, n=4), hd.HD_ERR_UNSUPPORTED),
])
@pytest.mark.parametrize("entry", ["hd_sfa_fwd", "hd_sfa_fwd_final"])
def test_fwd_validation(lib, kw, code, entry):
    assert fwd(lib, entry, **kw) == code
    assert hd.last_error() != ""


def fwd_rope(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, k_rot=FAKE, B=1, L=8, n=2, Hq=4, Hkv=2, d=64,
             mode=0, window=0, scale=0.0, theta=10000.0, dt=0, stream=None)
    a.update(kw)
    return lib.hd_sfa_fwd_rope(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(theta=0.0), hd.HD_ERR_INVALID), (dict(theta=-1.0), hd.HD_ERR_INVALID),
    (dict(theta=float("inf")), hd.HD_ERR_INVALID), (dict(k_rot=None), hd.HD_ERR_INVALID),
    (dict(k_rot=FAKE + 8), hd.HD_ERR_INVALID), (dict(B=0), hd.HD_ERR_INVALID), (dict(Hq=3), hd.HD_ERR_INVALID),
    (dict(d=96), hd.HD_ERR_UNSUPPORTED), (dict(mode=2), hd.HD_ERR_UNSUPPORTED),
])
def test_fwd_rope_validation(lib, kw, code):
    assert fwd_rope(lib, **kw) == code
    assert hd.last_error() != ""


def dec(lib, **kw):
    a = dict(q=FAKE, k_new=FAKE, v_new=FAKE, k_cache=FAKE, v_cache=FAKE, cache_len=FAKE, T_cap=16,
             o=FAKE, B=2, n=4, Hq=8, Hkv=2, d=128, mode=1, window=0, scale=0.0, dt=0,
             workspace=FAKE, workspace_bytes=0, stream=None)
    a.update(kw)
    return lib.hd_sfa_decode(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(T_cap=0), hd.HD_ERR_INVALID), (dict(B=0), hd.HD_ERR_INVALID), (dict(Hq=6, Hkv=4), hd.HD_ERR_INVALID),
    (dict(cache_len=None), hd.HD_ERR_INVALID), (dict(k_cache=FAKE + 4), hd.HD_ERR_INVALID),
    (dict(workspace_bytes=16), hd.HD_ERR_INVALID),  # too small for the bf16 path
    (dict(n=8, Hq=32, Hkv=2), hd.HD_ERR_UNSUPPORTED),  # 8*16 = 128 query rows per kv head
    (dict(d=48), hd.HD_ERR_UNSUPPORTED), (dict(window=-3), hd.HD_ERR_INVALID),
])
def test_decode_validation(lib, kw, code):
    assert dec(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(T_cap=0), hd.HD_ERR_INVALID), (dict(cache_len=None), hd.HD_ERR_INVALID),
    (dict(workspace_bytes=16), hd.HD_ERR_INVALID), (dict(d=48), hd.HD_ERR_UNSUPPORTED),
    (dict(Hq=130, Hkv=2), hd.HD_ERR_UNSUPPORTED),   # 65 final-stream rows per kv head
])
def test_decode_final_validation(lib, kw, code):
    a = dict(q=FAKE, k_new=FAKE, v_new=FAKE, k_cache=FAKE, v_cache=FAKE, cache_len=FAKE, T_cap=16,
             o=FAKE, B=2, n=4, Hq=8, Hkv=2, d=128, mode=1, window=0, scale=0.0, dt=0,
             workspace=FAKE, workspace_bytes=0, stream=None)
    a.update(kw)
    assert lib.hd_sfa_decode_final(*a.values()) == code


@pytest.mark.parametrize("kw,code", [
    (dict(T_cap=0), hd.HD_ERR_INVALID), (dict(B=0), hd.HD_ERR_INVALID), (dict(Hq=6, Hkv=4), hd.HD_ERR_INVALID),
    (dict(cache_len=None), hd.HD_ERR_INVALID), (dict(d=48), hd.HD_ERR_UNSUPPORTED),
    (dict(n=8, Hq=32, Hkv=2), hd.HD_ERR_UNSUPPORTED),
    # 1024 sequences need 68 MB of split-KV partials, above the 32 MiB scratch
    (dict(B=1024, n=4, Hq=32, Hkv=8, T_cap=64), hd.HD_ERR_INVALID),
])
def test_decode_noalloc_validation(lib, kw, code):
    a = dict(q=FAKE, k_new=FAKE, v_new=FAKE, k_cache=FAKE, v_cache=FAKE, cache_len=FAKE, T_cap=16,
             o=FAKE, B=2, n=4, Hq=8, Hkv=2, d=128, mode=1, window=0, scale=0.0, dt=0, stream=None)
    a.update(kw)
    assert lib.hd_sfa_decode_noalloc(*a.values()) == code
    if kw.get("B") == 1024:
        assert "scratch" in hd.last_error()


def test_workspace_size_is_monotone_and_zero_on_bad_sizes(lib):
    f = hd.hd_sfa_decode_workspace_bytes
    assert f(0, 4, 32, 8, 128, 8193) == 0
    assert f(64, 4, 30, 8, 128, 8193) == 0
    a, b = f(64, 4, 32, 8, 128, 8193), f(64, 4, 32, 8, 128, 16385)
    assert 0 < a <= b
    # partials: B*n*Hq*(d+2) floats per split
    assert a % (64 * 4 * 32 * 130 * 4) == 0


def bwd(lib, entry="hd_sfa_bwd", **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, dout=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             B=1, L=8, n=2, Hq=4, Hkv=2, d=64, mode=0, window=0, scale=0.0, dt=0,
             workspace=FAKE, workspace_bytes=1 << 20, stream=None)
    a.update(kw)
    return getattr(lib, entry)(*a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), hd.HD_ERR_INVALID), (dict(L=0), hd.HD_ERR_INVALID), (dict(Hq=3), hd.HD_ERR_INVALID),
    (dict(window=-1), hd.HD_ERR_INVALID), (dict(dout=None), hd.HD_ERR_INVALID),
    (dict(lse=None), hd.HD_ERR_INVALID), (dict(lse=FAKE + 4), hd.HD_ERR_INVALID),
    (dict(dk=FAKE + 8), hd.HD_ERR_INVALID), (dict(workspace=None), hd.HD_ERR_INVALID),
    (dict(workspace_bytes=1 * 4 * 16 * 4 - 1), hd.HD_ERR_INVALID),   # B*Hq*nL*4 = 256 bytes needed
    (dict(d=96), hd.HD_ERR_UNSUPPORTED), (dict(dt=3), hd.HD_ERR_UNSUPPORTED), (dict(mode=5), hd.HD_ERR_UNSUPPORTED),
])
def test_bwd_validation(lib, kw, code):
    assert bwd(lib, **kw) == code
    assert hd.last_error() != ""


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), hd.HD_ERR_INVALID), (dict(Hq=3), hd.HD_ERR_INVALID), (dict(dv=None), hd.HD_ERR_INVALID),
    (dict(workspace_bytes=1 * 4 * 8 * 4 - 1), hd.HD_ERR_INVALID),   # B*Hq*L*4 = 128 bytes needed
    (dict(d=16), hd.HD_ERR_UNSUPPORTED), (dict(mode=2), hd.HD_ERR_UNSUPPORTED),
    (dict(L=1 << 29, n=4), hd.HD_ERR_UNSUPPORTED),
])
def test_bwd_final_validation(lib, kw, code):
    assert bwd(lib, "hd_sfa_bwd_final", **kw) == code
    assert hd.last_error() != ""


def bwd_ws_model(B, L, n, Hq, Hkv, d, final_only):
    """The documented workspace rule: the per-row D array (rounded up to 256
    bytes) plus, when the dK/dV pass has fewer than 4096 key waves of 32 keys
    and at least 256 queries, fp32 partial dK/dV rows of nseg query segments
    (about 8192 / waves segments, at most 8, of >= 128 queries, a multiple of
    32); the larger of the intra and cross layers."""
    def ceil(a, b):
        return -(-a // b)

    need = 0
    for cross in (False, True):
        if final_only:
            nsub, Lsub, Lq, qrows = 1, (n * L if cross else L), L, L
        else:
            nsub, Lsub = (1, n * L) if cross else (n, L)
            Lq, qrows = Lsub, n * L
        total = (B * Hq * qrows * 4 + 255) // 256 * 256
        waves = B * Hkv * nsub * ((Lsub + 31) // 32)
        if waves < 4096 and Lq >= 256:
            want = min(8, ceil(8192, waves))
            segq = max(128, ceil(ceil(Lq, want), 32) * 32)
            nseg = ceil(Lq, segq)
            if nseg > 1:
                total += nseg * B * nsub * Hkv * Lsub * 2 * d * 4
        need = max(need, total)
    return need


def test_bwd_workspace_size(lib):
    f = hd.hd_sfa_bwd_workspace_bytes
    assert f(1, 4096, 4, 32, 8, 128) == 4096 * 4 * 32 * 4  # 4096 key waves in both layers: D only
    # n = 1 control: 1024 key waves -> 8 segments of 512 queries
    assert f(1, 4096, 1, 32, 8, 128) == 4096 * 32 * 4 + 8 * 8 * 4096 * 2 * 128 * 4
    # cross layer of 300 positions: 40 key waves -> 3 segments of 128 queries
    assert f(2, 100, 3, 8, 2, 64) == 2 * 8 * 300 * 4 + 3 * 2 * 2 * 300 * 2 * 64 * 4
    assert f(0, 8, 2, 4, 2, 64) == 0 and f(1, 8, 2, 4, 3, 64) == 0 and f(1, 8, 2, 4, 2, 96) == 0
    ff = hd.hd_sfa_bwd_final_workspace_bytes
    assert ff(1, 4096, 4, 32, 8, 128) == 4096 * 32 * 4 + 8 * 8 * 4096 * 2 * 128 * 4  # intra: stream 3's keys
    assert ff(2, 100, 3, 8, 2, 64) == (2 * 8 * 100 * 4 + 255) // 256 * 256
    assert ff(0, 8, 2, 4, 2, 64) == 0 and ff(1, 8, 2, 4, 2, 96) == 0
    for shape in [(1, 300, 4, 8, 2, 128), (2, 150, 3, 8, 2, 128), (1, 257, 4, 8, 8, 64), (1, 97, 1, 6, 3, 64),
                  (1, 200, 8, 4, 1, 128), (3, 1, 4, 4, 1, 128), (1, 32768, 4, 16, 4, 128), (4, 1000, 2, 8, 8, 32)]:
        assert f(*shape) == bwd_ws_model(*shape, False), shape
        assert ff(*shape) == bwd_ws_model(*shape, True), shape
    # the float32 path needs the D array only
    assert f(1, 4096, 1, 32, 8, 128, torch.float32) == 4096 * 32 * 4


def test_rope_validation(lib):
    f = lib.hd_rope
    ok = dict(x=FAKE, out=FAKE, B=1, T=8, H=2, d=64, pos_base=None, pos_mul=0, t_mul=1, t_add=0, theta=10000.0,
              dt=0, stream=None)
    for kw, code in [(dict(B=0), hd.HD_ERR_INVALID), (dict(T=0), hd.HD_ERR_INVALID), (dict(d=48), hd.HD_ERR_UNSUPPORTED),
                     (dict(theta=0.0), hd.HD_ERR_INVALID), (dict(theta=-1.0), hd.HD_ERR_INVALID),
                     (dict(pos_mul=-1), hd.HD_ERR_INVALID), (dict(t_mul=-1), hd.HD_ERR_INVALID),
                     (dict(t_add=-3), hd.HD_ERR_INVALID), (dict(x=None), hd.HD_ERR_INVALID),
                     (dict(out=FAKE + 2), hd.HD_ERR_INVALID), (dict(pos_base=FAKE + 2), hd.HD_ERR_INVALID),
                     (dict(dt=9), hd.HD_ERR_UNSUPPORTED)]:
        a = dict(ok)
        a.update(kw)
        assert f(*a.values()) == code, kw


def test_embed_validation(lib):
    tabs = (ctypes.c_void_p * 2)(FAKE, FAKE)
    f = lib.hd_expand_embed
    assert f(FAKE, 0, 4, 2, tabs, 10, 8, 0, FAKE, None) == hd.HD_ERR_INVALID
    assert f(FAKE, 1, 4, 0, tabs, 10, 8, 0, FAKE, None) == hd.HD_ERR_INVALID
    assert f(FAKE, 1, 4, 2, None, 10, 8, 0, FAKE, None) == hd.HD_ERR_INVALID
    assert f(FAKE, 1, 4, 2, tabs, 0, 8, 0, FAKE, None) == hd.HD_ERR_INVALID
    assert f(FAKE, 1, 4, 2, tabs, 10, 8, 5, FAKE, None) == hd.HD_ERR_UNSUPPORTED
    bad = (ctypes.c_void_p * 2)(FAKE, FAKE + 2)
    assert f(FAKE, 1, 4, 2, bad, 10, 8, 0, FAKE, None) == hd.HD_ERR_INVALID
    assert f(None, 1, 4, 2, tabs, 10, 8, 0, FAKE, None) == hd.HD_ERR_INVALID


def test_binding_refuses_cpu_tensors(lib):
    import torch

    q = torch.zeros(1, 8, 2, 32, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        hd.sfa_fwd(q, q, q, 2, 0)


# ---------------------------------------------------------------------------
# Debug mode of the binding (HD_DEBUG=1): the two caller contracts the C ABI
# does not check on the host -- ids in [0, V), cache_len in [0, T_cap) -- are
# checked before anything reaches the library.  The tensors here live on the
# CPU: with the contract broken the wrapper raises ValueError before it looks
# at the device; with it kept, the call gets as far as the GPU-tensor check.
# ---------------------------------------------------------------------------

def _embed_args(ids):
    tabs = [torch.zeros(10, 8, dtype=torch.bfloat16) for _ in range(2)]
    out = torch.empty(ids.shape[0], 2 * ids.shape[1], 8, dtype=torch.bfloat16)
    return ids, tabs, out


@pytest.mark.parametrize("bad", [-1, 10, 1 << 20])
def test_debug_mode_rejects_ids_outside_the_table(monkeypatch, bad):
    monkeypatch.setenv("HD_DEBUG", "1")
    ids = torch.tensor([[0, 3, bad, 9]], dtype=torch.int32)
    with pytest.raises(ValueError, match=r"\[0, 10\)"):
        hd.hd_expand_embed(*_embed_args(ids))


def test_debug_mode_passes_valid_ids_on(monkeypatch):
    monkeypatch.setenv("HD_DEBUG", "1")
    ids = torch.tensor([[0, 3, 9, 9]], dtype=torch.int32)
    with pytest.raises(TypeError, match="GPU tensor"):
        hd.hd_expand_embed(*_embed_args(ids))


def test_debug_mode_off_by_default(monkeypatch):
    monkeypatch.delenv("HD_DEBUG", raising=False)
    ids = torch.tensor([[0, 3, 77, 9]], dtype=torch.int32)
    with pytest.raises(TypeError, match="GPU tensor"):  # no id check without debug mode
        hd.hd_expand_embed(*_embed_args(ids))


def _decode_args(lens, T_cap=16):
    B, n, Hq, Hkv, d = len(lens), 2, 4, 2, 32
    q = torch.zeros(B, n, Hq, d, dtype=torch.bfloat16)
    kn = torch.zeros(B, n, Hkv, d, dtype=torch.bfloat16)
    kc = torch.zeros(B, T_cap, n, Hkv, d, dtype=torch.bfloat16)
    cl = torch.tensor(lens, dtype=torch.int32)
    return q, kn, kn.clone(), kc, kc.clone(), cl, torch.empty_like(q)


@pytest.mark.parametrize("lens", [[3, 16], [-1, 0], [15, 40]])
@pytest.mark.parametrize("entry", ["hd_sfa_decode", "hd_sfa_decode_noalloc"])
def test_debug_mode_rejects_cache_len_outside_the_cache(monkeypatch, lens, entry):
    monkeypatch.setenv("HD_DEBUG", "1")
    with pytest.raises(ValueError, match="T_cap=16"):
        getattr(hd, entry)(*_decode_args(lens), 0)


def test_debug_mode_rejects_cache_len_of_final_stream_decode(monkeypatch):
    monkeypatch.setenv("HD_DEBUG", "1")
    q, kn, vn, kc, vc, cl, _ = _decode_args([2, 16])
    qf = q[:, 1:].contiguous()
    with pytest.raises(ValueError, match="T_cap=16"):
        hd.hd_sfa_decode(qf, kn, vn, kc, vc, cl, torch.empty_like(qf), 1, final_only=True)


@pytest.mark.parametrize("entry", ["hd_sfa_decode", "hd_sfa_decode_noalloc"])
def test_debug_mode_passes_valid_cache_len_on(monkeypatch, entry):
    monkeypatch.setenv("HD_DEBUG", "1")
    with pytest.raises(TypeError, match="GPU tensor"):
        getattr(hd, entry)(*_decode_args([0, 15]), 0)
