"""Thin ctypes binding over libhd.so (include/hd.h), same names as the C ABI.

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current HIP stream.  There is no
fallback: if ``libhd.so`` is absent or a tensor is not on the GPU, the call
raises.

Debug mode (environment variable ``HD_DEBUG=1``): the two caller contracts
the C ABI cannot check without synchronising -- token ids in [0, V) for the
expansion, ``cache_len[b]`` in [0, T_cap) for a decode step -- are checked
here before anything is launched (one device-to-host read each), raising
ValueError.
"""
import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhd.so")

HD_OK, HD_ERR_INVALID, HD_ERR_UNSUPPORTED, HD_ERR_DEVICE = 0, 1, 2, 3
HD_MODE_INTRA, HD_MODE_CROSS = 0, 1
HD_BF16, HD_F32 = 0, 1
HD_MAX_STREAMS = 16

_DT = {torch.bfloat16: HD_BF16, torch.float32: HD_F32}
_lib = None


class HDError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{status_string(status)}: {detail}")


def load():
    """Load libhd.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m latent_sequence_length_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.hd_expand_embed.argtypes = [P, I, I, I, P, I64, I, I, P, P]
    lib.hd_sfa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, P]
    lib.hd_sfa_fwd_final.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, P]
    lib.hd_sfa_fwd_rope.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, F, I, P]
    lib.hd_sfa_decode_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.hd_sfa_decode_workspace_bytes.restype = SZ
    lib.hd_sfa_decode.argtypes = [P, P, P, P, P, P, I, P, I, I, I, I, I, I, I, F, I, P, SZ, P]
    lib.hd_sfa_decode_final.argtypes = [P, P, P, P, P, P, I, P, I, I, I, I, I, I, I, F, I, P, SZ, P]
    lib.hd_sfa_decode_noalloc.argtypes = [P, P, P, P, P, P, I, P, I, I, I, I, I, I, I, F, I, P]
    lib.hd_sfa_bwd_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.hd_sfa_bwd_workspace_bytes.restype = SZ
    lib.hd_sfa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, P, SZ, P]
    lib.hd_sfa_bwd_final_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.hd_sfa_bwd_final_workspace_bytes.restype = SZ
    lib.hd_sfa_bwd_final.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, P, SZ, P]
    lib.hd_rope.argtypes = [P, P, I, I, I, I, P, I64, I64, I64, F, I, P]
    for f in (lib.hd_expand_embed, lib.hd_sfa_fwd, lib.hd_sfa_fwd_final, lib.hd_sfa_fwd_rope, lib.hd_sfa_decode,
              lib.hd_sfa_decode_final, lib.hd_sfa_decode_noalloc, lib.hd_sfa_bwd, lib.hd_sfa_bwd_final, lib.hd_rope):
        f.restype = ctypes.c_int
    lib.hd_status_string.argtypes = [I]
    lib.hd_status_string.restype = ctypes.c_char_p
    lib.hd_last_error.argtypes = []
    lib.hd_last_error.restype = ctypes.c_char_p
    lib.hd_version.argtypes = []
    lib.hd_version.restype = I
    _lib = lib
    return lib


def status_string(s):
    return load().hd_status_string(int(s)).decode()


def last_error():
    return load().hd_last_error().decode()


def debug_enabled():
    """True when HD_DEBUG=1: the wrapper checks ids and cache lengths."""
    return os.environ.get("HD_DEBUG", "") == "1"


def _debug_check_ids(ids, V):
    """Every id in [0, V) (debug mode only; reads ids back to the host)."""
    if ids.numel() == 0:
        return
    lo, hi = int(ids.min()), int(ids.max())
    if lo < 0 or hi >= V:
        raise ValueError(f"token ids must lie in [0, {V}); found min {lo}, max {hi}")


def _debug_check_lens(cache_len, T_cap):
    """Every cache_len[b] in [0, T_cap) (debug mode only)."""
    lo, hi = int(cache_len.min()), int(cache_len.max())
    if lo < 0 or hi >= T_cap:
        raise ValueError(f"cache_len must lie in [0, T_cap={T_cap}) so the new token fits; "
                         f"found min {lo}, max {hi}")


def _check(status):
    if status != HD_OK:
        raise HDError(status, last_error())


def _dev(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _dtype_code(t):
    if t.dtype not in _DT:
        raise TypeError(f"dtype {t.dtype} not supported (bfloat16, float32)")
    return _DT[t.dtype]


# --------------------------------------------------------------------------
# Raw entry points (caller allocates every output), same names as the C ABI.
# --------------------------------------------------------------------------

def hd_expand_embed(ids, tables, out):
    """out[b, i*n+s, :] = tables[s][ids[b, i], :]  (ids int32 [B, L])."""
    n = len(tables)
    if not 1 <= n <= HD_MAX_STREAMS:
        raise ValueError(f"need 1..{HD_MAX_STREAMS} tables, got {n}")
    B, L = ids.shape
    V, D = tables[0].shape
    for t in tables:
        if t.shape != (V, D) or t.dtype != tables[0].dtype:
            raise ValueError("tables must share shape and dtype")
    if out.shape != (B, n * L, D) or out.dtype != tables[0].dtype:
        raise ValueError(f"out must be {(B, n * L, D)} of {tables[0].dtype}")
    if debug_enabled():
        _debug_check_ids(ids, V)
    ptrs = (ctypes.c_void_p * n)(*[_dev(t, f"tables[{s}]") for s, t in enumerate(tables)])
    _check(load().hd_expand_embed(_dev(ids, "ids", torch.int32), B, L, n, ptrs, V, D,
                                  _dtype_code(tables[0]), _dev(out, "out"), _stream(out)))
    return out


def hd_sfa_fwd(q, k, v, o, n, mode, window=0, scale=0.0, lse=None):
    """Stream-Factorized Attention prefill into o (and lse [B, Hq, nL] if given)."""
    B, nL, Hq, d = q.shape
    Hkv = k.shape[2]
    if nL % n:
        raise ValueError(f"sequence length {nL} is not a multiple of n={n}")
    if k.shape != (B, nL, Hkv, d) or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("shape mismatch among q, k, v, o")
    dt = _dtype_code(q)
    for t, name in ((k, "k"), (v, "v"), (o, "o")):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} dtype {t.dtype} differs from q's {q.dtype}")
    lp = None
    if lse is not None:
        if lse.shape != (B, Hq, nL):
            raise ValueError(f"lse must be {(B, Hq, nL)}")
        lp = _dev(lse, "lse", torch.float32)
    _check(load().hd_sfa_fwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), lp,
                             B, nL // n, n, Hq, Hkv, d, int(mode), int(window), float(scale), dt,
                             _stream(q)))
    return o


def hd_sfa_fwd_final(q, k, v, o, n, mode, window=0, scale=0.0, lse=None):
    """Final-stream queries of a KV-mirror layer: q, o [B, L, Hq, d] hold the
    rows of stream n-1 only; k, v [B, n*L, Hkv, d]; lse [B, Hq, L] if given."""
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, n * L, Hkv, d) or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("shape mismatch among q [B, L, Hq, d], k/v [B, n*L, Hkv, d], o")
    dt = _dtype_code(q)
    for t, name in ((k, "k"), (v, "v"), (o, "o")):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} dtype {t.dtype} differs from q's {q.dtype}")
    lp = None
    if lse is not None:
        if lse.shape != (B, Hq, L):
            raise ValueError(f"lse must be {(B, Hq, L)}")
        lp = _dev(lse, "lse", torch.float32)
    _check(load().hd_sfa_fwd_final(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), lp,
                                   B, L, n, Hq, Hkv, d, int(mode), int(window), float(scale), dt, _stream(q)))
    return o


def hd_sfa_fwd_rope(q, k, v, o, k_rot, n, mode, window=0, scale=0.0, theta=10000.0, lse=None):
    """Prefill with RoPE at the expanded positions fused in: k rotated into
    k_rot, q rotated inside the kernel; o (and lse) as hd_sfa_fwd."""
    B, nL, Hq, d = q.shape
    Hkv = k.shape[2]
    if nL % n:
        raise ValueError(f"sequence length {nL} is not a multiple of n={n}")
    if k.shape != (B, nL, Hkv, d) or v.shape != k.shape or o.shape != q.shape or k_rot.shape != k.shape:
        raise ValueError("shape mismatch among q, k, v, o, k_rot")
    dt = _dtype_code(q)
    for t, name in ((k, "k"), (v, "v"), (o, "o"), (k_rot, "k_rot")):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} dtype {t.dtype} differs from q's {q.dtype}")
    lp = None
    if lse is not None:
        if lse.shape != (B, Hq, nL):
            raise ValueError(f"lse must be {(B, Hq, nL)}")
        lp = _dev(lse, "lse", torch.float32)
    _check(load().hd_sfa_fwd_rope(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), lp, _dev(k_rot, "k_rot"),
                                  B, nL // n, n, Hq, Hkv, d, int(mode), int(window), float(scale), float(theta), dt,
                                  _stream(q)))
    return o, k_rot


def hd_sfa_decode_workspace_bytes(B, n, Hq, Hkv, d, T_cap):
    return int(load().hd_sfa_decode_workspace_bytes(B, n, Hq, Hkv, d, T_cap))


def _decode_shapes(q, k_new, v_new, k_cache, v_cache, cache_len, o, final_only):
    """Validate the decode tensors; returns (B, n, Hq, Hkv, d, T_cap, dtype code)."""
    B, nq, Hq, d = q.shape
    n = k_new.shape[1]
    if nq != (1 if final_only else n):
        raise ValueError(f"q must be [B, {1 if final_only else n}, Hq, d]")
    Hkv = k_new.shape[2]
    T_cap = k_cache.shape[1]
    if k_new.shape != (B, n, Hkv, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must be [B, n, Hkv, d]")
    if k_cache.shape != (B, T_cap, n, Hkv, d) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B, T_cap, n, Hkv, d]")
    if o.shape != q.shape or cache_len.shape != (B,):
        raise ValueError("o must match q and cache_len must be [B]")
    dt = _dtype_code(q)
    for t, name in ((k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache"), (o, "o")):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} dtype {t.dtype} differs from q's {q.dtype}")
    if debug_enabled():
        _debug_check_lens(cache_len, T_cap)
    return B, n, Hq, Hkv, d, T_cap, dt


def hd_sfa_decode(q, k_new, v_new, k_cache, v_cache, cache_len, o, mode, window=0, scale=0.0,
                  workspace=None, final_only=False):
    """One decode step: append k_new/v_new at cache_len, attend, write o.
    final_only: q and o are [B, 1, Hq, d], the final stream's query of a
    KV-mirror layer (hd_sfa_decode_final)."""
    B, n, Hq, Hkv, d, T_cap, dt = _decode_shapes(q, k_new, v_new, k_cache, v_cache, cache_len, o, final_only)
    need = hd_sfa_decode_workspace_bytes(B, n, Hq, Hkv, d, T_cap)
    if workspace is None and dt == HD_BF16:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    wp = _dev(workspace, "workspace") if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    entry = load().hd_sfa_decode_final if final_only else load().hd_sfa_decode
    _check(entry(_dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                 _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                 _dev(cache_len, "cache_len", torch.int32), T_cap, _dev(o, "o"),
                 B, n, Hq, Hkv, d, int(mode), int(window), float(scale), dt,
                 wp, wbytes, _stream(q)))
    return o


def hd_sfa_decode_noalloc(q, k_new, v_new, k_cache, v_cache, cache_len, o, mode, window=0, scale=0.0):
    """hd_sfa_decode without a workspace: the library's own per-GPU scratch
    holds the split-KV partials (HD_NOALLOC_SCRATCH_BYTES at most)."""
    B, n, Hq, Hkv, d, T_cap, dt = _decode_shapes(q, k_new, v_new, k_cache, v_cache, cache_len, o, False)
    _check(load().hd_sfa_decode_noalloc(_dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                                        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                        _dev(cache_len, "cache_len", torch.int32), T_cap, _dev(o, "o"),
                                        B, n, Hq, Hkv, d, int(mode), int(window), float(scale), dt, _stream(q)))
    return o


def hd_rope(x, out, theta=10000.0, pos_base=None, pos_mul=0, t_mul=1, t_add=0):
    """Rotary embedding of x [B, T, H, d] at positions
    t*t_mul + t_add + pos_mul*pos_base[b] into out (may be x)."""
    B, T, H, d = x.shape
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    pb = None
    if pos_base is not None:
        if pos_base.shape != (B,):
            raise ValueError("pos_base must be [B]")
        pb = _dev(pos_base, "pos_base", torch.int32)
    _check(load().hd_rope(_dev(x, "x"), _dev(out, "out"), B, T, H, d, pb, int(pos_mul), int(t_mul), int(t_add),
                          float(theta), _dtype_code(x), _stream(x)))
    return out


def hd_sfa_bwd_workspace_bytes(B, L, n, Hq, Hkv, d, dtype=torch.bfloat16):
    return int(load().hd_sfa_bwd_workspace_bytes(B, L, n, Hq, Hkv, d, _DT[dtype]))


def hd_sfa_bwd(q, k, v, o, dout, lse, dq, dk, dv, n, mode, window=0, scale=0.0, workspace=None):
    """Gradients of sum(dout * o) into dq, dk, dv (lse from hd_sfa_fwd)."""
    B, nL, Hq, d = q.shape
    Hkv = k.shape[2]
    if nL % n:
        raise ValueError(f"sequence length {nL} is not a multiple of n={n}")
    if (k.shape != (B, nL, Hkv, d) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape
            or dq.shape != q.shape or dk.shape != k.shape or dv.shape != k.shape):
        raise ValueError("shape mismatch among q, k, v, o, dout, dq, dk, dv")
    if lse.shape != (B, Hq, nL):
        raise ValueError(f"lse must be {(B, Hq, nL)}")
    dt = _dtype_code(q)
    for t, name in ((k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} dtype {t.dtype} differs from q's {q.dtype}")
    if workspace is None:
        need = hd_sfa_bwd_workspace_bytes(B, nL // n, n, Hq, Hkv, d, q.dtype)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    _check(load().hd_sfa_bwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), _dev(dout, "dout"),
                             _dev(lse, "lse", torch.float32), _dev(dq, "dq"), _dev(dk, "dk"), _dev(dv, "dv"),
                             B, nL // n, n, Hq, Hkv, d, int(mode), int(window), float(scale), dt,
                             _dev(workspace, "workspace"), wbytes, _stream(q)))
    return dq, dk, dv


def hd_sfa_bwd_final_workspace_bytes(B, L, n, Hq, Hkv, d, dtype=torch.bfloat16):
    return int(load().hd_sfa_bwd_final_workspace_bytes(B, L, n, Hq, Hkv, d, _DT[dtype]))


def hd_sfa_bwd_final(q, k, v, o, dout, lse, dq, dk, dv, n, mode, window=0, scale=0.0, workspace=None):
    """Backward of the final-stream queries: q, o, dout, dq [B, L, Hq, d];
    k, v, dk, dv [B, n*L, Hkv, d]; lse [B, Hq, L] from hd_sfa_fwd_final."""
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    if (k.shape != (B, n * L, Hkv, d) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape
            or dq.shape != q.shape or dk.shape != k.shape or dv.shape != k.shape):
        raise ValueError("shape mismatch among q, k, v, o, dout, dq, dk, dv")
    if lse.shape != (B, Hq, L):
        raise ValueError(f"lse must be {(B, Hq, L)}")
    dt = _dtype_code(q)
    for t, name in ((k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} dtype {t.dtype} differs from q's {q.dtype}")
    if workspace is None:
        need = hd_sfa_bwd_final_workspace_bytes(B, L, n, Hq, Hkv, d, q.dtype)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    _check(load().hd_sfa_bwd_final(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), _dev(dout, "dout"),
                                   _dev(lse, "lse", torch.float32), _dev(dq, "dq"), _dev(dk, "dk"),
                                   _dev(dv, "dv"), B, L, n, Hq, Hkv, d, int(mode), int(window), float(scale), dt,
                                   _dev(workspace, "workspace"), wbytes, _stream(q)))
    return dq, dk, dv


# --------------------------------------------------------------------------
# Allocating conveniences.
# --------------------------------------------------------------------------

def expand_embed(ids, tables):
    B, L = ids.shape
    out = torch.empty((B, len(tables) * L, tables[0].shape[1]), dtype=tables[0].dtype, device=tables[0].device)
    return hd_expand_embed(ids, tables, out)


def sfa_fwd(q, k, v, n, mode, window=0, scale=0.0, return_lse=False):
    o = torch.empty_like(q)
    lse = None
    if return_lse:
        B, nL, Hq, _ = q.shape
        lse = torch.empty((B, Hq, nL), dtype=torch.float32, device=q.device)
    hd_sfa_fwd(q, k, v, o, n, mode, window, scale, lse)
    return (o, lse) if return_lse else o


def sfa_fwd_rope(q, k, v, n, mode, window=0, scale=0.0, theta=10000.0, return_lse=False):
    o, k_rot = torch.empty_like(q), torch.empty_like(k)
    lse = None
    if return_lse:
        B, nL, Hq, _ = q.shape
        lse = torch.empty((B, Hq, nL), dtype=torch.float32, device=q.device)
    hd_sfa_fwd_rope(q, k, v, o, k_rot, n, mode, window, scale, theta, lse)
    return (o, k_rot, lse) if return_lse else (o, k_rot)


def sfa_fwd_final(q, k, v, n, mode, window=0, scale=0.0, return_lse=False):
    o = torch.empty_like(q)
    lse = None
    if return_lse:
        B, L, Hq, _ = q.shape
        lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
    hd_sfa_fwd_final(q, k, v, o, n, mode, window, scale, lse)
    return (o, lse) if return_lse else o


def sfa_decode(q, k_new, v_new, k_cache, v_cache, cache_len, mode, window=0, scale=0.0, workspace=None):
    o = torch.empty_like(q)
    return hd_sfa_decode(q, k_new, v_new, k_cache, v_cache, cache_len, o, mode, window, scale, workspace)


def sfa_decode_final(q, k_new, v_new, k_cache, v_cache, cache_len, mode, window=0, scale=0.0, workspace=None):
    o = torch.empty_like(q)
    return hd_sfa_decode(q, k_new, v_new, k_cache, v_cache, cache_len, o, mode, window, scale, workspace,
                         final_only=True)


def sfa_bwd(q, k, v, o, dout, lse, n, mode, window=0, scale=0.0):
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    return hd_sfa_bwd(q, k, v, o, dout, lse, dq, dk, dv, n, mode, window, scale)


def sfa_bwd_final(q, k, v, o, dout, lse, n, mode, window=0, scale=0.0):
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    return hd_sfa_bwd_final(q, k, v, o, dout, lse, dq, dk, dv, n, mode, window, scale)


def rope(x, theta=10000.0, pos_base=None, pos_mul=0, t_mul=1, t_add=0):
    return hd_rope(x, torch.empty_like(x), theta, pos_base, pos_mul, t_mul, t_add)
