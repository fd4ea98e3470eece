"""CPU oracle for Stream-Factorized Attention (Hidden Decoding).

TEST INFRASTRUCTURE ONLY.  This package is the checker that the GPU library is
held against; it is not part of the product.  Only ``tests/``, the smoke check
in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` import it.  It
shares no code with ``latent_sequence_length_amd`` and never imports it.

Two independent implementations live here:

* ``hd_oracle.c`` (wrapped below through ctypes): the plain definition of every
  step, evaluated in double precision with keys visited in ascending order.
* ``brute.py``: a NumPy float64 brute force that materialises the nL x nL mask
  straight from the 1-based index maps of the pages, for tiny shapes.

Sources (WeLM blog "Hidden Decoding at Scale", section "Method Recap and New
Designs"): the expansion equation S_t = E_k(x_i) with t = (i-1)n + k; the index
maps i(t) = ceil(t/n), s(t) = (t-1) mod n + 1 and Figure 2's three masks; the
per-stream KV cache retained for decoding.

The backward (``sfa_bwd*``) is the chain-rule derivative of that forward.
``sfa_final*`` computes only the final stream's query rows (section
"Persistent KV and the KV-mirror Saving": mirrored layers run the last stream
alone over K/V of every stream).

Every function here is pinned by ``tests/test_oracle_*.py`` against library
routines, closed forms, invariants, finite differences and hand-worked golden
values.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhd_oracle.so")

INTRA, CROSS = 0, 1
_F32, _BF16 = 0, 1

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH) or (
        os.path.getmtime(LIB_PATH) < os.path.getmtime(os.path.join(HERE, "hd_oracle.c"))
    ):
        from . import build as _build  # compiling the checker is not using it

        _build.build()
    lib = _configure(ctypes.CDLL(LIB_PATH))
    _lib = lib
    return lib


def _configure(lib):
    """Declare the C signatures on a loaded oracle library."""
    P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_expand_embed.argtypes = [P, I, I, I, P, I64, I64, P]
    lib.oracle_visible.argtypes = [I64, I64, I, I, I64]
    lib.oracle_sfa_rows.argtypes = [P, P, P, I, I, I, I, I, I, I, I, I64, D, P, I64, P, P]
    lib.oracle_sfa_fwd.argtypes = [P, P, P, I, I, I, I, I, I, I, I, I64, D, P, P]
    lib.oracle_sfa_final_rows.argtypes = [P, P, P, I, I, I, I, I, I, I, I, I64, D, P, I64, P, P]
    lib.oracle_sfa_final.argtypes = [P, P, P, I, I, I, I, I, I, I, I, I64, D, P, P]
    lib.oracle_sfa_final_bwd_rows.argtypes = [P, P, P, P, I, I, I, I, I, I, I, I, I64, D, P, P, P, I64, P, P,
                                              I64, P, P]
    lib.oracle_sfa_decode.argtypes = [P, P, P, P, P, I, P, I, I, I, I, I, I, I, I64, D, P]
    lib.oracle_decode_append.argtypes = [P, P, P, I, I, I, I, I, I64]
    lib.oracle_sfa_bwd_rows.argtypes = [P, P, P, P, I, I, I, I, I, I, I, I, I64, D, P, P, P, I64, P, P, I64, P, P]
    lib.oracle_rope.argtypes = [P, I, I, I, I, I, P, I64, I64, I64, D, P]
    for f in (lib.oracle_expand_embed, lib.oracle_visible, lib.oracle_sfa_rows,
              lib.oracle_sfa_fwd, lib.oracle_sfa_decode, lib.oracle_decode_append, lib.oracle_sfa_bwd_rows,
              lib.oracle_rope):
        f.restype = ctypes.c_int
    return lib


def _buf(x):
    """Return (contiguous numpy array, dtype code) for float32 / bfloat16 data.

    Accepts numpy float32 arrays, numpy uint16 arrays holding raw bfloat16
    bits, or CPU torch tensors of dtype float32 / bfloat16."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return np.ascontiguousarray(x.view(torch.int16).numpy().view(np.uint16)), _BF16
            if x.dtype == torch.float32:
                return np.ascontiguousarray(x.numpy()), _F32
            raise TypeError(f"oracle input dtype {x.dtype} not float32/bfloat16")
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, _F32
    if x.dtype == np.uint16:
        return x, _BF16
    raise TypeError(f"oracle input dtype {x.dtype} not float32 / uint16(bf16 bits)")


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def visible(tq, tk, n, mode, window=0):
    """Figure 2 predicate on 0-based expanded positions (1 = visible)."""
    return _load().oracle_visible(int(tq), int(tk), int(n), int(mode), int(window))


def expand_embed(ids, tables):
    """out[b, i*n+s, :] = tables[s][ids[b,i], :] as a raw byte copy.

    ids: int32 [B, L]; tables: list of n arrays [V, D] of one dtype.
    Returns a numpy array [B, n*L, D] of the tables' dtype (bf16 as uint16 bits)."""
    ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
    bufs = [_buf(t)[0] for t in tables]
    B, L = ids.shape
    n = len(bufs)
    V, D = bufs[0].shape
    for t in bufs:
        if t.shape != (V, D) or t.dtype != bufs[0].dtype:
            raise ValueError("tables must share shape and dtype")
    out = np.empty((B, n * L, D), dtype=bufs[0].dtype)
    ptrs = (ctypes.c_void_p * n)(*[t.ctypes.data for t in bufs])
    rc = _load().oracle_expand_embed(_p(ids), B, L, n, ptrs, V, D * bufs[0].itemsize, _p(out))
    if rc:
        raise ValueError("id outside [0, V)")
    return out


def sfa_rows(q, k, v, n, mode, window=0, scale=0.0, rows=None):
    """Attention output (float64) for selected flat query rows r = (b*nL+t)*Hq+h.

    q [B, nL, Hq, d], k/v [B, nL, Hkv, d].  Returns (o [nrows, d], lse [nrows])."""
    qb, dt = _buf(q)
    kb, dt2 = _buf(k)
    vb, dt3 = _buf(v)
    if not (dt == dt2 == dt3):
        raise TypeError("q, k, v must share a dtype")
    B, nL, Hq, d = qb.shape
    Hkv = kb.shape[2]
    if nL % n:
        raise ValueError("sequence length not a multiple of n")
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    o = np.empty((rows.size, d), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    rc = _load().oracle_sfa_rows(_p(qb), _p(kb), _p(vb), dt, B, nL // n, n, Hq, Hkv, d,
                                 int(mode), int(window), float(scale), _p(rows), rows.size,
                                 _p(o), _p(lse))
    if rc:
        raise ValueError("oracle_sfa_rows rejected its arguments")
    return o, lse


def sfa_fwd(q, k, v, n, mode, window=0, scale=0.0):
    """Full prefill: returns (o [B, nL, Hq, d] float64, lse [B, Hq, nL] float64)."""
    qb, dt = _buf(q)
    kb, _ = _buf(k)
    vb, _ = _buf(v)
    B, nL, Hq, d = qb.shape
    Hkv = kb.shape[2]
    if nL % n:
        raise ValueError("sequence length not a multiple of n")
    o = np.empty((B, nL, Hq, d), dtype=np.float64)
    lse = np.empty((B, Hq, nL), dtype=np.float64)
    rc = _load().oracle_sfa_fwd(_p(qb), _p(kb), _p(vb), dt, B, nL // n, n, Hq, Hkv, d,
                                int(mode), int(window), float(scale), _p(o), _p(lse))
    if rc:
        raise ValueError("oracle_sfa_fwd rejected its arguments")
    return o, lse


def _final_shapes(qf, k, v, n):
    qb, dt = _buf(qf)
    kb, dt2 = _buf(k)
    vb, dt3 = _buf(v)
    if not (dt == dt2 == dt3):
        raise TypeError("qf, k, v must share a dtype")
    B, L, Hq, d = qb.shape
    if kb.shape[0] != B or kb.shape[1] != n * L or kb.shape[3] != d or vb.shape != kb.shape:
        raise ValueError("k/v must be [B, n*L, Hkv, d] for qf [B, L, Hq, d]")
    return qb, kb, vb, dt, B, L, Hq, kb.shape[2], d


def sfa_final_rows(qf, k, v, n, mode, window=0, scale=0.0, rows=None):
    """Final-stream queries of a KV-mirror layer, for selected flat rows
    r = (b*L + i)*Hq + h of qf [B, L, Hq, d] (query i at expanded position
    i*n + n-1); k/v [B, n*L, Hkv, d].  Returns (o [nrows, d], lse [nrows])."""
    qb, kb, vb, dt, B, L, Hq, Hkv, d = _final_shapes(qf, k, v, n)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    o = np.empty((rows.size, d), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    rc = _load().oracle_sfa_final_rows(_p(qb), _p(kb), _p(vb), dt, B, L, n, Hq, Hkv, d,
                                       int(mode), int(window), float(scale), _p(rows), rows.size,
                                       _p(o), _p(lse))
    if rc:
        raise ValueError("oracle_sfa_final_rows rejected its arguments")
    return o, lse


def sfa_final(qf, k, v, n, mode, window=0, scale=0.0):
    """All final-stream queries: (o [B, L, Hq, d], lse [B, Hq, L]), float64."""
    qb, kb, vb, dt, B, L, Hq, Hkv, d = _final_shapes(qf, k, v, n)
    o = np.empty((B, L, Hq, d), dtype=np.float64)
    lse = np.empty((B, Hq, L), dtype=np.float64)
    rc = _load().oracle_sfa_final(_p(qb), _p(kb), _p(vb), dt, B, L, n, Hq, Hkv, d,
                                  int(mode), int(window), float(scale), _p(o), _p(lse))
    if rc:
        raise ValueError("oracle_sfa_final rejected its arguments")
    return o, lse


def sfa_decode(q, k_new, v_new, k_cache, v_cache, cache_len, mode, window=0, scale=0.0):
    """One decode step; returns o [B, n, Hq, d] float64 (caches are not modified)."""
    qb, dt = _buf(q)
    knb, _ = _buf(k_new)
    vnb, _ = _buf(v_new)
    kcb, _ = _buf(k_cache)
    vcb, _ = _buf(v_cache)
    lens = np.ascontiguousarray(np.asarray(cache_len, dtype=np.int32))
    B, n, Hq, d = qb.shape
    T_cap, Hkv = kcb.shape[1], kcb.shape[3]
    o = np.empty((B, n, Hq, d), dtype=np.float64)
    rc = _load().oracle_sfa_decode(_p(qb), _p(knb), _p(vnb), _p(kcb), _p(vcb), dt, _p(lens),
                                   T_cap, B, n, Hq, Hkv, d, int(mode), int(window),
                                   float(scale), _p(o))
    if rc:
        raise ValueError("oracle_sfa_decode rejected its arguments")
    return o


def sfa_decode_final(q_final, k_new, v_new, k_cache, v_cache, cache_len, mode, window=0, scale=0.0):
    """Decode step of a KV-mirror layer: only the final stream's query
    q_final [B, 1, Hq, d] (at expanded position len*n + n-1) is run; the
    answer is that row of ``sfa_decode`` (a query row's attention does not
    depend on the other streams' queries).  Returns o [B, 1, Hq, d]."""
    qb, _ = _buf(q_final)
    n = tuple(k_new.shape)[1]
    q = np.zeros((qb.shape[0], n) + qb.shape[2:], dtype=qb.dtype)
    q[:, n - 1] = qb[:, 0]
    o = sfa_decode(q, k_new, v_new, k_cache, v_cache, cache_len, mode, window, scale)
    return np.ascontiguousarray(o[:, n - 1:n])


def decode_append(x_new, cache, cache_len):
    """Return a copy of cache with x_new written at token cache_len[b] (bytewise)."""
    xb, _ = _buf(x_new)
    cb, _ = _buf(cache)
    out = cb.copy()
    lens = np.ascontiguousarray(np.asarray(cache_len, dtype=np.int32))
    B, T_cap, n, Hkv, d = out.shape
    rc = _load().oracle_decode_append(_p(xb), _p(out), _p(lens), T_cap, B, n, Hkv, d, out.itemsize)
    if rc:
        raise ValueError("cache_len outside [0, T_cap)")
    return out


def row_stats(q, k, v, dout, n, mode, window=0, scale=0.0):
    """Per query row softmax normaliser lse and D = dO . O, both [B, Hq, nL]
    float64, from the forward definition (``sfa_fwd``)."""
    o, lse = sfa_fwd(q, k, v, n, mode, window, scale)
    db, _ = _buf(dout)
    dbl = db.astype(np.float64) if db.dtype == np.float32 else _bf16_to_f64(db)
    D = np.einsum("btHc,btHc->bHt", dbl, o)
    return np.ascontiguousarray(lse), np.ascontiguousarray(D)


def _bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def sfa_bwd_rows(q, k, v, dout, n, mode, window=0, scale=0.0, qrows=None, krows=None, stats=None):
    """Gradients of sum(dO * O): dq for flat query rows (b*nL+t)*Hq+h and dk, dv
    for flat key rows (b*nL+t)*Hkv+hk (float64 arrays [rows, d]).  stats =
    (lse, D) from ``row_stats`` (computed here when None)."""
    qb, dt = _buf(q)
    kb, _ = _buf(k)
    vb, _ = _buf(v)
    db, dt2 = _buf(dout)
    if dt != dt2:
        raise TypeError("dout must share q's dtype")
    B, nL, Hq, d = qb.shape
    Hkv = kb.shape[2]
    if stats is None:
        stats = row_stats(q, k, v, dout, n, mode, window, scale)
    lse, D = (np.ascontiguousarray(x, dtype=np.float64) for x in stats)
    qrows = np.ascontiguousarray(np.asarray([] if qrows is None else qrows, dtype=np.int64))
    krows = np.ascontiguousarray(np.asarray([] if krows is None else krows, dtype=np.int64))
    dq = np.empty((qrows.size, d))
    dk = np.empty((krows.size, d))
    dv = np.empty((krows.size, d))
    rc = _load().oracle_sfa_bwd_rows(_p(qb), _p(kb), _p(vb), _p(db), dt, B, nL // n, n, Hq, Hkv, d,
                                     int(mode), int(window), float(scale), _p(lse), _p(D),
                                     _p(qrows), qrows.size, _p(dq), _p(krows), krows.size, _p(dk), _p(dv))
    if rc:
        raise ValueError("oracle_sfa_bwd_rows rejected its arguments")
    return dq, dk, dv


def sfa_bwd(q, k, v, dout, n, mode, window=0, scale=0.0):
    """Full backward: dq [B, nL, Hq, d], dk / dv [B, nL, Hkv, d] (float64)."""
    B, nL, Hq, d = tuple(q.shape)
    Hkv = tuple(k.shape)[2]
    dq, dk, dv = sfa_bwd_rows(q, k, v, dout, n, mode, window, scale,
                              qrows=np.arange(B * nL * Hq), krows=np.arange(B * nL * Hkv))
    return dq.reshape(B, nL, Hq, d), dk.reshape(B, nL, Hkv, d), dv.reshape(B, nL, Hkv, d)


def final_row_stats(qf, k, v, doutf, n, mode, window=0, scale=0.0):
    """lse and D = dO . O of the final-stream rows, both [B, Hq, L] float64,
    from the forward definition (``sfa_final``)."""
    o, lse = sfa_final(qf, k, v, n, mode, window, scale)
    db, _ = _buf(doutf)
    dbl = db.astype(np.float64) if db.dtype == np.float32 else _bf16_to_f64(db)
    D = np.einsum("biHc,biHc->bHi", dbl, o)
    return np.ascontiguousarray(lse), np.ascontiguousarray(D)


def sfa_final_bwd_rows(qf, k, v, doutf, n, mode, window=0, scale=0.0, qrows=None, krows=None, stats=None):
    """Gradients of sum(dOf * Of) for the final-stream queries: dq for flat
    rows (b*L+i)*Hq+h of qf, dk / dv for flat key rows (b*nL+t)*Hkv+hk
    (float64 [rows, d]).  stats = (lse, D) from ``final_row_stats``."""
    qb, kb, vb, dt, B, L, Hq, Hkv, d = _final_shapes(qf, k, v, n)
    db, dt2 = _buf(doutf)
    if dt != dt2 or db.shape != qb.shape:
        raise TypeError("doutf must match qf in shape and dtype")
    if stats is None:
        stats = final_row_stats(qf, k, v, doutf, n, mode, window, scale)
    lse, D = (np.ascontiguousarray(x, dtype=np.float64) for x in stats)
    qrows = np.ascontiguousarray(np.asarray([] if qrows is None else qrows, dtype=np.int64))
    krows = np.ascontiguousarray(np.asarray([] if krows is None else krows, dtype=np.int64))
    dq = np.empty((qrows.size, d))
    dk = np.empty((krows.size, d))
    dv = np.empty((krows.size, d))
    rc = _load().oracle_sfa_final_bwd_rows(_p(qb), _p(kb), _p(vb), _p(db), dt, B, L, n, Hq, Hkv, d,
                                           int(mode), int(window), float(scale), _p(lse), _p(D),
                                           _p(qrows), qrows.size, _p(dq), _p(krows), krows.size,
                                           _p(dk), _p(dv))
    if rc:
        raise ValueError("oracle_sfa_final_bwd_rows rejected its arguments")
    return dq, dk, dv


def sfa_final_bwd(qf, k, v, doutf, n, mode, window=0, scale=0.0):
    """Full backward of the final-stream queries: dq [B, L, Hq, d], dk / dv
    [B, nL, Hkv, d] (float64)."""
    B, L, Hq, d = tuple(qf.shape)
    nL, Hkv = tuple(k.shape)[1], tuple(k.shape)[2]
    dq, dk, dv = sfa_final_bwd_rows(qf, k, v, doutf, n, mode, window, scale,
                                    qrows=np.arange(B * L * Hq), krows=np.arange(B * nL * Hkv))
    return dq.reshape(B, L, Hq, d), dk.reshape(B, nL, Hkv, d), dv.reshape(B, nL, Hkv, d)


def rope(x, theta=10000.0, pos_base=None, pos_mul=0, t_mul=1, t_add=0):
    """Rotary embedding of x [B, T, H, d] at positions
    t*t_mul + t_add + pos_mul*pos_base[b] ("rotate half" pairing c <-> c + d/2);
    returns float64 [B, T, H, d]."""
    xb, dt = _buf(x)
    B, T, H, d = xb.shape
    out = np.empty((B, T, H, d), dtype=np.float64)
    pb = None
    if pos_base is not None:
        pb = np.ascontiguousarray(np.asarray(pos_base, dtype=np.int32))
    rc = _load().oracle_rope(_p(xb), dt, B, T, H, d, _p(pb) if pb is not None else None, int(pos_mul),
                             int(t_mul), int(t_add), float(theta), _p(out))
    if rc:
        raise ValueError("oracle_rope rejected its arguments")
    return out
