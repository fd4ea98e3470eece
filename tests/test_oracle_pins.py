"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test ties the oracle to something independent: the hand-written Figure 2
masks, a library routine (torch's scaled_dot_product_attention and embedding,
NumPy fancy indexing), a closed form, or an invariant the definitions imply.
All run on the CPU.  Source of the definitions: WeLM blog "Hidden Decoding at
Scale", section "Method Recap and New Designs" (expansion equation, index maps,
Figure 2, per-stream KV retention).
"""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from latent_sequence_length_amd import synth
from oracle import brute
from tests.golden_io import mask_from_rows, read_blocks

INTRA, CROSS = 0, 1


def _rand(shape, seed, dtype=torch.float32):
    return synth.normal(shape, seed, dtype)


def sdpa64(q, k, v, attn_mask=None, causal=False, scale=None):
    """torch SDPA in float64 on [B, T, H, d] tensors with GQA by repetition."""
    q64, k64, v64 = (x.double().permute(0, 2, 1, 3) for x in (q, k, v))
    g = q64.shape[1] // k64.shape[1]
    k64 = k64.repeat_interleave(g, dim=1)
    v64 = v64.repeat_interleave(g, dim=1)
    out = F.scaled_dot_product_attention(q64, k64, v64, attn_mask=attn_mask, is_causal=causal, scale=scale)
    return out.permute(0, 2, 1, 3).contiguous()


# --------------------------------------------------------------------------
# Mask predicate and index maps
# --------------------------------------------------------------------------

def test_golden_masks_figure2(oracle):
    blocks = read_blocks("fig2_masks_n2_L3.txt")
    n, L = 2, 3
    for header, rows in blocks.items():
        if not header.startswith("mask"):
            continue
        _, mode_s, w_s = header.split()
        mode = INTRA if mode_s == "intra" else CROSS
        W = int(w_s.split("=")[1])
        want = mask_from_rows(rows)
        got_c = np.array([[oracle.visible(tq, tk, n, mode, W) for tk in range(n * L)]
                          for tq in range(n * L)], dtype=bool)
        np.testing.assert_array_equal(got_c, want, err_msg=header)
        np.testing.assert_array_equal(brute.mask(n, L, mode, W), want, err_msg=header)


def test_golden_index_maps():
    blocks = read_blocks("fig2_masks_n2_L3.txt")
    for line in blocks["index n=4"]:
        t, i, s = map(int, line.split())
        assert brute.token_index(t, 4) == i and brute.stream_index(t, 4) == s


def test_mask_exhaustive_c_vs_onebased(oracle):
    """0-based C predicate == explicit mask built from the 1-based index maps."""
    for n, L, W, mode in itertools.product(range(1, 5), range(1, 9), range(0, 4), (INTRA, CROSS)):
        want = brute.mask(n, L, mode, W)
        got = np.array([[oracle.visible(tq, tk, n, mode, W) for tk in range(n * L)]
                        for tq in range(n * L)], dtype=bool)
        assert np.array_equal(got, want), (n, L, W, mode)


def test_mask_structure_invariants():
    """intra = cross restricted to the same stream (any window); n=1: intra == cross."""
    for n, L, W in itertools.product(range(1, 5), range(1, 7), range(0, 4)):
        intra, cross = brute.mask(n, L, INTRA, W), brute.mask(n, L, CROSS, W)
        t = np.arange(n * L)
        same = (t[:, None] % n) == (t[None, :] % n)
        if W == 0:
            assert np.array_equal(intra, cross & same)
        assert not (intra & ~same).any()
        assert np.tril(np.ones_like(cross)).astype(bool)[cross].all()
        assert np.diag(intra).all() and np.diag(cross).all()
        if n == 1:
            assert np.array_equal(intra, cross)


# --------------------------------------------------------------------------
# Expansion
# --------------------------------------------------------------------------

def test_expand_golden_order(oracle):
    blocks = read_blocks("fig2_masks_n2_L3.txt")
    tabs = [np.arange(10 * 3, dtype=np.float32).reshape(10, 3) + 1000 * (s + 1) for s in range(2)]
    ids = np.array([[7, 2]], dtype=np.int32)
    out = oracle.expand_embed(ids, tabs)
    for line in blocks["expand n=2 L=2"]:
        t, table, token = map(int, line.split())
        np.testing.assert_array_equal(out[0, t - 1], tabs[table - 1][ids[0, token - 1]])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_expand_deinterleave_identity(oracle, dtype):
    n, V, D, B, L = 3, 50, 24, 2, 9
    tabs = synth.tables(n, V, D, dtype)
    ids = synth.token_ids(B, L, V, force_edges=True)
    out = oracle.expand_embed(ids.numpy(), tabs)
    for s in range(n):
        want = tabs[s][ids.long()]  # library gather
        want = want.view(torch.int16).numpy().view(np.uint16) if dtype == torch.bfloat16 else want.numpy()
        np.testing.assert_array_equal(out[:, s::n], want)


def test_expand_n1_is_embedding(oracle):
    V, D = 40, 16
    tab = synth.tables(1, V, D, torch.float32)
    ids = synth.token_ids(3, 11, V)
    out = oracle.expand_embed(ids.numpy(), tab)
    np.testing.assert_array_equal(out, F.embedding(ids.long(), tab[0]).numpy())


def test_expand_rejects_bad_ids(oracle):
    tab = synth.tables(2, 10, 4, torch.float32)
    with pytest.raises(ValueError):
        oracle.expand_embed(np.array([[0, 10]], dtype=np.int32), tab)
    with pytest.raises(ValueError):
        oracle.expand_embed(np.array([[-1]], dtype=np.int32), tab)


# --------------------------------------------------------------------------
# Attention: library special cases
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mode", [INTRA, CROSS])
def test_n1_is_textbook_causal(oracle, mode):
    B, L, Hq, Hkv, d = 2, 37, 4, 2, 16
    q, k, v = (_rand((B, L, h, d), s) for s, h in ((0, Hq), (1, Hkv), (2, Hkv)))
    o, _ = oracle.sfa_fwd(q, k, v, 1, mode)
    np.testing.assert_allclose(o, sdpa64(q, k, v, causal=True).numpy(), rtol=0, atol=1e-12)


def test_intra_is_n_independent_causal(oracle):
    B, L, n, Hq, Hkv, d = 1, 23, 4, 4, 2, 8
    q, k, v = synth.qkv(B, L, n, Hq, Hkv, d, torch.float32)
    o, _ = oracle.sfa_fwd(q, k, v, n, INTRA)
    for s in range(n):
        want = sdpa64(q[:, s::n], k[:, s::n], v[:, s::n], causal=True).numpy()
        np.testing.assert_allclose(o[:, s::n], want, rtol=0, atol=1e-12)


def test_cross_is_dense_causal(oracle):
    B, L, n, Hq, Hkv, d = 2, 13, 3, 2, 1, 8
    q, k, v = synth.qkv(B, L, n, Hq, Hkv, d, torch.float32)
    o, _ = oracle.sfa_fwd(q, k, v, n, CROSS)
    np.testing.assert_allclose(o, sdpa64(q, k, v, causal=True).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("W", [1, 2, 5])
def test_windows_are_banded_sdpa(oracle, W):
    B, L, n, Hq, Hkv, d = 1, 17, 3, 2, 2, 8
    q, k, v = synth.qkv(B, L, n, Hq, Hkv, d, torch.float32)
    # intra: per-stream band of W tokens
    o, _ = oracle.sfa_fwd(q, k, v, n, INTRA, W)
    i = torch.arange(L)
    band = (i[:, None] >= i[None, :]) & (i[:, None] - i[None, :] < W)
    for s in range(n):
        want = sdpa64(q[:, s::n], k[:, s::n], v[:, s::n], attn_mask=band).numpy()
        np.testing.assert_allclose(o[:, s::n], want, rtol=0, atol=1e-12)
    # cross: band of n*W expanded positions
    o, _ = oracle.sfa_fwd(q, k, v, n, CROSS, W)
    t = torch.arange(n * L)
    band = (t[:, None] >= t[None, :]) & (t[:, None] - t[None, :] < n * W)
    np.testing.assert_allclose(o, sdpa64(q, k, v, attn_mask=band).numpy(), rtol=0, atol=1e-12)


def test_gqa_equals_repeated_mha(oracle):
    B, L, n, Hq, Hkv, d = 1, 11, 2, 6, 2, 8
    q, k, v = synth.qkv(B, L, n, Hq, Hkv, d, torch.float32)
    g = Hq // Hkv
    for mode in (INTRA, CROSS):
        o, _ = oracle.sfa_fwd(q, k, v, n, mode)
        o2, _ = oracle.sfa_fwd(q, k.repeat_interleave(g, 2), v.repeat_interleave(g, 2), n, mode)
        np.testing.assert_array_equal(o, o2)


def test_lse_matches_logsumexp_and_scale(oracle):
    B, L, n, H, d = 1, 9, 2, 2, 8
    q, k, v = synth.qkv(B, L, n, H, H, d, torch.float32)
    for mode, W, scale in ((INTRA, 0, 0.0), (CROSS, 2, 0.3)):
        _, lse = oracle.sfa_fwd(q, k, v, n, mode, W, scale)
        m = torch.from_numpy(brute.mask(n, L, mode, W))
        sc = (scale if scale > 0 else 1 / math.sqrt(d))
        s = torch.einsum("bthd,bshd->bhts", q.double(), k.double()) * sc
        s = s.masked_fill(~m, float("-inf"))
        np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# Attention: closed forms and invariants
# --------------------------------------------------------------------------

def test_window1_intra_returns_v(oracle):
    q, k, v = synth.qkv(1, 10, 3, 4, 2, 8, torch.float32)
    o, _ = oracle.sfa_fwd(q, k, v, 3, INTRA, 1)
    np.testing.assert_array_equal(o, v.double().repeat_interleave(2, 2).numpy())


def test_zero_query_prefix_means(oracle):
    B, L, n, Hq, Hkv, d = 1, 12, 3, 2, 1, 4
    _, k, v = synth.qkv(B, L, n, Hq, Hkv, d, torch.float32)
    q = torch.zeros(B, n * L, Hq, d)
    v64 = v.double()
    # intra: mean of stream s's values over tokens 0..i
    o, lse = oracle.sfa_fwd(q, k, v, n, INTRA)
    for s in range(n):
        vs = v64[:, s::n, 0]
        mean = vs.cumsum(1) / torch.arange(1, L + 1, dtype=torch.float64)[None, :, None]
        for h in range(Hq):
            np.testing.assert_allclose(o[:, s::n, h], mean.numpy(), rtol=0, atol=1e-13)
    # lse with zero scores = log(number of visible keys)
    np.testing.assert_allclose(lse[0, 0, :], np.log(np.arange(n * L) // n + 1), atol=1e-13)
    # cross: positional prefix mean
    o, lse = oracle.sfa_fwd(q, k, v, n, CROSS)
    mean = v64[:, :, 0].cumsum(1) / torch.arange(1, n * L + 1, dtype=torch.float64)[None, :, None]
    np.testing.assert_allclose(o[:, :, 0], mean.numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0, :], np.log(np.arange(n * L) + 1), atol=1e-13)


def test_worked_example_closed_form(oracle):
    """n=2, L=2, d=1, scale 1: every output written out by hand as a softmax."""
    qv = [0.5, -1.0, 2.0, 0.25]
    kv = [1.0, 2.0, -0.5, 3.0]
    vv = [10.0, 20.0, 30.0, 40.0]
    q = torch.tensor(qv).view(1, 4, 1, 1)
    k = torch.tensor(kv).view(1, 4, 1, 1)
    v = torch.tensor(vv).view(1, 4, 1, 1)
    e = math.exp

    def sm(t, keys):
        w = [e(qv[t] * kv[j]) for j in keys]
        return sum(wi * vv[j] for wi, j in zip(w, keys)) / sum(w)

    o, _ = oracle.sfa_fwd(q, k, v, 2, INTRA, 0, 1.0)
    want = [sm(0, [0]), sm(1, [1]), sm(2, [0, 2]), sm(3, [1, 3])]
    np.testing.assert_allclose(o[0, :, 0, 0], want, rtol=1e-15)
    o, _ = oracle.sfa_fwd(q, k, v, 2, CROSS, 0, 1.0)
    want = [sm(0, [0]), sm(1, [0, 1]), sm(2, [0, 1, 2]), sm(3, [0, 1, 2, 3])]
    np.testing.assert_allclose(o[0, :, 0, 0], want, rtol=1e-15)
    o, _ = oracle.sfa_fwd(q, k, v, 2, CROSS, 1, 1.0)
    want = [sm(0, [0]), sm(1, [0, 1]), sm(2, [1, 2]), sm(3, [2, 3])]
    np.testing.assert_allclose(o[0, :, 0, 0], want, rtol=1e-15)


@pytest.mark.parametrize("mode,W", [(INTRA, 0), (CROSS, 0), (INTRA, 3), (CROSS, 2)])
def test_constant_v_and_convex_hull(oracle, mode, W):
    B, L, n, Hq, Hkv, d = 1, 15, 3, 4, 2, 8
    q, k, v = synth.qkv(B, L, n, Hq, Hkv, d, torch.float32)
    c = torch.full_like(v, 0.375)
    o, _ = oracle.sfa_fwd(q, k, c, n, mode, W)
    np.testing.assert_allclose(o, 0.375, rtol=0, atol=1e-15)
    o, _ = oracle.sfa_fwd(q, k, v, n, mode, W)
    m = brute.mask(n, L, mode, W)
    vv = v.double().numpy()
    for t in range(n * L):
        vis = vv[0, m[t]]  # [nvis, Hkv, d]
        for h in range(Hq):
            lo, hi = vis[:, h // 2].min(0), vis[:, h // 2].max(0)
            assert (o[0, t, h] >= lo - 1e-12).all() and (o[0, t, h] <= hi + 1e-12).all()


def test_stream_permutation_equivariance(oracle):
    B, L, n, Hq, Hkv, d = 1, 9, 4, 2, 2, 8
    q, k, v = synth.qkv(B, L, n, Hq, Hkv, d, torch.float32)
    perm = [2, 0, 3, 1]
    idx = torch.tensor([i * n + perm[s] for i in range(L) for s in range(n)])
    o, _ = oracle.sfa_fwd(q, k, v, n, INTRA)
    op, _ = oracle.sfa_fwd(q[:, idx], k[:, idx], v[:, idx], n, INTRA)
    np.testing.assert_array_equal(op, o[:, idx.numpy()])


def test_c_oracle_matches_brute_force(oracle):
    for (B, L, n, Hq, Hkv, d), mode, W in itertools.product(
            [(1, 64, 2, 4, 4, 32), (2, 7, 3, 4, 2, 8), (1, 5, 1, 2, 1, 16)],
            (INTRA, CROSS), (0, 1, 3)):
        q, k, v = synth.qkv(B, L, n, Hq, Hkv, d, torch.float32)
        o, lse = oracle.sfa_fwd(q, k, v, n, mode, W)
        ob, lseb = brute.attention(q.numpy(), k.numpy(), v.numpy(), n, mode, W)
        np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lseb, rtol=0, atol=1e-12)


def test_bf16_inputs_widen_exactly(oracle):
    q, k, v = synth.qkv(1, 8, 2, 2, 1, 16, torch.bfloat16)
    o16, _ = oracle.sfa_fwd(q, k, v, 2, CROSS)
    o32, _ = oracle.sfa_fwd(q.float(), k.float(), v.float(), 2, CROSS)
    np.testing.assert_array_equal(o16, o32)


def test_rows_subset_matches_full(oracle):
    q, k, v = synth.qkv(2, 10, 2, 4, 2, 8, torch.float32)
    o, lse = oracle.sfa_fwd(q, k, v, 2, INTRA, 3)
    rows = np.array([0, 5, 17, 79, 80, 159], dtype=np.int64)
    orow, lrow = oracle.sfa_rows(q, k, v, 2, INTRA, 3, rows=rows)
    np.testing.assert_array_equal(orow, o.reshape(-1, 8)[rows])
    b, t, h = rows // (20 * 4), (rows // 4) % 20, rows % 4
    np.testing.assert_array_equal(lrow, lse[b, h, t])


# --------------------------------------------------------------------------
# Decode over the retained per-stream cache
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mode,W", [(INTRA, 0), (CROSS, 0), (INTRA, 2), (CROSS, 1)])
def test_decode_equals_prefill_rows(oracle, mode, W):
    B, n, Hq, Hkv, d, T_cap = 3, 3, 4, 2, 8, 9
    q, kn, vn, kc, vc = synth.decode_inputs(B, n, Hq, Hkv, d, T_cap, torch.float32)
    lens = [0, 4, 8]
    o = oracle.sfa_decode(q, kn, vn, kc, vc, lens, mode, W)
    for b, ln in enumerate(lens):
        L = ln + 1
        kseq = torch.cat([kc[b, :ln], kn[b:b + 1]], 0).reshape(1, L * n, Hkv, d)
        vseq = torch.cat([vc[b, :ln], vn[b:b + 1]], 0).reshape(1, L * n, Hkv, d)
        qseq = torch.zeros(1, L * n, Hq, d)
        qseq[0, ln * n:] = q[b]
        of, _ = oracle.sfa_fwd(qseq, kseq, vseq, n, mode, W)
        np.testing.assert_allclose(o[b], of[0, ln * n:], rtol=0, atol=1e-14)


def test_decode_ignores_cache_rows_beyond_len(oracle):
    B, n, Hq, Hkv, d, T_cap = 2, 2, 2, 1, 8, 6
    q, kn, vn, kc, vc = synth.decode_inputs(B, n, Hq, Hkv, d, T_cap, torch.float32)
    lens = [2, 3]
    o1 = oracle.sfa_decode(q, kn, vn, kc, vc, lens, CROSS)
    kc2, vc2 = kc.clone(), vc.clone()
    kc2[0, 2:] = 1e30
    vc2[1, 3:] = float("nan")
    o2 = oracle.sfa_decode(q, kn, vn, kc2, vc2, lens, CROSS)
    np.testing.assert_array_equal(o1, o2)


def test_decode_append_bytes(oracle):
    B, n, Hkv, d, T_cap = 3, 2, 2, 4, 5
    _, kn, _, kc, _ = synth.decode_inputs(B, n, 2, Hkv, d, T_cap, torch.bfloat16)
    lens = [0, 2, 4]
    out = oracle.decode_append(kn, kc, lens)
    want = kc.clone()
    for b, ln in enumerate(lens):
        want[b, ln] = kn[b]
    np.testing.assert_array_equal(out, want.view(torch.int16).numpy().view(np.uint16))
    with pytest.raises(ValueError):
        oracle.decode_append(kn, kc, [0, 5, 1])


# --------------------------------------------------------------------------
# Backward (gradient of sum(dO * O)); the forward's chain-rule derivative
# --------------------------------------------------------------------------

def _bwd_inputs(B, L, n, Hq, Hkv, d, seed=0):
    q = _rand((B, n * L, Hq, d), 10 + seed)
    k = _rand((B, n * L, Hkv, d), 20 + seed)
    v = _rand((B, n * L, Hkv, d), 30 + seed)
    do = _rand((B, n * L, Hq, d), 40 + seed)
    return q, k, v, do


def autograd_bwd(q, k, v, do, n, mode, W, scale=None):
    """torch float64 autograd of masked softmax attention (explicit Figure 2
    mask from the 1-based index maps, GQA by repeating K/V)."""
    L = q.shape[1] // n
    m = torch.from_numpy(brute.mask(n, L, mode, W))
    q64, k64, v64 = (x.double().requires_grad_(True) for x in (q, k, v))
    out = sdpa64(q64, k64, v64, attn_mask=m, scale=scale)
    (out * do.double()).sum().backward()
    return q64.grad.numpy(), k64.grad.numpy(), v64.grad.numpy()


@pytest.mark.parametrize("mode,W,g", [(INTRA, 0, 1), (CROSS, 0, 1), (INTRA, 2, 2), (CROSS, 3, 2),
                                      (INTRA, 0, 4), (CROSS, 0, 3)])
def test_bwd_matches_autograd(oracle, mode, W, g):
    B, L, n, Hkv, d = 2, 7, 3, 2, 16
    q, k, v, do = _bwd_inputs(B, L, n, g * Hkv, Hkv, d, seed=mode + W + g)
    dq, dk, dv = oracle.sfa_bwd(q, k, v, do, n, mode, W)
    wq, wk, wv = autograd_bwd(q, k, v, do, n, mode, W)
    np.testing.assert_allclose(dq, wq, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dk, wk, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv, wv, rtol=1e-9, atol=1e-11)


def test_bwd_custom_scale_matches_autograd(oracle):
    q, k, v, do = _bwd_inputs(1, 6, 2, 2, 1, 8, seed=5)
    dq, dk, dv = oracle.sfa_bwd(q, k, v, do, 2, CROSS, 0, scale=0.3)
    wq, wk, wv = autograd_bwd(q, k, v, do, 2, CROSS, 0, scale=0.3)
    for got, want in ((dq, wq), (dk, wk), (dv, wv)):
        np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-11)


@pytest.mark.parametrize("mode,W", [(INTRA, 0), (CROSS, 2)])
def test_bwd_finite_differences(oracle, mode, W):
    """Central differences of sum(dO * O) through the forward oracle only."""
    B, L, n, Hq, Hkv, d = 1, 3, 2, 2, 1, 4
    q, k, v, do = _bwd_inputs(B, L, n, Hq, Hkv, d, seed=7)
    dq, dk, dv = oracle.sfa_bwd(q, k, v, do, n, mode, W)
    h = 2.0 ** -12   # exactly representable; inputs stay float32

    def loss(qq, kk, vv):
        o, _ = oracle.sfa_fwd(qq, kk, vv, n, mode, W)
        return float((o * do.double().numpy()).sum())

    rng = np.random.default_rng(3)
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        base = [q, k, v]
        for _ in range(6):
            idx = tuple(int(rng.integers(s)) for s in base[which].shape)
            plus = [x.clone() for x in base]
            minus = [x.clone() for x in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd = (loss(*plus) - loss(*minus)) / (2 * h)
            assert abs(fd - grad[idx]) <= 2e-5 * max(1.0, abs(grad[idx])), (which, idx, fd, grad[idx])


def test_bwd_window1_closed_form(oracle):
    """Intra, W=1: each query sees only itself, so O = V, dQ = dK = 0 and
    dV[t, hk] = sum of dO[t, h] over the heads of the group."""
    B, L, n, Hq, Hkv, d = 1, 5, 3, 4, 2, 8
    q, k, v, do = _bwd_inputs(B, L, n, Hq, Hkv, d, seed=11)
    dq, dk, dv = oracle.sfa_bwd(q, k, v, do, n, INTRA, 1)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    want = do.double().numpy().reshape(B, n * L, Hkv, Hq // Hkv, d).sum(axis=3)
    np.testing.assert_allclose(dv, want, rtol=1e-12, atol=1e-13)


def test_bwd_zero_query_closed_form(oracle):
    """Q = 0: uniform weights over the visible keys, so dV_j = sum over the
    queries i that see j of dO_i / (number of keys i sees)."""
    B, L, n, Hq, Hkv, d = 1, 6, 2, 2, 1, 4
    _, k, v, do = _bwd_inputs(B, L, n, Hq, Hkv, d, seed=13)
    q = torch.zeros(B, n * L, Hq, d)
    for mode in (INTRA, CROSS):
        m = brute.mask(n, L, mode, 0)
        _, _, dv = oracle.sfa_bwd(q, k, v, do, n, mode, 0)
        w = m / m.sum(axis=1, keepdims=True)          # [tq, tk]
        dosum = do.double().numpy()[0].sum(axis=1)      # heads of the single group
        want = w.T @ dosum
        np.testing.assert_allclose(dv[0, :, 0], want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("mode,W", [(INTRA, 0), (CROSS, 0), (CROSS, 4), (INTRA, 3)])
def test_bwd_invariants(oracle, mode, W):
    """Softmax rows sum to one: summed over all keys, dK vanishes and dV
    equals the sum of dO over the group's heads and all positions."""
    B, L, n, Hq, Hkv, d = 2, 9, 4, 4, 2, 8
    q, k, v, do = _bwd_inputs(B, L, n, Hq, Hkv, d, seed=17)
    _, dk, dv = oracle.sfa_bwd(q, k, v, do, n, mode, W)
    assert np.abs(dk.sum(axis=1)).max() < 1e-10
    want = do.double().numpy().reshape(B, n * L, Hkv, Hq // Hkv, d).sum(axis=(1, 3))
    np.testing.assert_allclose(dv.sum(axis=1), want, rtol=1e-10, atol=1e-10)


def test_bwd_rows_subset_matches_full(oracle):
    B, L, n, Hq, Hkv, d = 1, 8, 2, 4, 2, 16
    q, k, v, do = _bwd_inputs(B, L, n, Hq, Hkv, d, seed=19)
    dq, dk, dv = oracle.sfa_bwd(q, k, v, do, n, CROSS, 3)
    qrows = np.array([0, 5, 17, 40, B * n * L * Hq - 1])
    krows = np.array([0, 3, 11, B * n * L * Hkv - 1])
    sq, sk, sv = oracle.sfa_bwd_rows(q, k, v, do, n, CROSS, 3, qrows=qrows, krows=krows)
    np.testing.assert_array_equal(sq, dq.reshape(-1, d)[qrows])
    np.testing.assert_array_equal(sk, dk.reshape(-1, d)[krows])
    np.testing.assert_array_equal(sv, dv.reshape(-1, d)[krows])


# --------------------------------------------------------------------------
# Rotary embedding at the expanded (contiguous) positions
# --------------------------------------------------------------------------

def test_rope_matches_transformers_rotate_half(oracle):
    """Library pin: transformers' Llama apply_rotary_pos_emb / rotate_half with
    inv_freq = theta^(-2c/d) and positions 0..T-1, in float64."""
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb
    B, T, H, d, theta = 2, 11, 3, 16, 500.0
    x = _rand((B, T, H, d), 51)
    got = oracle.rope(x, theta)
    inv = 1.0 / (theta ** (torch.arange(0, d, 2, dtype=torch.float64) / d))
    ang = torch.arange(T, dtype=torch.float64)[:, None] * inv[None, :]
    emb = torch.cat([ang, ang], dim=-1)
    cos, sin = emb.cos()[None], emb.sin()[None]                    # [1, T, d]
    xt = x.double().permute(0, 2, 1, 3)                            # [B, H, T, d]
    want, _ = apply_rotary_pos_emb(xt, xt, cos, sin, unsqueeze_dim=1)
    np.testing.assert_allclose(got, want.permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-12)


def test_rope_golden_d4(oracle):
    """Hand-worked: d=4, theta=100 -> frequencies 1 and 0.1; position 1."""
    x = torch.tensor([[[[0.0, 0.0, 0.0, 0.0]], [[1.0, 2.0, 3.0, 4.0]]]])   # T=2, position 1 is row 1
    got = oracle.rope(x, 100.0)[0, 1, 0]
    c1, s1, c2, s2 = math.cos(1.0), math.sin(1.0), math.cos(0.1), math.sin(0.1)
    want = [1 * c1 - 3 * s1, 2 * c2 - 4 * s2, 3 * c1 + 1 * s1, 4 * c2 + 2 * s2]
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-14)


def test_rope_relative_position_and_norm(oracle):
    """q(t1).k(t2) depends only on t1 - t2; position 0 is the identity;
    each (c, c + d/2) pair keeps its norm."""
    d, theta = 32, 10000.0
    q = _rand((1, 1, 1, d), 52)
    k = _rand((1, 1, 1, d), 53)
    T = 40
    qs = oracle.rope(q.expand(1, T, 1, d).contiguous(), theta)[0, :, 0]
    ks = oracle.rope(k.expand(1, T, 1, d).contiguous(), theta)[0, :, 0]
    for t1, t2, s in ((7, 3, 20), (30, 30, 5), (2, 9, 17)):
        if t1 + s < T and t2 + s < T:
            assert abs(qs[t1] @ ks[t2] - qs[t1 + s] @ ks[t2 + s]) < 1e-12
    np.testing.assert_allclose(qs[0], q[0, 0, 0].double().numpy(), rtol=0, atol=0)
    h = d // 2
    qn = q[0, 0, 0].double().numpy()
    for t in (1, 13, 39):
        np.testing.assert_allclose(qs[t][:h] ** 2 + qs[t][h:] ** 2, qn[:h] ** 2 + qn[h:] ** 2, rtol=1e-12)


def test_rope_decode_positions(oracle):
    """pos_base/pos_mul place stream s of the new token at len*n + s: equal to
    the rows len*n + s of a prefill rotation."""
    n, H, d = 4, 2, 16
    lens = [5, 0, 12]
    x = _rand((3, n, H, d), 54)
    got = oracle.rope(x, 10000.0, pos_base=lens, pos_mul=n)
    for b, ln in enumerate(lens):
        full = torch.zeros(1, (ln + 1) * n, H, d)
        full[0, ln * n:] = x[b]
        want = oracle.rope(full, 10000.0)[0, ln * n:]
        np.testing.assert_allclose(got[b], want, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# Final-stream queries of a KV-mirror layer
# --------------------------------------------------------------------------

def _final_inputs(B, L, n, Hq, Hkv, d, seed=60):
    qf = _rand((B, L, Hq, d), seed)
    k = _rand((B, n * L, Hkv, d), seed + 1)
    v = _rand((B, n * L, Hkv, d), seed + 2)
    return qf, k, v


@pytest.mark.parametrize("mode,W", [(INTRA, 0), (CROSS, 0), (INTRA, 2), (CROSS, 3), (CROSS, 1)])
def test_final_matches_sdpa_with_onebased_rows(oracle, mode, W):
    """Library pin: torch SDPA (float64) with the rectangular mask made of the
    rows of the 1-based Figure 2 mask at t = i*n (the last stream of token i);
    lse against torch.logsumexp of the same masked scores."""
    B, L, n, Hq, Hkv, d = 2, 7, 3, 4, 2, 16
    qf, k, v = _final_inputs(B, L, n, Hq, Hkv, d)
    full = brute.mask(n, L, mode, W)
    rows = np.array([i * n - 1 for i in range(1, L + 1)])     # 1-based t = i*n  ->  0-based row i*n - 1
    m = torch.from_numpy(full[rows])                           # [L, nL]
    want = sdpa64(qf, k, v, attn_mask=m)
    got, lse = oracle.sfa_final(qf, k, v, n, mode, W)
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-12)
    s = torch.einsum("bihc,bjhc->bhij", qf.double(), k.double().repeat_interleave(Hq // Hkv, dim=2)) / math.sqrt(d)
    want_lse = torch.logsumexp(s.masked_fill(~m, -math.inf), dim=-1)
    np.testing.assert_allclose(lse, want_lse.numpy(), rtol=1e-12, atol=1e-12)


def test_final_intra_is_causal_on_last_stream(oracle):
    """Intra mirrored layer: causal attention of the final-stream queries over
    the final stream's keys alone (rows n-1, 2n-1, ... of K/V)."""
    B, L, n, Hq, Hkv, d = 1, 9, 4, 2, 1, 8
    qf, k, v = _final_inputs(B, L, n, Hq, Hkv, d, seed=63)
    got, _ = oracle.sfa_final(qf, k, v, n, INTRA)
    want = sdpa64(qf, k[:, n - 1::n], v[:, n - 1::n], causal=True)
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mode", [INTRA, CROSS])
def test_final_n1_is_textbook_causal(oracle, mode):
    qf, k, v = _final_inputs(2, 11, 1, 2, 2, 8, seed=66)
    got, _ = oracle.sfa_final(qf, k, v, 1, mode)
    np.testing.assert_allclose(got, sdpa64(qf, k, v, causal=True).numpy(), rtol=1e-12, atol=1e-12)


def test_final_closed_forms(oracle):
    """Zero queries give uniform weights: cross sees the (i+1)*n positions of
    tokens 0..i (lse = log((i+1)n)); cross with W=1 sees the n streams of token
    i only; intra with W=1 returns the final-stream value row itself."""
    B, L, n, Hq, Hkv, d = 1, 6, 3, 2, 1, 4
    qf, k, v = _final_inputs(B, L, n, Hq, Hkv, d, seed=69)
    zero = torch.zeros_like(qf)
    v64 = v.double().numpy()[0, :, 0]
    o, lse = oracle.sfa_final(zero, k, v, n, CROSS)
    for i in range(L):
        np.testing.assert_allclose(o[0, i, 0], v64[:(i + 1) * n].mean(axis=0), rtol=1e-13, atol=1e-14)
        assert abs(lse[0, 1, i] - math.log((i + 1) * n)) < 1e-13
    o, lse = oracle.sfa_final(zero, k, v, n, CROSS, 1)
    for i in range(L):
        np.testing.assert_allclose(o[0, i, 1], v64[i * n:(i + 1) * n].mean(axis=0), rtol=1e-13, atol=1e-14)
        assert abs(lse[0, 0, i] - math.log(n)) < 1e-13
    o, _ = oracle.sfa_final(qf, k, v, n, INTRA, 1)
    for i in range(L):
        np.testing.assert_array_equal(o[0, i, 0], v64[i * n + n - 1])


@pytest.mark.parametrize("mode,W", [(INTRA, 0), (CROSS, 0), (CROSS, 2), (INTRA, 3)])
def test_final_equals_full_layer_last_stream_rows(oracle, mode, W):
    """Running the final stream alone changes nothing for it: its rows equal
    rows n-1, 2n-1, ... of the full layer whatever the other streams' queries."""
    B, L, n, Hq, Hkv, d = 2, 5, 3, 4, 2, 8
    qf, k, v = _final_inputs(B, L, n, Hq, Hkv, d, seed=72)
    q = _rand((B, n * L, Hq, d), 75)
    q[:, n - 1::n] = qf
    o_full, lse_full = oracle.sfa_fwd(q, k, v, n, mode, W)
    o, lse = oracle.sfa_final(qf, k, v, n, mode, W)
    np.testing.assert_allclose(o, o_full[:, n - 1::n], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lse_full[:, :, n - 1::n], rtol=1e-13, atol=1e-13)


def test_final_rows_subset_matches_full(oracle):
    B, L, n, Hq, Hkv, d = 2, 6, 2, 4, 2, 8
    qf, k, v = _final_inputs(B, L, n, Hq, Hkv, d, seed=78)
    o, lse = oracle.sfa_final(qf, k, v, n, CROSS, 2)
    rows = np.array([0, 5, 17, B * L * Hq - 1])
    so, sl = oracle.sfa_final_rows(qf, k, v, n, CROSS, 2, rows=rows)
    np.testing.assert_array_equal(so, o.reshape(-1, d)[rows])
    np.testing.assert_array_equal(sl, lse.transpose(0, 2, 1).reshape(-1)[rows])


def _final_bwd_inputs(B, L, n, Hq, Hkv, d, seed=80):
    qf, k, v = _final_inputs(B, L, n, Hq, Hkv, d, seed)
    dof = _rand((B, L, Hq, d), seed + 3)
    return qf, k, v, dof


def autograd_final_bwd(qf, k, v, dof, n, mode, W, scale=None):
    """torch float64 autograd of SDPA with the rectangular mask made of the
    1-based Figure 2 mask's rows t = i*n (GQA by repeating K/V)."""
    L = qf.shape[1]
    m = torch.from_numpy(brute.mask(n, L, mode, W)[np.arange(1, L + 1) * n - 1])
    q64, k64, v64 = (x.double().requires_grad_(True) for x in (qf, k, v))
    out = sdpa64(q64, k64, v64, attn_mask=m, scale=scale)
    (out * dof.double()).sum().backward()
    return q64.grad.numpy(), k64.grad.numpy(), v64.grad.numpy()


@pytest.mark.parametrize("mode,W,g", [(INTRA, 0, 1), (CROSS, 0, 2), (INTRA, 3, 2), (CROSS, 2, 3), (CROSS, 1, 1)])
def test_final_bwd_matches_autograd(oracle, mode, W, g):
    B, L, n, Hkv, d = 2, 6, 3, 2, 8
    qf, k, v, dof = _final_bwd_inputs(B, L, n, g * Hkv, Hkv, d, seed=81 + W + g)
    dq, dk, dv = oracle.sfa_final_bwd(qf, k, v, dof, n, mode, W)
    wq, wk, wv = autograd_final_bwd(qf, k, v, dof, n, mode, W)
    for got, want in ((dq, wq), (dk, wk), (dv, wv)):
        np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-11)


@pytest.mark.parametrize("mode,W", [(INTRA, 0), (CROSS, 0), (CROSS, 2)])
def test_final_bwd_equals_full_bwd_with_other_streams_silent(oracle, mode, W):
    """The full layer's backward with dO = 0 on every non-final row gives the
    same dK, dV, the final rows' dQ, and dQ = 0 elsewhere."""
    B, L, n, Hq, Hkv, d = 1, 5, 3, 4, 2, 8
    qf, k, v, dof = _final_bwd_inputs(B, L, n, Hq, Hkv, d, seed=90)
    q = _rand((B, n * L, Hq, d), 93)
    q[:, n - 1::n] = qf
    do = torch.zeros((B, n * L, Hq, d))
    do[:, n - 1::n] = dof
    fq, fk, fv = oracle.sfa_bwd(q, k, v, do, n, mode, W)
    dq, dk, dv = oracle.sfa_final_bwd(qf, k, v, dof, n, mode, W)
    np.testing.assert_allclose(dk, fk, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv, fv, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dq, fq[:, n - 1::n], rtol=1e-12, atol=1e-13)
    mask = np.ones(n * L, dtype=bool)
    mask[n - 1::n] = False
    assert np.abs(fq[:, mask]).max() == 0.0


def test_final_bwd_finite_differences(oracle):
    """Central differences of sum(dOf * Of) through the final-stream forward."""
    B, L, n, Hq, Hkv, d = 1, 3, 2, 2, 1, 4
    qf, k, v, dof = _final_bwd_inputs(B, L, n, Hq, Hkv, d, seed=95)
    dq, dk, dv = oracle.sfa_final_bwd(qf, k, v, dof, n, CROSS, 0)
    h = 2.0 ** -12

    def loss(qq, kk, vv):
        o, _ = oracle.sfa_final(qq, kk, vv, n, CROSS)
        return float((o * dof.double().numpy()).sum())

    rng = np.random.default_rng(4)
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        base = [qf, k, v]
        for _ in range(6):
            idx = tuple(int(rng.integers(s)) for s in base[which].shape)
            plus = [x.clone() for x in base]
            minus = [x.clone() for x in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd = (loss(*plus) - loss(*minus)) / (2 * h)
            assert abs(fd - grad[idx]) <= 2e-5 * max(1.0, abs(grad[idx])), (which, idx, fd, grad[idx])


@pytest.mark.parametrize("mode,W", [(INTRA, 0), (CROSS, 0), (CROSS, 3)])
def test_final_bwd_invariants(oracle, mode, W):
    """Per (b, kv head): sum over all key rows of dK is 0 (each query's dS
    sums to 0) and of dV is the sum of dOf over the group's heads and rows."""
    B, L, n, Hq, Hkv, d = 2, 7, 4, 4, 2, 8
    qf, k, v, dof = _final_bwd_inputs(B, L, n, Hq, Hkv, d, seed=97)
    _, dk, dv = oracle.sfa_final_bwd(qf, k, v, dof, n, mode, W)
    assert np.abs(dk.sum(axis=1)).max() < 1e-12
    want = dof.double().numpy().reshape(B, L, Hkv, Hq // Hkv, d).sum(axis=(1, 3))
    np.testing.assert_allclose(dv.sum(axis=1), want, rtol=1e-12, atol=1e-12)
    if mode == INTRA:   # keys of streams 0..n-2 get nothing in an intra layer
        keep = np.zeros(n * L, dtype=bool)
        keep[n - 1::n] = True
        assert np.abs(dk[:, ~keep]).max() == 0.0 and np.abs(dv[:, ~keep]).max() == 0.0


@pytest.mark.parametrize("mode,W", [(INTRA, 0), (CROSS, 0), (INTRA, 2), (CROSS, 1)])
def test_decode_final_equals_final_prefill_rows(oracle, mode, W):
    """A KV-mirror layer's decode step (final-stream query only) equals the
    final-stream prefill's last row on the appended sequence."""
    B, n, Hq, Hkv, d, T_cap = 3, 3, 4, 2, 8, 9
    q, kn, vn, kc, vc = synth.decode_inputs(B, n, Hq, Hkv, d, T_cap, torch.float32)
    qf = q[:, n - 1:n].contiguous()
    lens = [0, 4, 8]
    o = oracle.sfa_decode_final(qf, kn, vn, kc, vc, lens, mode, W)
    assert o.shape == (B, 1, Hq, d)
    for b, ln in enumerate(lens):
        L = ln + 1
        kseq = torch.cat([kc[b, :ln], kn[b:b + 1]], 0).reshape(1, L * n, Hkv, d)
        vseq = torch.cat([vc[b, :ln], vn[b:b + 1]], 0).reshape(1, L * n, Hkv, d)
        qseq = torch.zeros(1, L, Hq, d)
        qseq[0, ln] = qf[b, 0]
        of, _ = oracle.sfa_final(qseq, kseq, vseq, n, mode, W)
        np.testing.assert_allclose(o[b, 0], of[0, ln], rtol=0, atol=1e-14)


def test_rope_final_stream_and_final_decode_positions(oracle):
    """t_mul / t_add place compact final-stream rows (row i at i*n + n-1) and
    the final stream's decode row (len*n + n-1): equal to those rows of the
    plain prefill rotation."""
    n, H, d, L = 3, 2, 16, 6
    x = _rand((2, n * L, H, d), 56)
    full = oracle.rope(x, 10000.0)
    xf = x[:, n - 1::n].contiguous()
    got = oracle.rope(xf, 10000.0, t_mul=n, t_add=n - 1)
    np.testing.assert_allclose(got, full[:, n - 1::n], rtol=0, atol=1e-13)
    lens = [4, 0]
    q1 = _rand((2, 1, H, d), 57)
    dec = oracle.rope(q1, 10000.0, pos_base=lens, pos_mul=n, t_add=n - 1)
    for b, ln in enumerate(lens):
        seq = torch.zeros(1, (ln + 1) * n, H, d)
        seq[0, ln * n + n - 1] = q1[b, 0]
        np.testing.assert_allclose(dec[b, 0], oracle.rope(seq, 10000.0)[0, ln * n + n - 1], rtol=0, atol=1e-13)
