"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Every input comes from the seeded generators in ``latent_sequence_length_amd.synth``;
the oracle receives a host copy of the very same tensors.  Bars:
  - expansion gather and decode cache append: bit-exact;
  - bf16 attention: max |gpu - oracle| <= 2e-2 and mean <= 2e-3;
  - float32 attention: max |gpu - oracle| <= 1e-4;
  - lse: max abs <= 4e-3 for bf16 (the softmax denominator is summed from
    the bf16-rounded probabilities that enter the PV product; bf16 carries 8
    significant bits, so each has a relative rounding error <= 2^-8 and ln of
    their sum is within ln(1 + 2^-8) = 3.9e-3 of ln of the exact sum, plus
    ~1e-4 for fp32 scores and exp2), 1e-4 for float32.
Small shapes are compared on every output; the full workload sizes are
compared on sampled rows (stream boundaries, window edges, first/last tokens,
tile edges, random interior rows).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from latent_sequence_length_amd import hd, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
INTRA, CROSS = 0, 1


@pytest.fixture(autouse=True)
def announce(request):
    sys.__stdout__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stdout__.flush()
    yield
    torch.cuda.synchronize()


def to_np(t):
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to(torch.float64).cpu().numpy()


def check_bf16(got, want, what, max_abs=2e-2, mean_abs=2e-3):
    diff = np.abs(to_np(got).reshape(want.shape) - want)
    assert np.isfinite(diff).all(), f"{what}: non-finite output"
    assert diff.max() <= max_abs, f"{what}: max abs {diff.max():.3e} > {max_abs}"
    assert diff.mean() <= mean_abs, f"{what}: mean abs {diff.mean():.3e} > {mean_abs}"


# The bf16 kernels sum the fp32 probabilities for l (lse = m + ln l): the
# bar is the worst case of sequential fp32 summation over up to 4096
# 32-key sub-tile sums (131072-key rows: 4096 * 2^-24 = 2.5e-4 relative in
# l, the same absolute in lse), plus fp32 accumulation of the 128-term
# scores (<= 128 * 2^-24 * sum|q_i k_i| * scale, ~6e-5 for unit-variance
# inputs) and the exp2 / log / scale roundings (~1e-6).
LSE_TOL_BF16 = 5e-4


def check_f32(got, want, what, tol=1e-4):
    diff = np.abs(to_np(got).reshape(want.shape) - want)
    assert np.isfinite(diff).all(), f"{what}: non-finite output"
    assert diff.max() <= tol, f"{what}: max abs {diff.max():.3e} > {tol}"


def bits(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy()


# ---------------------------------------------------------------------------
# Expansion
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B,L,n,V,D,dtype", [
    (1, 64, 2, 512, 64, torch.float32),     # tiny oracle case
    (1, 64, 1, 512, 64, torch.float32),     # n = 1 control
    (3, 5, 16, 37, 7, torch.bfloat16),      # 14-byte rows (2-byte path), HD_MAX_STREAMS tables
    (2, 9, 3, 11, 3, torch.float32),        # 12-byte rows
    (2, 33, 4, 1000, 520, torch.bfloat16),  # 1040-byte rows: vector path + tail
])
def test_expand_embed_small(B, L, n, V, D, dtype):
    tabs = synth.tables(n, V, D, dtype, DEV)
    ids = synth.token_ids(B, L, V, device=DEV, force_edges=True)
    out = hd.expand_embed(ids, tabs)
    want = oracle.expand_embed(ids.cpu().numpy(), [t.cpu() for t in tabs])
    np.testing.assert_array_equal(bits(out), want.view(np.uint16 if dtype == torch.bfloat16 else np.int32))


def test_expand_embed_full_tables():
    """64 sequences x 1 new token x 4 streams, then 4096 tokens x 4 streams,
    from four 160000 x 7168 bf16 tables: bit-exact against the oracle."""
    c = synth.EMBED_DECODE
    tabs = synth.tables(c["n"], c["V"], c["D"], c["dtype"], DEV)
    host = [t.cpu() for t in tabs]
    for B, L in ((c["B"], c["L"]), (synth.EMBED_PREFILL["B"], synth.EMBED_PREFILL["L"])):
        ids = synth.token_ids(B, L, c["V"], device=DEV, force_edges=True)
        out = hd.expand_embed(ids, tabs)
        want = oracle.expand_embed(ids.cpu().numpy(), host)
        np.testing.assert_array_equal(bits(out), want)


# ---------------------------------------------------------------------------
# Prefill
# ---------------------------------------------------------------------------

def run_fwd(shape_args, mode, window, dtype, scale=0.0):
    B, L, n, Hq, Hkv, d = shape_args
    q, k, v = synth.qkv(B, L, n, Hq, Hkv, d, dtype, DEV)
    o, lse = hd.sfa_fwd(q, k, v, n, mode, window, scale, return_lse=True)
    torch.cuda.synchronize()
    return q, k, v, o, lse


@pytest.mark.parametrize("n", [1, 2])
@pytest.mark.parametrize("mode", [INTRA, CROSS])
def test_fwd_f32_tiny(n, mode):
    shape = (1, 64, n, 4, 4, 32)
    q, k, v, o, lse = run_fwd(shape, mode, 0, torch.float32)
    want, wlse = oracle.sfa_fwd(q.cpu(), k.cpu(), v.cpu(), n, mode)
    check_f32(o, want, "o")
    check_f32(lse, wlse, "lse")


@pytest.mark.parametrize("shape,mode,window", [
    ((2, 37, 3, 4, 2, 64), INTRA, 5),
    ((1, 50, 2, 2, 1, 128), CROSS, 7),
    ((1, 19, 4, 8, 1, 32), INTRA, 0),
])
def test_fwd_f32_shapes(shape, mode, window):
    q, k, v, o, lse = run_fwd(shape, mode, window, torch.float32)
    want, wlse = oracle.sfa_fwd(q.cpu(), k.cpu(), v.cpu(), shape[2], mode, window)
    check_f32(o, want, "o")
    check_f32(lse, wlse, "lse")


BF16_SHAPES = [
    # (B, L, n, Hq, Hkv, d), mode, window
    ((1, 64, 2, 4, 4, 32), INTRA, 0),
    ((1, 64, 2, 4, 4, 32), CROSS, 0),
    ((2, 200, 3, 8, 2, 128), INTRA, 0),     # g=4, ragged tail
    ((2, 200, 3, 8, 2, 128), CROSS, 0),
    ((1, 257, 4, 8, 8, 64), INTRA, 0),      # MHA: 4 token blocks per workgroup
    ((1, 130, 4, 16, 2, 128), CROSS, 0),    # g=8: two head groups
    ((1, 97, 2, 6, 3, 64), INTRA, 0),       # g=2
    ((1, 300, 1, 8, 2, 128), INTRA, 0),     # n=1
    ((1, 300, 4, 8, 2, 128), INTRA, 1),     # window of one token: o = v
    ((1, 300, 4, 8, 2, 128), INTRA, 70),    # window edge inside tiles
    ((1, 160, 4, 8, 2, 128), CROSS, 10),    # local cross-stream (mask b)
    ((1, 160, 4, 8, 2, 32), CROSS, 33),
    ((3, 1, 4, 4, 1, 128), INTRA, 0),       # one token
    ((1, 1, 1, 2, 1, 64), CROSS, 0),        # one position
    ((1, 129, 3, 4, 2, 128), CROSS, 1000),  # window wider than the sequence
    ((2, 40, 4, 8, 2, 128), INTRA, 0),      # 64-query waves whose second half is partly past the end
    ((1, 97, 2, 4, 1, 128), CROSS, 45),     # window edges in different sub-tiles for the two halves
]


@pytest.mark.parametrize("shape,mode,window", BF16_SHAPES)
def test_fwd_bf16_vs_oracle(shape, mode, window):
    q, k, v, o, lse = run_fwd(shape, mode, window, torch.bfloat16)
    want, wlse = oracle.sfa_fwd(q.cpu(), k.cpu(), v.cpu(), shape[2], mode, window)
    check_bf16(o, want, f"o {shape} mode={mode} W={window}")
    check_f32(lse, wlse, "lse", tol=LSE_TOL_BF16)


# Layers with more d=128 workgroups than the chip has compute units, each
# workgroup-to-XCD map branch, compared on every output (the full workloads
# are only compared on sampled rows).
MANY_WG_SHAPES = [
    ((4, 700, 4, 8, 2, 128), INTRA, 0),     # 352 workgroups: whole groups per XCD, ragged tail
    ((4, 700, 4, 8, 2, 128), INTRA, 100),   # the same with a window
    ((3, 1984, 1, 12, 3, 128), INTRA, 0),   # 279 workgroups: count not a multiple of 8
    ((4, 600, 4, 8, 8, 128), CROSS, 0),     # 320 workgroups, MHA (g = 1)
    ((1, 1024, 4, 16, 4, 128), CROSS, 0),   # 4 groups: each spread over two XCDs
    # persistent launch with several items per CU: 768 items (3 rounds of
    # 256, 24 groups: three per XCD), ragged last block, windowed
    ((3, 2000, 4, 8, 2, 128), INTRA, 200),
    ((2, 1500, 4, 8, 2, 128), CROSS, 100),  # 376 items, 4 groups, window edges inside tiles
]


@pytest.mark.parametrize("shape,mode,window", MANY_WG_SHAPES)
def test_fwd_bf16_many_workgroups(shape, mode, window):
    q, k, v, o, lse = run_fwd(shape, mode, window, torch.bfloat16)
    want, wlse = oracle.sfa_fwd(q.cpu(), k.cpu(), v.cpu(), shape[2], mode, window)
    check_bf16(o, want, f"o {shape} mode={mode} W={window}")
    check_f32(lse, wlse, "lse", tol=LSE_TOL_BF16)


def test_fwd_bf16_custom_scale():
    shape = (1, 70, 2, 4, 2, 64)
    q, k, v, o, lse = run_fwd(shape, CROSS, 0, torch.bfloat16, scale=0.05)
    want, wlse = oracle.sfa_fwd(q.cpu(), k.cpu(), v.cpu(), 2, CROSS, 0, 0.05)
    check_bf16(o, want, "o scale=0.05")
    check_f32(lse, wlse, "lse", tol=LSE_TOL_BF16)


def sample_rows(B, L, n, Hq, window, count, seed):
    """Flat query rows (b*nL + t)*Hq + h covering edges and random interior."""
    rng = np.random.default_rng(seed)
    toks = {0, 1, L - 1, L - 2, L // 2}
    for e in (31, 32, 63, 64, 127, 128):
        toks.update({e, L - 1 - e})
    if window:
        toks.update({window - 1, window, window + 1, L - window})
    toks = [i for i in toks if 0 <= i < L]
    rows = []
    for i in toks:
        for s in range(n):
            for h in (0, Hq - 1, int(rng.integers(Hq))):
                b = int(rng.integers(B))
                rows.append((b * n * L + i * n + s) * Hq + h)
    while len(rows) < count:
        b, t, h = rng.integers(B), rng.integers(n * L), rng.integers(Hq)
        rows.append(int((b * n * L + t) * Hq + h))
    return np.unique(np.array(rows, dtype=np.int64))


FULL = [synth.INTRA_4K, synth.INTRA_4K_N1, synth.CROSS_4K, synth.LONG_INTRA_W, synth.LONG_CROSS_W, synth.LONG_CROSS]


@pytest.mark.parametrize("cfg", FULL, ids=[c.name for c in FULL])
def test_fwd_full_size_sampled(cfg):
    count = 4096
    q, k, v, o, lse = run_fwd((cfg.B, cfg.L, cfg.n, cfg.Hq, cfg.Hkv, cfg.d), cfg.mode, cfg.window, cfg.dtype)
    rows = sample_rows(cfg.B, cfg.L, cfg.n, cfg.Hq, cfg.window, count, seed=11)
    want, wlse = oracle.sfa_rows(q.cpu(), k.cpu(), v.cpu(), cfg.n, cfg.mode, cfg.window, rows=rows)
    got = o.reshape(-1, cfg.d)[torch.from_numpy(rows).to(DEV)]
    check_bf16(got, want, cfg.name)
    nL = cfg.n * cfg.L
    b, t, h = rows // (nL * cfg.Hq), (rows // cfg.Hq) % nL, rows % cfg.Hq
    check_f32(lse.cpu().numpy()[b, h, t], wlse, "lse", tol=LSE_TOL_BF16)
    assert torch.isfinite(o).all()


def test_fwd_deterministic_and_guarded():
    shape = (1, 300, 4, 8, 2, 128)
    B, L, n, Hq, Hkv, d = shape
    q, k, v = synth.qkv(B, L, n, Hq, Hkv, d, torch.bfloat16, DEV)
    for mode, window in ((INTRA, 0), (CROSS, 0), (INTRA, 50)):
        guard = 4096
        buf = torch.full((q.numel() + 2 * guard,), -7.0, dtype=torch.bfloat16, device=DEV)
        o1 = buf[guard:guard + q.numel()].view(q.shape)
        hd.hd_sfa_fwd(q, k, v, o1, n, mode, window)
        o2 = hd.sfa_fwd(q, k, v, n, mode, window)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
        assert (buf[:guard] == -7.0).all() and (buf[guard + q.numel():] == -7.0).all()


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------

def run_decode(B, n, Hq, Hkv, d, T_cap, lens, mode, window, dtype):
    q, kn, vn, kc, vc = synth.decode_inputs(B, n, Hq, Hkv, d, T_cap, dtype, DEV)
    kc0, vc0 = kc.cpu(), vc.cpu()
    cl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o = hd.sfa_decode(q, kn, vn, kc, vc, cl, mode, window)
    torch.cuda.synchronize()
    return q, kn, vn, kc0, vc0, kc, vc, o


DEC_SHAPES = [
    # B, n, Hq, Hkv, d, T_cap, lens
    (3, 4, 8, 2, 128, 40, [0, 5, 37]),      # 16 query rows per kv head
    (2, 2, 4, 4, 32, 70, [69, 1]),          # g=1
    (2, 4, 16, 2, 64, 33, [32, 7]),         # 32 rows: two query blocks
    (1, 8, 32, 4, 128, 20, [19]),           # 64 rows: four query blocks
    (2, 3, 10, 2, 128, 50, [11, 48]),       # 15 rows: padded block
    (2, 1, 8, 1, 128, 300, [299, 150]),     # n=1
]


@pytest.mark.parametrize("shape", DEC_SHAPES)
@pytest.mark.parametrize("mode,window", [(INTRA, 0), (CROSS, 0), (INTRA, 3), (CROSS, 2)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_vs_oracle(shape, mode, window, dtype):
    B, n, Hq, Hkv, d, T_cap, lens = shape
    q, kn, vn, kc0, vc0, kc, vc, o = run_decode(B, n, Hq, Hkv, d, T_cap, lens, mode, window, dtype)
    want = oracle.sfa_decode(q.cpu(), kn.cpu(), vn.cpu(), kc0, vc0, lens, mode, window)
    if dtype == torch.bfloat16:
        check_bf16(o, want, f"decode {shape} mode={mode} W={window}")
    else:
        check_f32(o, want, f"decode {shape} mode={mode} W={window}")
    np.testing.assert_array_equal(bits(kc), oracle.decode_append(kn.cpu(), kc0, lens).view(bits(kc).dtype))
    np.testing.assert_array_equal(bits(vc), oracle.decode_append(vn.cpu(), vc0, lens).view(bits(vc).dtype))


@pytest.mark.parametrize("mode,window,ragged,nseq", [
    # the decode workload (64 sequences, 8192 cached tokens): 32 whole
    # sequences = 4096 query rows against the oracle
    (INTRA, 0, False, 32), (CROSS, 0, False, 32),
    # ragged lengths (0 and T_cap-1 included)
    (INTRA, 0, True, 6), (CROSS, 0, True, 6),
    # 4096-token sliding window at full size (the window starts mid-split)
    (INTRA, 4096, False, 8), (CROSS, 4096, False, 8),
])
def test_decode_full_size_sampled(mode, window, ragged, nseq):
    cfg = synth.DECODE_8K
    T_cap = cfg.ctx + 8
    if ragged:
        lens = [int(x) for x in np.random.default_rng(5).integers(0, T_cap, cfg.B)]
        lens[0], lens[-1] = 0, T_cap - 1
    else:
        lens = [cfg.ctx] * cfg.B
    q, kn, vn, kc, vc = synth.decode_inputs(cfg.B, cfg.n, cfg.Hq, cfg.Hkv, cfg.d, T_cap, cfg.dtype, DEV)
    picks = sorted(set([0, cfg.B - 1] + [int(x) for x in np.linspace(0, cfg.B - 1, nseq)]))[:max(nseq, 2)]
    if ragged:
        picks = sorted(set(picks[:nseq - 2] + [0, cfg.B - 1]))
    idx = torch.tensor(picks, device=DEV)
    # cache rows [0, len) are all the oracle reads; the step writes row len
    kc0, vc0 = kc[idx].cpu(), vc[idx].cpu()
    cl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o = hd.sfa_decode(q, kn, vn, kc, vc, cl, mode, window)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    lp = [lens[b] for b in picks]
    want = oracle.sfa_decode(q[idx].cpu(), kn[idx].cpu(), vn[idx].cpu(), kc0, vc0, lp, mode, window)
    check_bf16(o[idx], want, f"decode {len(picks)} sequences mode={mode} W={window} ragged={ragged}")
    for b in picks:
        np.testing.assert_array_equal(bits(kc[b, lens[b]]), bits(kn[b]))
        np.testing.assert_array_equal(bits(vc[b, lens[b]]), bits(vn[b]))


def test_decode_deterministic_and_guarded():
    B, n, Hq, Hkv, d, T_cap = 4, 4, 32, 8, 128, 600
    q, kn, vn, kc, vc = synth.decode_inputs(B, n, Hq, Hkv, d, T_cap, torch.bfloat16, DEV)
    cl = torch.tensor([599, 0, 300, 64], dtype=torch.int32, device=DEV)
    for mode in (INTRA, CROSS):
        guard = 2048
        buf = torch.full((q.numel() + 2 * guard,), 3.0, dtype=torch.bfloat16, device=DEV)
        o1 = buf[guard:guard + q.numel()].view(q.shape)
        ws = torch.full((hd.hd_sfa_decode_workspace_bytes(B, n, Hq, Hkv, d, T_cap) + 4096,), 255,
                        dtype=torch.uint8, device=DEV)
        hd.hd_sfa_decode(q, kn, vn, kc, vc, cl, o1, mode, 0, 0.0, ws)
        o2 = hd.sfa_decode(q, kn, vn, kc, vc, cl, mode)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
        assert (buf[:guard] == 3.0).all() and (buf[guard + q.numel():] == 3.0).all()


@pytest.mark.parametrize("mode", [INTRA, CROSS])
def test_fwd_bf16_extreme_score_growth(mode):
    """Scores spanning hundreds of log2 units (scale 1, |q| ~ 8): the running
    max must be raised mid-row (probabilities against a stale max overflow
    fp32), exercising the rescale path of every kernel."""
    B, L, n, Hq, Hkv, d = 1, 300, 2, 4, 2, 128
    q, k, v = synth.qkv(B, L, n, Hq, Hkv, d, torch.bfloat16, DEV)
    q = (q.float() * 8.0).to(torch.bfloat16)
    o, lse = hd.sfa_fwd(q, k, v, n, mode, 0, 1.0, return_lse=True)
    want, wlse = oracle.sfa_fwd(q.cpu(), k.cpu(), v.cpu(), n, mode, 0, 1.0)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    check_bf16(o, want, f"extreme mode={mode}")
    # lse is ~1e3 here: its bar is relative to fp32 score rounding
    check_f32(lse, wlse, "lse", tol=LSE_TOL_BF16 + 1e-6 * float(np.abs(wlse).max()))
