"""GPU parity of the final-stream queries of a KV-mirror layer
(hd_sfa_fwd_final through the C ABI) against the CPU oracle.

q holds the rows of stream n-1 only ([B, L, Hq, d], query i at expanded
position i*n + n-1); k and v cover all n*L positions.  Bars are the prefill's:
  - bf16: max |gpu - oracle| <= 2e-2, mean <= 2e-3; lse max abs <= 4e-3;
  - float32: max abs <= 1e-4 (output and lse).
The kernels visit, for every query, the same key tiles in the same order as
the full layer's kernel does for that row, and a key tile wholly outside a
query's band adds exact zeros.  Without a window every row's band starts at
key 0, so its running max is raised on the same tiles in both layouts and the
final-stream rows must be bit-identical to rows n-1, 2n-1, ... of hd_sfa_fwd;
with a window the max of a whole wave is raised together (when one of its
rows first sees a key), so those rows agree to rounding.
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
# The bf16 kernels sum the fp32 probabilities for l (lse = m + ln l): the
# bar is the worst case of sequential fp32 summation over up to 4096
# 32-key sub-tile sums (131072-key rows: 4096 * 2^-24 = 2.5e-4 relative in
# l, the same absolute in lse), plus fp32 accumulation of the 128-term
# scores (<= 128 * 2^-24 * sum|q_i k_i| * scale, ~6e-5 for unit-variance
# inputs) and the exp2 / log / scale roundings (~1e-6).
LSE_TOL_BF16 = 5e-4


@pytest.fixture(autouse=True)
def announce(request):
    sys.__stdout__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stdout__.flush()
    yield
    torch.cuda.synchronize()


def to_np(t):
    return t.detach().to(torch.float64).cpu().numpy()


def final_inputs(B, L, n, Hq, Hkv, d, dtype):
    q, k, v = synth.qkv(B, L, n, Hq, Hkv, d, dtype, DEV)
    return q, q[:, n - 1::n].contiguous(), k, v


def check(got, want, what, max_abs, mean_abs=None):
    diff = np.abs(to_np(got).reshape(want.shape) - want)
    assert np.isfinite(diff).all(), f"{what}: non-finite output"
    sys.__stdout__.write(f"  {what}: max {diff.max():.3e} mean {diff.mean():.3e}\n")
    assert diff.max() <= max_abs, f"{what}: max abs {diff.max():.3e} > {max_abs}"
    if mean_abs is not None:
        assert diff.mean() <= mean_abs, f"{what}: mean abs {diff.mean():.3e} > {mean_abs}"


FINAL_SHAPES = [
    # (B, L, n, Hq, Hkv, d), mode, window
    ((1, 64, 2, 4, 4, 32), INTRA, 0),
    ((1, 64, 2, 4, 4, 32), CROSS, 0),
    ((2, 150, 3, 8, 2, 128), CROSS, 0),     # g=4, ragged tails, several tiles
    ((2, 150, 3, 8, 2, 128), INTRA, 0),
    ((1, 257, 4, 8, 8, 64), CROSS, 0),      # MHA, d=64
    ((1, 130, 4, 16, 2, 128), CROSS, 10),   # g=8, local cross-stream window
    ((1, 300, 4, 8, 2, 128), INTRA, 70),    # window edges inside tiles
    ((1, 97, 1, 6, 3, 64), CROSS, 0),       # n=1: plain causal
    ((1, 200, 8, 4, 1, 128), CROSS, 3),     # n=8, window of 24 positions
    ((1, 50, 4, 4, 2, 128), CROSS, 60),     # window wider than the sequence
    ((3, 1, 4, 4, 1, 128), CROSS, 0),       # one token
    ((1, 1, 1, 2, 1, 64), INTRA, 0),        # one position
    ((1, 100, 16, 4, 2, 32), CROSS, 1),     # HD_MAX_STREAMS streams, window of one token
]


@pytest.mark.parametrize("shape,mode,window", FINAL_SHAPES)
def test_final_bf16_vs_oracle(shape, mode, window):
    B, L, n, Hq, Hkv, d = shape
    _, qf, k, v = final_inputs(B, L, n, Hq, Hkv, d, torch.bfloat16)
    o, lse = hd.sfa_fwd_final(qf, k, v, n, mode, window, return_lse=True)
    want, want_lse = oracle.sfa_final(qf.cpu(), k.cpu(), v.cpu(), n, mode, window)
    check(o, want, f"o {shape} mode={mode} W={window}", 2e-2, 2e-3)
    check(lse, want_lse, "lse", LSE_TOL_BF16)


@pytest.mark.parametrize("shape,mode,window", [
    ((1, 40, 2, 4, 4, 32), INTRA, 0),
    ((1, 40, 2, 4, 4, 32), CROSS, 0),
    ((2, 23, 3, 4, 2, 64), CROSS, 5),
    ((1, 30, 4, 2, 1, 128), INTRA, 7),
])
def test_final_f32_vs_oracle(shape, mode, window):
    B, L, n, Hq, Hkv, d = shape
    _, qf, k, v = final_inputs(B, L, n, Hq, Hkv, d, torch.float32)
    o, lse = hd.sfa_fwd_final(qf, k, v, n, mode, window, return_lse=True)
    want, want_lse = oracle.sfa_final(qf.cpu(), k.cpu(), v.cpu(), n, mode, window)
    check(o, want, "o", 1e-4)
    check(lse, want_lse, "lse", 1e-4)


def test_final_custom_scale():
    B, L, n, Hq, Hkv, d = 1, 90, 4, 8, 2, 128
    _, qf, k, v = final_inputs(B, L, n, Hq, Hkv, d, torch.bfloat16)
    o = hd.sfa_fwd_final(qf, k, v, n, CROSS, 0, 0.05)
    want, _ = oracle.sfa_final(qf.cpu(), k.cpu(), v.cpu(), n, CROSS, 0, 0.05)
    check(o, want, "o", 2e-2, 2e-3)


@pytest.mark.parametrize("shape,mode,window,dtype", [
    ((2, 150, 3, 8, 2, 128), CROSS, 0, torch.bfloat16),
    ((2, 150, 3, 8, 2, 128), INTRA, 0, torch.bfloat16),
    ((1, 300, 4, 8, 2, 128), CROSS, 9, torch.bfloat16),
    ((1, 300, 4, 8, 2, 128), INTRA, 70, torch.bfloat16),
    ((1, 257, 4, 8, 8, 64), CROSS, 0, torch.bfloat16),
    ((1, 60, 3, 4, 2, 32), CROSS, 4, torch.float32),
])
def test_final_equals_full_layer_rows(shape, mode, window, dtype):
    B, L, n, Hq, Hkv, d = shape
    q, qf, k, v = final_inputs(B, L, n, Hq, Hkv, d, dtype)
    o_full, lse_full = hd.sfa_fwd(q, k, v, n, mode, window, return_lse=True)
    o, lse = hd.sfa_fwd_final(qf, k, v, n, mode, window, return_lse=True)
    if window == 0:
        assert torch.equal(o, o_full[:, n - 1::n])
        assert torch.equal(lse, lse_full[:, :, n - 1::n])
    else:
        check(o, to_np(o_full[:, n - 1::n]), "o vs full layer", 2e-2, 2e-3)
        check(lse, to_np(lse_full[:, :, n - 1::n]), "lse vs full layer", LSE_TOL_BF16)


def test_final_full_size_sampled():
    """Final-stream queries of the 4096-token cross layer (n=4, 32 q / 8 kv
    heads, d=128) and its intra counterpart: sampled rows against the oracle
    (first and last tokens, tile edges of the 64-query blocks, random rows)."""
    c = synth.CROSS_4K
    q, qf, k, v = final_inputs(c.B, c.L, c.n, c.Hq, c.Hkv, c.d, c.dtype)
    del q
    rng = np.random.default_rng(11)
    edge_i = [0, 1, 2, 31, 32, 63, 64, 65, 127, 128, 2047, 2048, c.L - 2, c.L - 1]
    rows = np.unique(np.concatenate([
        np.array([i * c.Hq + h for i in edge_i for h in (0, 1, c.Hq - 1)]),
        rng.integers(0, c.L * c.Hq, 1536)]))
    qc, kc, vc = qf.cpu(), k.cpu(), v.cpu()
    for mode in (CROSS, INTRA):
        o, lse = hd.sfa_fwd_final(qf, k, v, c.n, mode, return_lse=True)
        want, want_lse = oracle.sfa_final_rows(qc, kc, vc, c.n, mode, rows=rows)
        check(o.reshape(-1, c.d)[torch.from_numpy(rows).to(DEV)], want, f"o rows mode={mode}", 2e-2, 2e-3)
        lse_rows = lse.permute(0, 2, 1).reshape(-1)[torch.from_numpy(rows).to(DEV)]
        check(lse_rows, want_lse, "lse rows", LSE_TOL_BF16)
        assert torch.isfinite(o).all()


def test_final_deterministic_and_guarded():
    B, L, n, Hq, Hkv, d = 1, 150, 4, 8, 2, 128
    _, qf, k, v = final_inputs(B, L, n, Hq, Hkv, d, torch.bfloat16)
    guard = 4096
    for mode, window in ((INTRA, 0), (CROSS, 0), (CROSS, 9)):
        ob = torch.full((qf.numel() + 2 * guard,), -7.0, dtype=torch.bfloat16, device=DEV)
        lb = torch.full((B * Hq * L + 2 * guard,), -7.0, dtype=torch.float32, device=DEV)
        o = ob[guard:guard + qf.numel()].view(qf.shape)
        lse = lb[guard:guard + B * Hq * L].view(B, Hq, L)
        hd.hd_sfa_fwd_final(qf, k, v, o, n, mode, window, lse=lse)
        o2, lse2 = hd.sfa_fwd_final(qf, k, v, n, mode, window, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(lse, lse2)
        assert (ob[:guard] == -7.0).all() and (ob[guard + qf.numel():] == -7.0).all()
        assert (lb[:guard] == -7.0).all() and (lb[guard + B * Hq * L:] == -7.0).all()
