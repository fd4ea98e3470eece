"""GPU parity of the attention backward (hd_sfa_bwd through the C ABI) against
the CPU oracle's chain-rule gradients.

The GPU path is run as a trainer would run it: hd_sfa_fwd produces o and lse,
then hd_sfa_bwd consumes them; the oracle computes its own forward and
gradients in double from the same seeded q, k, v, dO.  Bars:
  - float32: max |gpu - oracle| <= 1e-4 * max(1, max |oracle|);
  - bf16: max |gpu - oracle| <= 2e-2 * max(1, max |oracle|) and
          mean |gpu - oracle| <= 4e-3 * max(1, mean |oracle|).
    Every gradient term carries at most two bf16 roundings (P or dS as an
    MFMA operand, each <= 2^-8 relative: bf16 carries 8 significant bits) on top of fp32 accumulation, and the
    output is rounded once more; D = dO . o uses the bf16 forward output.
    The max bar is the forward's (2e-2) scaled by the size of the gradient,
    since dK and dV sum over many queries and heads.
    Mean bar: the arithmetic a bf16 backward must do rounds each P or dS
    operand and each output to bf16 (unit roundoff u = 2^-8); averaged over
    the elements the output rounding is about u/4 of the gradient's size and
    the operand rounding, random in sign over the summed terms, about
    u/(2 sqrt 3); their sum stays below u, so mean <= 4e-3 * max(1, mean |oracle|).
    An exact emulation of just these two roundings gives 2.1e-3 on a
    17-token, 3-stream, 8-head layer (few terms per sum).
Small shapes are compared on every element; the full 4096-token workload on
sampled rows plus the row-sum invariants over all keys.
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
SEED_DOUT = 9


@pytest.fixture(autouse=True)
def announce(request):
    sys.__stdout__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stdout__.flush()
    yield
    torch.cuda.synchronize()


BWD_MEAN_BF16 = 4e-3  # mean bar for bf16 gradients (see the module docstring)


def to_np(t):
    return t.detach().to(torch.float64).cpu().numpy()


def check_grad(got, want, what, rel_max, rel_mean=None):
    g = to_np(got).reshape(want.shape)
    diff = np.abs(g - want)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    ref_max, ref_mean = np.abs(want).max(), np.abs(want).mean()
    sys.__stdout__.write(f"  {what}: max err {diff.max():.3e} (ref max {ref_max:.3e}), "
                         f"mean err {diff.mean():.3e} (ref mean {ref_mean:.3e})\n")
    assert diff.max() <= rel_max * max(1.0, ref_max), f"{what}: max abs {diff.max():.3e}"
    if rel_mean is not None:
        assert diff.mean() <= rel_mean * max(1.0, ref_mean), f"{what}: mean abs {diff.mean():.3e}"


def run_fwd_bwd(shape, mode, window, dtype, scale=0.0):
    B, L, n, Hq, Hkv, d = shape
    q, k, v = synth.qkv(B, L, n, Hq, Hkv, d, dtype, DEV)
    dout = synth.normal(q.shape, SEED_DOUT, dtype, DEV)
    o, lse = hd.sfa_fwd(q, k, v, n, mode, window, scale, return_lse=True)
    dq, dk, dv = hd.sfa_bwd(q, k, v, o, dout, lse, n, mode, window, scale)
    torch.cuda.synchronize()
    return q, k, v, dout, dq, dk, dv


@pytest.mark.parametrize("shape,mode,window", [
    ((1, 40, 2, 4, 4, 32), INTRA, 0),
    ((1, 40, 2, 4, 4, 32), CROSS, 0),
    ((2, 23, 3, 4, 2, 64), INTRA, 5),
    ((1, 30, 2, 2, 1, 128), CROSS, 7),
])
def test_bwd_f32_vs_oracle(shape, mode, window):
    q, k, v, dout, dq, dk, dv = run_fwd_bwd(shape, mode, window, torch.float32)
    wq, wk, wv = oracle.sfa_bwd(q.cpu(), k.cpu(), v.cpu(), dout.cpu(), shape[2], mode, window)
    check_grad(dq, wq, "dq", 1e-4)
    check_grad(dk, wk, "dk", 1e-4)
    check_grad(dv, wv, "dv", 1e-4)


BWD_SHAPES = [
    # (B, L, n, Hq, Hkv, d), mode, window
    ((1, 64, 2, 4, 4, 32), INTRA, 0),
    ((1, 64, 2, 4, 4, 32), CROSS, 0),
    ((2, 150, 3, 8, 2, 128), INTRA, 0),     # g=4, ragged tails, two key blocks
    ((2, 150, 3, 8, 2, 128), CROSS, 0),
    ((1, 257, 4, 8, 8, 64), INTRA, 0),      # MHA
    ((1, 130, 4, 16, 2, 128), CROSS, 0),    # g=8
    ((1, 97, 2, 6, 3, 64), INTRA, 0),       # g=2
    ((1, 300, 1, 8, 2, 128), INTRA, 0),     # n=1
    ((1, 200, 4, 8, 2, 128), INTRA, 1),     # window of one token
    ((1, 300, 4, 8, 2, 128), INTRA, 70),    # window edges inside tiles
    ((1, 160, 4, 8, 2, 128), CROSS, 10),    # local cross-stream window
    ((3, 1, 4, 4, 1, 128), INTRA, 0),       # one token
    ((1, 1, 1, 2, 1, 64), CROSS, 0),        # one position
    ((1, 100, 2, 4, 4, 128), CROSS, 0),     # d=128 MHA: one head per staged round
    ((1, 90, 3, 4, 2, 128), INTRA, 0),      # d=128, g=2
    ((1, 70, 2, 6, 2, 128), CROSS, 5),      # d=128, g=3, window
    ((1, 80, 2, 12, 2, 128), INTRA, 0),     # d=128, g=6: head rounds of 4 then 2
    ((1, 600, 1, 4, 1, 128), CROSS, 0),     # 5 query segments of the dK/dV pass + reduction
    ((2, 520, 1, 8, 2, 128), INTRA, 100),   # segments with a window: empty ones skipped
]


@pytest.mark.parametrize("shape,mode,window", BWD_SHAPES)
def test_bwd_bf16_vs_oracle(shape, mode, window):
    q, k, v, dout, dq, dk, dv = run_fwd_bwd(shape, mode, window, torch.bfloat16)
    wq, wk, wv = oracle.sfa_bwd(q.cpu(), k.cpu(), v.cpu(), dout.cpu(), shape[2], mode, window)
    tag = f"{shape} mode={mode} W={window}"
    check_grad(dq, wq, f"dq {tag}", 2e-2, BWD_MEAN_BF16)
    check_grad(dk, wk, f"dk {tag}", 2e-2, BWD_MEAN_BF16)
    check_grad(dv, wv, f"dv {tag}", 2e-2, BWD_MEAN_BF16)


def test_bwd_bf16_custom_scale():
    shape = (1, 70, 2, 4, 2, 64)
    q, k, v, dout, dq, dk, dv = run_fwd_bwd(shape, CROSS, 0, torch.bfloat16, scale=0.05)
    wq, wk, wv = oracle.sfa_bwd(q.cpu(), k.cpu(), v.cpu(), dout.cpu(), 2, CROSS, 0, 0.05)
    check_grad(dq, wq, "dq", 2e-2, BWD_MEAN_BF16)
    check_grad(dk, wk, "dk", 2e-2, BWD_MEAN_BF16)
    check_grad(dv, wv, "dv", 2e-2, BWD_MEAN_BF16)


def test_bwd_full_size_sampled():
    """The 4096-token intra-stream workload (n=4, 32 q / 8 kv heads, d=128):
    sampled dq rows and dk/dv rows against the oracle, plus the invariants
    sum_j dK_j = 0 and sum_j dV_j = sum of dO over each group's heads."""
    c = synth.INTRA_4K
    q, k, v, dout, dq, dk, dv = run_fwd_bwd((c.B, c.L, c.n, c.Hq, c.Hkv, c.d), c.mode, c.window, c.dtype)
    nL = c.n * c.L
    rng = np.random.default_rng(5)
    edge_t = [0, 1, 2, 3, 4, 5, 6, 7, nL - 1, nL - 2, nL - 5, 4 * 64, 4 * 64 - 1, 4 * 128 + 3]
    qrows = np.unique(np.concatenate([
        np.array([t * c.Hq + h for t in edge_t for h in (0, c.Hq - 1)]),
        rng.integers(0, nL * c.Hq, 1024)]))
    krows = np.unique(np.concatenate([
        np.array([t * c.Hkv + h for t in edge_t for h in (0, c.Hkv - 1)]),
        rng.integers(0, nL * c.Hkv, 512)]))
    qc, kc, vc, dc = q.cpu(), k.cpu(), v.cpu(), dout.cpu()
    stats = oracle.row_stats(qc, kc, vc, dc, c.n, c.mode, c.window)
    wq, wk, wv = oracle.sfa_bwd_rows(qc, kc, vc, dc, c.n, c.mode, c.window, qrows=qrows, krows=krows,
                                     stats=stats)
    check_grad(dq.reshape(-1, c.d)[torch.from_numpy(qrows).to(DEV)], wq, "dq rows", 2e-2, BWD_MEAN_BF16)
    check_grad(dk.reshape(-1, c.d)[torch.from_numpy(krows).to(DEV)], wk, "dk rows", 2e-2, BWD_MEAN_BF16)
    check_grad(dv.reshape(-1, c.d)[torch.from_numpy(krows).to(DEV)], wv, "dv rows", 2e-2, BWD_MEAN_BF16)
    # invariants over all keys of each (kv head, stream)
    dk64 = dk.double().reshape(c.B, c.L, c.n, c.Hkv, c.d)
    dv64 = dv.double().reshape(c.B, c.L, c.n, c.Hkv, c.d)
    do64 = dout.double().reshape(c.B, c.L, c.n, c.Hkv, c.Hq // c.Hkv, c.d)
    sk = dk64.sum(dim=1)
    assert sk.abs().max().item() <= 2e-2 * max(1.0, dk64.abs().max().item() * np.sqrt(c.L)), sk.abs().max()
    want_v = do64.sum(dim=(1, 4))
    err_v = (dv64.sum(dim=1) - want_v).abs().max().item()
    assert err_v <= 2e-2 * max(1.0, want_v.abs().max().item()), err_v
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()


def test_bwd_deterministic_and_guarded():
    shape = (1, 150, 4, 8, 2, 128)
    B, L, n, Hq, Hkv, d = shape
    q, k, v = synth.qkv(B, L, n, Hq, Hkv, d, torch.bfloat16, DEV)
    dout = synth.normal(q.shape, SEED_DOUT, torch.bfloat16, DEV)
    for mode, window in ((INTRA, 0), (CROSS, 0), (CROSS, 9)):
        o, lse = hd.sfa_fwd(q, k, v, n, mode, window, return_lse=True)
        guard = 4096
        bufs = [torch.full((x.numel() + 2 * guard,), -7.0, dtype=torch.bfloat16, device=DEV) for x in (q, k, v)]
        outs = [b_[guard:guard + x.numel()].view(x.shape) for b_, x in zip(bufs, (q, k, v))]
        nb = hd.hd_sfa_bwd_workspace_bytes(B, L, n, Hq, Hkv, d)
        ws = torch.full((nb + 2 * guard,), 0xAB, dtype=torch.uint8, device=DEV)
        hd.hd_sfa_bwd(q, k, v, o, dout, lse, *outs, n, mode, window, workspace=ws[guard:guard + nb])
        again = hd.sfa_bwd(q, k, v, o, dout, lse, n, mode, window)
        torch.cuda.synchronize()
        for a, b_ in zip(outs, again):
            assert torch.equal(a, b_)
        for b_, x in zip(bufs, (q, k, v)):
            assert (b_[:guard] == -7.0).all() and (b_[guard + x.numel():] == -7.0).all()
        assert (ws[:guard] == 0xAB).all() and (ws[guard + nb:] == 0xAB).all()
