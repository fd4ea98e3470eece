"""GPU parity of the backward of the final-stream queries of a KV-mirror layer
(hd_sfa_fwd_final then hd_sfa_bwd_final through the C ABI) against the CPU
oracle's chain-rule gradients.

Bars (as for the full layer's backward):
  - float32: max |gpu - oracle| <= 1e-4 * max(1, max |oracle|);
  - bf16: max <= 2e-2 * max(1, max |oracle|), mean <= 4e-3 * max(1, mean |oracle|).
Small shapes are compared on every element (dk and dv over all n*L key rows,
including the rows of streams no final query sees in an intra layer, which
must be exactly zero); the 4096-token workload on sampled rows plus the
row-sum invariants over all keys.
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


# mean bar for bf16 gradients: rounding each P / dS operand and each output to
# bf16 (u = 2^-8) averages about u/4 + u/(2 sqrt 3) of the gradient's size, below u
BWD_MEAN_BF16 = 4e-3


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


def run_final_fwd_bwd(shape, mode, window, dtype, scale=0.0):
    B, L, n, Hq, Hkv, d = shape
    q, k, v = synth.qkv(B, L, n, Hq, Hkv, d, dtype, DEV)
    qf = q[:, n - 1::n].contiguous()
    del q
    dof = synth.normal(qf.shape, SEED_DOUT, dtype, DEV)
    o, lse = hd.sfa_fwd_final(qf, k, v, n, mode, window, scale, return_lse=True)
    # poison the outputs so rows the kernels fail to write are caught
    dq, dk, dv = (torch.full_like(x, 7.0) for x in (qf, k, v))
    hd.hd_sfa_bwd_final(qf, k, v, o, dof, lse, dq, dk, dv, n, mode, window, scale)
    torch.cuda.synchronize()
    return qf, k, v, dof, dq, dk, dv


@pytest.mark.parametrize("shape,mode,window", [
    ((1, 40, 2, 4, 4, 32), INTRA, 0),
    ((1, 40, 2, 4, 4, 32), CROSS, 0),
    ((2, 23, 3, 4, 2, 64), CROSS, 5),
    ((1, 30, 4, 2, 1, 128), INTRA, 7),
])
def test_final_bwd_f32_vs_oracle(shape, mode, window):
    qf, k, v, dof, dq, dk, dv = run_final_fwd_bwd(shape, mode, window, torch.float32)
    wq, wk, wv = oracle.sfa_final_bwd(qf.cpu(), k.cpu(), v.cpu(), dof.cpu(), shape[2], mode, window)
    check_grad(dq, wq, "dq", 1e-4)
    check_grad(dk, wk, "dk", 1e-4)
    check_grad(dv, wv, "dv", 1e-4)


FINAL_BWD_SHAPES = [
    # (B, L, n, Hq, Hkv, d), mode, window
    ((1, 64, 2, 4, 4, 32), INTRA, 0),
    ((1, 64, 2, 4, 4, 32), CROSS, 0),
    ((2, 150, 3, 8, 2, 128), CROSS, 0),     # g=4, ragged tails, several key blocks
    ((2, 150, 3, 8, 2, 128), INTRA, 0),
    ((1, 257, 4, 8, 8, 64), CROSS, 0),      # MHA, d=64
    ((1, 130, 4, 16, 2, 128), CROSS, 10),   # g=8, local cross-stream window
    ((1, 300, 4, 8, 2, 128), INTRA, 70),    # window edges inside tiles
    ((1, 97, 1, 6, 3, 64), CROSS, 0),       # n=1: plain causal, g=2
    ((1, 200, 8, 4, 1, 128), CROSS, 3),     # n=8
    ((3, 1, 4, 4, 1, 128), CROSS, 0),       # one token
    ((1, 1, 1, 2, 1, 64), INTRA, 0),        # one position
    ((1, 300, 4, 4, 2, 128), INTRA, 0),     # g=2; 3 query segments of the dK/dV pass
    ((1, 90, 3, 6, 2, 128), CROSS, 4),      # g=3, window
    # final-stream cross (non-identity query map) with query segments of the
    # dK/dV pass and their reduction: 300 final queries over 1200 positions
    ((1, 300, 4, 8, 2, 128), CROSS, 0),
    ((1, 300, 4, 8, 2, 128), CROSS, 20),
]


@pytest.mark.parametrize("shape,mode,window", FINAL_BWD_SHAPES)
def test_final_bwd_bf16_vs_oracle(shape, mode, window):
    qf, k, v, dof, dq, dk, dv = run_final_fwd_bwd(shape, mode, window, torch.bfloat16)
    wq, wk, wv = oracle.sfa_final_bwd(qf.cpu(), k.cpu(), v.cpu(), dof.cpu(), shape[2], mode, window)
    tag = f"{shape} mode={mode} W={window}"
    check_grad(dq, wq, f"dq {tag}", 2e-2, BWD_MEAN_BF16)
    check_grad(dk, wk, f"dk {tag}", 2e-2, BWD_MEAN_BF16)
    check_grad(dv, wv, f"dv {tag}", 2e-2, BWD_MEAN_BF16)
    if mode == INTRA:  # keys of streams 0..n-2 get exactly nothing
        n = shape[2]
        other = torch.ones(dk.shape[1], dtype=torch.bool, device=DEV)
        other[n - 1::n] = False
        assert (dk[:, other] == 0).all() and (dv[:, other] == 0).all()


def test_final_bwd_custom_scale():
    shape = (1, 70, 3, 4, 2, 64)
    qf, k, v, dof, dq, dk, dv = run_final_fwd_bwd(shape, CROSS, 0, torch.bfloat16, scale=0.05)
    wq, wk, wv = oracle.sfa_final_bwd(qf.cpu(), k.cpu(), v.cpu(), dof.cpu(), 3, CROSS, 0, 0.05)
    check_grad(dq, wq, "dq", 2e-2, BWD_MEAN_BF16)
    check_grad(dk, wk, "dk", 2e-2, BWD_MEAN_BF16)
    check_grad(dv, wv, "dv", 2e-2, BWD_MEAN_BF16)


@pytest.mark.parametrize("mode", [CROSS, INTRA])
def test_final_bwd_full_size_sampled(mode):
    """Final-stream queries of the 4096-token layer (n=4, 32 q / 8 kv heads,
    d=128): sampled dq rows and dk/dv rows (every stream) against the oracle,
    plus the invariants sum_j dK_j = 0 and sum_j dV_j = sum of dOf over the
    group's heads, over all key rows."""
    c = synth.CROSS_4K
    shape = (c.B, c.L, c.n, c.Hq, c.Hkv, c.d)
    qf, k, v, dof, dq, dk, dv = run_final_fwd_bwd(shape, mode, 0, c.dtype)
    nL = c.n * c.L
    rng = np.random.default_rng(6)
    edge_i = [0, 1, 2, 31, 32, 63, 64, c.L - 2, c.L - 1]
    edge_t = [0, 1, 2, 3, 4, 127, 128, 129, 255, 256, nL - 5, nL - 2, nL - 1]
    qrows = np.unique(np.concatenate([np.array([i * c.Hq + h for i in edge_i for h in (0, c.Hq - 1)]),
                                      rng.integers(0, c.L * c.Hq, 512)]))
    krows = np.unique(np.concatenate([np.array([t * c.Hkv + h for t in edge_t for h in (0, c.Hkv - 1)]),
                                      rng.integers(0, nL * c.Hkv, 384)]))
    qc, kc, vc, dc = qf.cpu(), k.cpu(), v.cpu(), dof.cpu()
    stats = oracle.final_row_stats(qc, kc, vc, dc, c.n, mode)
    wq, wk, wv = oracle.sfa_final_bwd_rows(qc, kc, vc, dc, c.n, mode, qrows=qrows, krows=krows, stats=stats)
    check_grad(dq.reshape(-1, c.d)[torch.from_numpy(qrows).to(DEV)], wq, "dq rows", 2e-2, BWD_MEAN_BF16)
    check_grad(dk.reshape(-1, c.d)[torch.from_numpy(krows).to(DEV)], wk, "dk rows", 2e-2, BWD_MEAN_BF16)
    check_grad(dv.reshape(-1, c.d)[torch.from_numpy(krows).to(DEV)], wv, "dv rows", 2e-2, BWD_MEAN_BF16)
    dk64 = dk.double().reshape(c.B, nL, c.Hkv, c.d)
    dv64 = dv.double().reshape(c.B, nL, c.Hkv, c.d)
    do64 = dof.double().reshape(c.B, c.L, c.Hkv, c.Hq // c.Hkv, c.d)
    sk = dk64.sum(dim=1)
    assert sk.abs().max().item() <= 2e-2 * max(1.0, dk64.abs().max().item() * np.sqrt(c.L)), sk.abs().max()
    want_v = do64.sum(dim=(1, 3))
    err_v = (dv64.sum(dim=1) - want_v).abs().max().item()
    assert err_v <= 2e-2 * max(1.0, want_v.abs().max().item()), err_v
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()


@pytest.mark.parametrize("L,cases", [
    (150, ((INTRA, 0), (CROSS, 0), (CROSS, 9))),
    (300, ((CROSS, 0), (CROSS, 20))),  # query segments on the final-stream cross map: partial rows in the workspace
])
def test_final_bwd_deterministic_and_guarded(L, cases):
    B, n, Hq, Hkv, d = 1, 4, 8, 2, 128
    q, k, v = synth.qkv(B, L, n, Hq, Hkv, d, torch.bfloat16, DEV)
    qf = q[:, n - 1::n].contiguous()
    dof = synth.normal(qf.shape, SEED_DOUT, torch.bfloat16, DEV)
    guard = 4096
    for mode, window in cases:
        o, lse = hd.sfa_fwd_final(qf, k, v, n, mode, window, return_lse=True)
        bufs = [torch.full((x.numel() + 2 * guard,), -7.0, dtype=torch.bfloat16, device=DEV) for x in (qf, k, v)]
        outs = [b_[guard:guard + x.numel()].view(x.shape) for b_, x in zip(bufs, (qf, k, v))]
        nb = hd.hd_sfa_bwd_final_workspace_bytes(B, L, n, Hq, Hkv, d)
        ws = torch.full((nb + 2 * guard,), 0xAB, dtype=torch.uint8, device=DEV)
        hd.hd_sfa_bwd_final(qf, k, v, o, dof, lse, *outs, n, mode, window, workspace=ws[guard:guard + nb])
        again = hd.sfa_bwd_final(qf, k, v, o, dof, lse, n, mode, window)
        torch.cuda.synchronize()
        for a, b_ in zip(outs, again):
            assert torch.equal(a, b_)
        for b_, x in zip(bufs, (qf, k, v)):
            assert (b_[:guard] == -7.0).all() and (b_[guard + x.numel():] == -7.0).all()
        assert (ws[:guard] == 0xAB).all() and (ws[guard + nb:] == 0xAB).all()
