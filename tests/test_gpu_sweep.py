"""Seeded sweeps of prefill, decode and backward shapes against the oracle.

The hand-listed cases elsewhere pin named corners; this sweep draws 40
layer shapes from a fixed seed so that the workgroup layouts the kernels
choose from the shape are all exercised together with windows and ragged
ends: query heads per kv head g = 1, 2, 3, 4, 6, 8 (head groups of 1, 2 or
4 per workgroup, hence 4, 2 or 1 blocks of 64 positions per d = 128
workgroup), 1-6 streams, sequence lengths that end anywhere inside a
64-key tile or a 32-query half, intra and cross masks with and without a
window, d = 128 (the hand-scheduled kernel) and d = 32 / 64 (the generic
one).  A quarter of the cases run through the final-stream entry point
(one query row per token, the non-identity query map).

Bars: the output's (2e-2 max / 2e-3 mean absolute) and the bf16 LSE bar
(fp32 summation of the row sum), as in the hand-listed tests.

The decode sweep draws 30 steps (1-4 sequences of ragged cache lengths, 0
and T_cap - 1 included, 1-8 streams, g = 1-8, d = 32 / 64 / 128, intra and
cross with and without a window, bf16 and float32) and checks the output
against the oracle and the appended cache rows bit for bit; the backward
sweep draws 16 bf16 layers and checks dq, dk, dv at the backward bars
(2e-2 max / 4e-3 mean, relative to the gradient's size: rounding each P or
dS operand and each output to bf16, u = 2^-8, averages about u/4 + u/(2
sqrt 3) of the gradient, below u).
"""
import numpy as np
import pytest
import torch

import oracle
from latent_sequence_length_amd import hd, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
INTRA, CROSS = 0, 1
LSE_TOL_BF16 = 5e-4


def _cases(count=40, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        d = int(rng.choice([128, 128, 128, 64, 32]))
        g = int(rng.choice([1, 2, 3, 4, 6, 8]))
        Hkv = int(rng.integers(1, 4))
        Hq = g * Hkv
        if Hq > 16:
            continue
        n = int(rng.integers(1, 7))
        L = int(rng.integers(1, 260))
        if n * L > 900:
            continue
        B = int(rng.choice([1, 1, 2]))
        mode = int(rng.integers(0, 2))
        window = 0 if rng.random() < 0.5 else int(rng.integers(1, max(2, L + 20)))
        final = bool(rng.random() < 0.25)
        out.append(((B, L, n, Hq, Hkv, d), mode, window, final))
    return out


CASES = _cases()


def _ids(c):
    (B, L, n, Hq, Hkv, d), mode, window, final = c
    return f"B{B}-L{L}-n{n}-h{Hq}x{Hkv}-d{d}-{'cross' if mode else 'intra'}-W{window}{'-final' if final else ''}"


def to_np(t):
    return t.detach().to(torch.float64).cpu().numpy()


def _check(got, want, what, max_abs, mean_abs=None):
    diff = np.abs(to_np(got).reshape(want.shape) - want)
    assert np.isfinite(diff).all(), f"{what}: non-finite output"
    assert diff.max() <= max_abs, f"{what}: max abs {diff.max():.3e} > {max_abs}"
    if mean_abs is not None:
        assert diff.mean() <= mean_abs, f"{what}: mean abs {diff.mean():.3e} > {mean_abs}"


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_fwd_bf16_sweep(case):
    (B, L, n, Hq, Hkv, d), mode, window, final = case
    q, k, v = synth.qkv(B, L, n, Hq, Hkv, d, torch.bfloat16, DEV)
    if final:
        qf = q[:, n - 1::n].contiguous()
        o, lse = hd.sfa_fwd_final(qf, k, v, n, mode, window, return_lse=True)
        want, wlse = oracle.sfa_final(qf.cpu(), k.cpu(), v.cpu(), n, mode, window)
    else:
        o, lse = hd.sfa_fwd(q, k, v, n, mode, window, return_lse=True)
        want, wlse = oracle.sfa_fwd(q.cpu(), k.cpu(), v.cpu(), n, mode, window)
    torch.cuda.synchronize()
    _check(o, want, f"o {_ids(case)}", 2e-2, 2e-3)
    _check(lse, wlse, f"lse {_ids(case)}", LSE_TOL_BF16)


def _decode_cases(count=30, seed=20261205):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        d = int(rng.choice([128, 128, 64, 32]))
        g = int(rng.choice([1, 2, 3, 4, 6, 8]))
        Hkv = int(rng.integers(1, 4))
        Hq = g * Hkv
        n = int(rng.integers(1, 9))
        if Hq > 24:
            continue
        B = int(rng.integers(1, 5))
        T_cap = int(rng.integers(1, 300))
        lens = [int(x) for x in rng.integers(0, T_cap, B)]
        if B > 1:
            lens[0] = 0
            lens[-1] = T_cap - 1
        mode = int(rng.integers(0, 2))
        window = 0 if rng.random() < 0.5 else int(rng.integers(1, 40))
        dtype = "bf16" if rng.random() < 0.6 else "f32"
        out.append((B, n, Hq, Hkv, d, T_cap, lens, mode, window, dtype))
    return out


DEC_CASES = _decode_cases()


def _dec_id(c):
    B, n, Hq, Hkv, d, T_cap, lens, mode, window, dtype = c
    return f"B{B}-n{n}-h{Hq}x{Hkv}-d{d}-T{T_cap}-{'cross' if mode else 'intra'}-W{window}-{dtype}"


def _bits(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy()


@pytest.mark.parametrize("case", DEC_CASES, ids=[_dec_id(c) for c in DEC_CASES])
def test_decode_sweep(case):
    B, n, Hq, Hkv, d, T_cap, lens, mode, window, dtype = case
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, kn, vn, kc, vc = synth.decode_inputs(B, n, Hq, Hkv, d, T_cap, dt, DEV)
    kc0, vc0 = kc.cpu(), vc.cpu()
    cl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o = hd.sfa_decode(q, kn, vn, kc, vc, cl, mode, window)
    torch.cuda.synchronize()
    want = oracle.sfa_decode(q.cpu(), kn.cpu(), vn.cpu(), kc0, vc0, lens, mode, window)
    if dt == torch.bfloat16:
        _check(o, want, f"decode {_dec_id(case)}", 2e-2, 2e-3)
    else:
        _check(o, want, f"decode {_dec_id(case)}", 1e-4)
    np.testing.assert_array_equal(_bits(kc), oracle.decode_append(kn.cpu(), kc0, lens).view(_bits(kc).dtype))
    np.testing.assert_array_equal(_bits(vc), oracle.decode_append(vn.cpu(), vc0, lens).view(_bits(vc).dtype))


def _bwd_cases(count=16, seed=20261206):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        d = int(rng.choice([128, 128, 64, 32]))
        g = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.integers(1, 3))
        Hq = g * Hkv
        n = int(rng.integers(1, 5))
        L = int(rng.integers(1, 140))
        if Hq > 16 or n * L > 400:
            continue
        mode = int(rng.integers(0, 2))
        window = 0 if rng.random() < 0.5 else int(rng.integers(1, L + 10))
        out.append(((1, L, n, Hq, Hkv, d), mode, window))
    return out


BWD_CASES = _bwd_cases()
SEED_DOUT = 9


def _check_grad(got, want, what):
    g = to_np(got).reshape(want.shape)
    diff = np.abs(g - want)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    ref_max, ref_mean = np.abs(want).max(), np.abs(want).mean()
    assert diff.max() <= 2e-2 * max(1.0, ref_max), f"{what}: max abs {diff.max():.3e}"
    assert diff.mean() <= 4e-3 * max(1.0, ref_mean), f"{what}: mean abs {diff.mean():.3e}"


@pytest.mark.parametrize("case", BWD_CASES, ids=[_ids((c[0], c[1], c[2], False)) for c in BWD_CASES])
def test_bwd_sweep(case):
    (B, L, n, Hq, Hkv, d), mode, window = case
    q, k, v = synth.qkv(B, L, n, Hq, Hkv, d, torch.bfloat16, DEV)
    dout = synth.normal(q.shape, SEED_DOUT, torch.bfloat16, DEV)
    o, lse = hd.sfa_fwd(q, k, v, n, mode, window, return_lse=True)
    dq, dk, dv = hd.sfa_bwd(q, k, v, o, dout, lse, n, mode, window)
    torch.cuda.synchronize()
    wq, wk, wv = oracle.sfa_bwd(q.cpu(), k.cpu(), v.cpu(), dout.cpu(), n, mode, window)
    tag = _ids((case[0], mode, window, False))
    _check_grad(dq, wq, f"dq {tag}")
    _check_grad(dk, wk, f"dk {tag}")
    _check_grad(dv, wv, f"dv {tag}")
