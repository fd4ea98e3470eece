"""GPU parity of the rotary embedding at expanded positions (hd_rope through
the C ABI) against the CPU oracle, alone and composed with the attention.

Bars, per element of a rotated pair (x0, x1) = (x[c], x[c + d/2]):
  bf16:    |gpu - oracle| <= (2^-8 + 1e-6) * (|x0| + |x1|): one round-to-
           nearest-even output rounding (bf16 carries 8 significant bits, unit
           roundoff 2^-8, and |out| <= |x0| + |x1|) plus the float sine and
           cosine of the double-reduced angle (~1e-7);
  float32: |gpu - oracle| <= 1e-5 * (|x0| + |x1|).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from latent_sequence_length_amd import hd, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def announce(request):
    sys.__stdout__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stdout__.flush()
    yield
    torch.cuda.synchronize()


def check_rope(got, x, want, rel):
    x64 = x.detach().double().cpu().numpy()
    h = x64.shape[-1] // 2
    mag = np.abs(x64[..., :h]) + np.abs(x64[..., h:])
    bound = rel * np.concatenate([mag, mag], axis=-1) + 1e-30
    err = np.abs(got.detach().double().cpu().numpy() - want)
    assert np.isfinite(err).all()
    worst = (err / bound).max()
    sys.__stdout__.write(f"  worst err / bound = {worst:.3f}, max err {err.max():.3e}\n")
    assert worst <= 1.0


@pytest.mark.parametrize("dtype,rel", [(torch.bfloat16, 2.0 ** -8 + 1e-6), (torch.float32, 1e-5)])
@pytest.mark.parametrize("shape,theta", [((1, 300, 4, 128), 10000.0), ((2, 77, 3, 64), 500000.0),
                                         ((1, 1000, 2, 32), 10000.0), ((1, 131072, 1, 128), 10000.0)])
def test_rope_vs_oracle(shape, theta, dtype, rel):
    x = synth.normal(shape, 31, dtype, DEV)
    got = hd.rope(x, theta)
    check_rope(got, x, oracle.rope(x.cpu(), theta), rel)


def test_rope_in_place_and_decode_positions():
    n, H, d = 4, 8, 128
    lens = torch.tensor([8192, 0, 17, 100000], dtype=torch.int32, device=DEV)
    x = synth.normal((4, n, H, d), 32, torch.bfloat16, DEV)
    out = hd.rope(x, 10000.0, lens, n)
    check_rope(out, x, oracle.rope(x.cpu(), 10000.0, pos_base=lens.cpu().numpy(), pos_mul=n), 2.0 ** -8 + 1e-6)
    y = x.clone()
    hd.hd_rope(y, y, 10000.0, lens, n)
    assert torch.equal(y, out)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("mode", [0, 1])
def test_rope_then_attention(dtype, mode):
    """q, k rotated at their expanded positions, then the prefill; the oracle
    composes its own rotation (rounded to the input dtype, RNE) with its own
    attention."""
    B, L, n, Hq, Hkv, d = 1, 96, 4, 8, 2, 128
    q, k, v = synth.qkv(B, L, n, Hq, Hkv, d, dtype, DEV)
    qr, kr = hd.rope(q, 10000.0), hd.rope(k, 10000.0)
    o = hd.sfa_fwd(qr, kr, v, n, mode)
    qo = torch.from_numpy(oracle.rope(q.cpu(), 10000.0)).to(dtype)
    ko = torch.from_numpy(oracle.rope(k.cpu(), 10000.0)).to(dtype)
    want, _ = oracle.sfa_fwd(qo, ko, v.cpu(), n, mode)
    err = np.abs(o.double().cpu().numpy() - want)
    sys.__stdout__.write(f"  max {err.max():.3e} mean {err.mean():.3e}\n")
    if dtype == torch.float32:
        assert err.max() <= 1e-4
    else:
        assert err.max() <= 2e-2 and err.mean() <= 2e-3


INTRA, CROSS = 0, 1


def rope_oracle_fwd(q, k, v, n, mode, window, dtype, rows=None):
    """The oracle's rotation (double, rounded to the input dtype RNE) composed
    with its attention (all rows, or the flat query rows given)."""
    qo = torch.from_numpy(oracle.rope(q.cpu(), 10000.0)).to(dtype)
    ko = torch.from_numpy(oracle.rope(k.cpu(), 10000.0)).to(dtype)
    if rows is None:
        return oracle.sfa_fwd(qo, ko, v.cpu(), n, mode, window)
    return oracle.sfa_rows(qo, ko, v.cpu(), n, mode, window, rows=rows)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape,mode,window", [
    ((1, 96, 4, 8, 2, 128), INTRA, 0), ((1, 96, 4, 8, 2, 128), CROSS, 0),
    ((2, 70, 3, 4, 4, 64), CROSS, 5), ((1, 130, 2, 4, 2, 32), INTRA, 7), ((1, 200, 1, 4, 1, 128), CROSS, 0),
])
def test_fwd_rope_vs_oracle(shape, mode, window, dtype):
    """hd_sfa_fwd_rope: k_rot is hd_rope's output bit for bit; o and lse match
    the oracle's rotation + attention within the prefill's bars."""
    B, L, n, Hq, Hkv, d = shape
    q, k, v = synth.qkv(B, L, n, Hq, Hkv, d, dtype, DEV)
    o, k_rot, lse = hd.sfa_fwd_rope(q, k, v, n, mode, window, return_lse=True)
    assert torch.equal(k_rot, hd.rope(k, 10000.0))
    want, wlse = rope_oracle_fwd(q, k, v, n, mode, window, dtype)
    err = np.abs(o.double().cpu().numpy() - want)
    lerr = np.abs(lse.double().cpu().numpy() - wlse)
    sys.__stdout__.write(f"  o max {err.max():.3e} mean {err.mean():.3e}; lse max {lerr.max():.3e}\n")
    if dtype == torch.float32:
        assert err.max() <= 1e-4 and lerr.max() <= 1e-4
    else:
        assert err.max() <= 2e-2 and err.mean() <= 2e-3 and lerr.max() <= 4e-3


def test_fwd_rope_in_place_and_final_layout():
    """k_rot may be k itself (rotated in place): same o, and k then holds k_rot."""
    B, L, n, Hq, Hkv, d = 1, 150, 4, 8, 2, 128
    q, k, v = synth.qkv(B, L, n, Hq, Hkv, d, torch.bfloat16, DEV)
    o, k_rot = hd.sfa_fwd_rope(q, k, v, n, CROSS, 0)
    kc = k.clone()
    o2 = torch.empty_like(q)
    hd.hd_sfa_fwd_rope(q, kc, v, o2, kc, n, CROSS)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(kc, k_rot)


def test_fwd_rope_full_size_sampled():
    """The 4096-token intra-stream layer (n=4, 32 q / 8 kv heads, d=128) with
    RoPE fused: 4096 sampled rows (expanded positions up to 16383) against the
    oracle's rotation + attention."""
    c = synth.INTRA_4K
    q, k, v = synth.qkv(c.B, c.L, c.n, c.Hq, c.Hkv, c.d, c.dtype, DEV)
    o, _ = hd.sfa_fwd_rope(q, k, v, c.n, c.mode, c.window)
    nL = c.n * c.L
    rng = np.random.default_rng(12)
    edge_t = [0, 1, 2, 3, 4, 5, nL - 1, nL - 2, nL - 5, 8191, 8192, 256, 257]
    rows = np.unique(np.concatenate([np.array([t * c.Hq + h for t in edge_t for h in (0, c.Hq - 1)]),
                                     rng.integers(0, nL * c.Hq, 4096)]))
    want, _ = rope_oracle_fwd(q, k, v, c.n, c.mode, c.window, c.dtype, rows=rows)
    got = o.reshape(-1, c.d)[torch.from_numpy(rows).to(DEV)].double().cpu().numpy()
    err = np.abs(got - want)
    sys.__stdout__.write(f"  rows max {err.max():.3e} mean {err.mean():.3e}\n")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_rope_final_stream_rows_and_final_decode():
    """Compact final-stream rows (t_mul = n, t_add = n-1) and the final
    stream's decode row (pos_base = len, pos_mul = n, t_add = n-1) against the
    oracle, and the final-stream rows equal rows n-1, 2n-1, ... of the plain
    prefill rotation bit for bit (same angles, same kernel)."""
    n, L, H, d = 4, 300, 8, 128
    x = synth.normal((2, n * L, H, d), 33, torch.bfloat16, DEV)
    full = hd.rope(x, 10000.0)
    xf = x[:, n - 1::n].contiguous()
    fin = hd.rope(xf, 10000.0, t_mul=n, t_add=n - 1)
    assert torch.equal(fin, full[:, n - 1::n])
    check_rope(fin, xf, oracle.rope(xf.cpu(), 10000.0, t_mul=n, t_add=n - 1), 2.0 ** -8 + 1e-6)
    lens = torch.tensor([8192, 0, 17], dtype=torch.int32, device=DEV)
    q1 = synth.normal((3, 1, H, d), 34, torch.bfloat16, DEV)
    got = hd.rope(q1, 10000.0, lens, n, t_add=n - 1)
    check_rope(got, q1, oracle.rope(q1.cpu(), 10000.0, pos_base=lens.cpu().numpy(), pos_mul=n, t_add=n - 1),
               2.0 ** -8 + 1e-6)
