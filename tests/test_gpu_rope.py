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
