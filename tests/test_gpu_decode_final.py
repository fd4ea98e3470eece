"""GPU parity of the decode step of a KV-mirror layer (hd_sfa_decode_final
through the C ABI: only the final stream's query of the new token) against
the CPU oracle, plus the append of all n new rows (bit-exact).

Bars are the decode's: bf16 max |gpu - oracle| <= 2e-2 and mean <= 2e-3;
float32 max <= 1e-4.  The output must also equal, bit for bit, row n-1 of a
full hd_sfa_decode on the same inputs in cross layers (the same key rows are
scanned in the same order); intra layers read only stream n-1's cache rows,
so there the comparison is to the oracle's bar.
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


def bits(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy()


def check(got, want, what, dtype):
    diff = np.abs(got.detach().double().cpu().numpy().reshape(want.shape) - want)
    assert np.isfinite(diff).all(), what
    sys.__stdout__.write(f"  {what}: max {diff.max():.3e} mean {diff.mean():.3e}\n")
    if dtype == torch.bfloat16:
        assert diff.max() <= 2e-2 and diff.mean() <= 2e-3, what
    else:
        assert diff.max() <= 1e-4, what


DEC_SHAPES = [
    # B, n, Hq, Hkv, d, T_cap, lens
    (3, 4, 8, 2, 128, 40, [0, 5, 37]),      # g=4 -> 4 query rows per kv head
    (2, 2, 4, 4, 32, 70, [69, 1]),          # g=1
    (2, 4, 16, 2, 64, 33, [32, 7]),         # g=8
    (1, 8, 32, 4, 128, 20, [19]),           # n=8
    (2, 3, 10, 2, 128, 50, [11, 48]),       # n=3 (generic path), g=5
    (2, 1, 8, 1, 128, 300, [299, 150]),     # n=1
    (1, 4, 128, 2, 128, 70, [69]),          # g=64: four query blocks
]


@pytest.mark.parametrize("shape", DEC_SHAPES)
@pytest.mark.parametrize("mode,window", [(INTRA, 0), (CROSS, 0), (INTRA, 3), (CROSS, 2)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_final_vs_oracle(shape, mode, window, dtype):
    B, n, Hq, Hkv, d, T_cap, lens = shape
    q, kn, vn, kc, vc = synth.decode_inputs(B, n, Hq, Hkv, d, T_cap, dtype, DEV)
    qf = q[:, n - 1:n].contiguous()
    kc0, vc0 = kc.cpu(), vc.cpu()
    cl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o = hd.sfa_decode_final(qf, kn, vn, kc, vc, cl, mode, window)
    torch.cuda.synchronize()
    want = oracle.sfa_decode_final(qf.cpu(), kn.cpu(), vn.cpu(), kc0, vc0, lens, mode, window)
    check(o, want, f"decode_final {shape} mode={mode} W={window}", dtype)
    np.testing.assert_array_equal(bits(kc), oracle.decode_append(kn.cpu(), kc0, lens).view(bits(kc).dtype))
    np.testing.assert_array_equal(bits(vc), oracle.decode_append(vn.cpu(), vc0, lens).view(bits(vc).dtype))


@pytest.mark.parametrize("window", [0, 5])
def test_decode_final_cross_equals_full_decode_row(window):
    B, n, Hq, Hkv, d, T_cap = 4, 4, 32, 8, 128, 600
    q, kn, vn, kc, vc = synth.decode_inputs(B, n, Hq, Hkv, d, T_cap, torch.bfloat16, DEV)
    cl = torch.tensor([599, 0, 300, 64], dtype=torch.int32, device=DEV)
    o_full = hd.sfa_decode(q, kn, vn, kc.clone(), vc.clone(), cl, CROSS, window)
    o = hd.sfa_decode_final(q[:, n - 1:n].contiguous(), kn, vn, kc, vc, cl, CROSS, window)
    torch.cuda.synchronize()
    assert torch.equal(o, o_full[:, n - 1:n])


@pytest.mark.parametrize("mode", [INTRA, CROSS])
def test_decode_final_full_size_sampled(mode):
    """B=64, 8192 cached tokens x 4 streams, 32 q / 8 kv heads, d=128: the
    final-stream query of every sequence, checked against the oracle on four
    sequences, ragged lengths (0 and T_cap-1 included)."""
    cfg = synth.DECODE_8K
    T_cap = cfg.ctx + 8
    lens = [int(x) for x in np.random.default_rng(6).integers(0, T_cap, cfg.B)]
    lens[0], lens[-1] = 0, T_cap - 1
    q, kn, vn, kc, vc = synth.decode_inputs(cfg.B, cfg.n, cfg.Hq, cfg.Hkv, cfg.d, T_cap, cfg.dtype, DEV)
    qf = q[:, cfg.n - 1:cfg.n].contiguous()
    picks = [0, 17, 42, cfg.B - 1]
    kc0 = [kc[b].cpu() for b in picks]
    vc0 = [vc[b].cpu() for b in picks]
    cl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o = hd.sfa_decode_final(qf, kn, vn, kc, vc, cl, mode)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    for j, b in enumerate(picks):
        want = oracle.sfa_decode_final(qf[b:b + 1].cpu(), kn[b:b + 1].cpu(), vn[b:b + 1].cpu(), kc0[j][None],
                                       vc0[j][None], [lens[b]], mode)
        check(o[b:b + 1], want, f"decode_final b={b} len={lens[b]} mode={mode}", cfg.dtype)
        np.testing.assert_array_equal(bits(kc[b, lens[b]]), bits(kn[b]))


def test_decode_final_deterministic_and_guarded():
    B, n, Hq, Hkv, d, T_cap = 4, 4, 32, 8, 128, 600
    q, kn, vn, kc, vc = synth.decode_inputs(B, n, Hq, Hkv, d, T_cap, torch.bfloat16, DEV)
    qf = q[:, n - 1:n].contiguous()
    cl = torch.tensor([599, 0, 300, 64], dtype=torch.int32, device=DEV)
    for mode in (INTRA, CROSS):
        guard = 2048
        buf = torch.full((qf.numel() + 2 * guard,), 3.0, dtype=torch.bfloat16, device=DEV)
        o1 = buf[guard:guard + qf.numel()].view(qf.shape)
        ws = torch.full((hd.hd_sfa_decode_workspace_bytes(B, n, Hq, Hkv, d, T_cap) + 4096,), 255,
                        dtype=torch.uint8, device=DEV)
        hd.hd_sfa_decode(qf, kn, vn, kc, vc, cl, o1, mode, 0, 0.0, ws, final_only=True)
        o2 = hd.sfa_decode_final(qf, kn, vn, kc, vc, cl, mode)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
        assert (buf[:guard] == 3.0).all() and (buf[guard + qf.numel():] == 3.0).all()
