"""Benchmark of the Stream-Factorized Attention hot path on one MI355X.

One step = one pass over every step of the hot path on synthetic inputs that
are already resident in HBM:
  expand-embed   64 sequences x 1 token x 4 streams from 4 tables 160000 x 7168 bf16
  intra prefill  n=4, L=4096 (nL=16384), 32 q / 8 kv heads, d=128, bf16   <- headline
  intra prefill  n=1, L=4096 control (for the n=4 / n=1 time ratio)
  cross prefill  same shapes as the headline, dense causal over 16384 positions
  decode         64 sequences, 8192 cached tokens x 4 streams, 32 q / 8 kv heads,
                 intra and cross (one new token, 4 stream queries each)
After the timed steps, the extension rows are timed in a loop of their own
(reported under "components", outside ms_per_step):
  final-stream   the final stream's queries of the headline shapes (intra and
                 cross) and the backward of the cross one; decode of the final
                 stream's query (intra and cross)
  rotary embed   q and k of the headline layer at the expanded positions, and
                 the prefill with the rotation of q fused in
  backward       dQ, dK, dV of the headline intra-stream layer (given o, lse, dO)
With --long, also the 32k-token layers (n=4, nL=131072, 16 q / 4 kv heads):
intra-stream with a 4096-token window, local cross-stream with a 4096-token
window, and a full cross-stream layer.
Each call is timed with HIP events on the stream it is launched on.  The
headline value is useful TFLOP/s of the intra-stream prefill (4*d*Hq FLOPs per
visible query/key pair).  Prints one JSON line.
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

from latent_sequence_length_amd import hd, synth

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E


def useful_flops(B, L, n, Hq, d, mode, window=0):
    """4*d*Hq*(number of visible (query, key) pairs): QK^T and PV, 2 flops per
    multiply-add.  Intra: per stream, tokens j <= i within the window; cross:
    positions t_k <= t_q within n*window positions."""
    def tri(T, w):  # sum over q in [0, T) of min(q + 1, w) (w = 0: no window)
        if w <= 0 or w >= T:
            return T * (T + 1) // 2
        return w * (w + 1) // 2 + (T - w) * w
    pairs = n * tri(L, window) if mode == 0 else tri(n * L, n * window)
    return 4.0 * d * Hq * B * pairs


def useful_flops_final(B, L, n, Hq, d, mode, window=0):
    """Final-stream queries of a KV-mirror layer: query i sees tokens
    j <= i (within the window) of stream n-1 only (intra) or of all n
    streams (cross)."""
    def tri(T, w):
        if w <= 0 or w >= T:
            return T * (T + 1) // 2
        return w * (w + 1) // 2 + (T - w) * w
    pairs = tri(L, window) * (n if mode == 1 else 1)
    return 4.0 * d * Hq * B * pairs


def measured_peaks(dev):
    """The machine's sustained rates, reported beside the published peaks:
    an MFMA-only loop (libhd_probe.so, 8 independent bf16 32x32x16 chains
    per wave, 4 waves per SIMD) and a 1 GiB device copy (read + write)."""
    out = {}
    path = os.path.join(ROOT, "latent_sequence_length_amd", "libhd_probe.so")
    if os.path.exists(path):
        lib = ctypes.CDLL(path)
        lib.hd_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        lib.hd_probe_mfma_bf16.restype = ctypes.c_double
        blocks, iters = 4096, 2048
        sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        lib.hd_probe_mfma_bf16(blocks, iters, ctypes.c_void_p(sink.data_ptr()), st)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fl = sum(lib.hd_probe_mfma_bf16(blocks, iters, ctypes.c_void_p(sink.data_ptr()), st) for _ in range(5))
        e.record()
        torch.cuda.synchronize()
        if fl > 0:
            out["mfma_bf16_TFLOPs"] = round(fl / s.elapsed_time(e) / 1e9, 1)
    src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(5):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    out["copy_GBps"] = round(5 * 2 * src.numel() * 2 / s.elapsed_time(e) / 1e6, 1)
    return out


def measured_traffic(name):
    """HBM bytes per launch of a kernel from its committed PMC summary
    (profiles/<name>.md: FETCH_SIZE + WRITE_SIZE scaled by a copy kernel), or
    None when the summary is missing or the kernel source has changed since
    the counters were taken (the summary records the source's SHA-256)."""
    path = os.path.join(ROOT, "profiles", name + ".md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.startswith("- `"):
            key, val = line[3:].split("`:", 1)
            fields[key.strip()] = val.strip().strip("`")
    src = fields.get("source")
    if not src or "traffic_bytes_per_launch" not in fields:
        return None
    digest = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()
    if digest != fields.get("source_sha256"):
        return None
    return int(fields["traffic_bytes_per_launch"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-oracle sample budget")
    ap.add_argument("--long", action="store_true", help="also time the 32k-token (nL=131072) layers")
    ap.add_argument("--only", default="", help="comma list of components to run (profiling); 'peaks' runs the measured-peak loops alone")
    return ap.parse_args()


class Timer:
    """Accumulates HIP-event durations of launches on the current stream."""

    def __init__(self):
        self.ms = {}
        self.pending = []

    def run(self, name, fn):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.pending.append((name, s, e))

    def collect(self):
        torch.cuda.synchronize()
        for name, s, e in self.pending:
            self.ms.setdefault(name, []).append(s.elapsed_time(e))
        self.pending = []


def cpu_baseline(budget_s):
    """Time the oracle on a bounded random sample of the headline workload."""
    import oracle

    c = synth.INTRA_4K
    q, k, v = synth.qkv(c.B, c.L, c.n, c.Hq, c.Hkv, c.d, c.dtype, "cpu")
    nL = c.n * c.L
    rng = np.random.default_rng(123)
    oracle.sfa_rows(q, k, v, c.n, c.mode, c.window, rows=np.array([0], dtype=np.int64))  # load + warm
    flops = 0.0
    rows_done = 0
    t0 = time.perf_counter()
    batch = 256
    while time.perf_counter() - t0 < budget_s:
        rows = rng.integers(0, c.B * nL * c.Hq, batch).astype(np.int64)
        oracle.sfa_rows(q, k, v, c.n, c.mode, c.window, rows=rows)
        t = (rows // c.Hq) % nL
        visible = t // c.n + 1  # intra, no window: tokens 0..i of the query's stream
        flops += float(4 * c.d * visible.sum())
        rows_done += batch
        batch = min(batch * 2, 8192)
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{rows_done} random query rows of the n=4 L=4096 intra-stream prefill "
                  f"({rows_done / (c.B * nL * c.Hq):.2%} of all rows), {dt:.1f} s, double-precision C oracle",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU path is not built.",
              file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    dev = "cuda"
    only = set(x for x in args.only.split(",") if x)
    want = (lambda name: not only or name in only)
    if only == {"peaks"}:  # profiling: the measured-peak loops alone
        print(json.dumps({"measured_peaks": measured_peaks(dev)}), flush=True)
        return

    I = synth.INTRA_4K
    I1 = synth.INTRA_4K_N1
    X = synth.CROSS_4K
    Dc = synth.DECODE_8K
    E = synth.EMBED_DECODE

    comps = {}   # name -> (callable, useful flops, algorithmic bytes)

    def prefill(cfg):
        """(callable, useful flops, algorithmic bytes) of one prefill call on
        inputs drawn once; bytes = q, k, v read + o written."""
        q, k, v = synth.qkv(cfg.B, cfg.L, cfg.n, cfg.Hq, cfg.Hkv, cfg.d, cfg.dtype, dev)
        o = torch.empty_like(q)
        fl = useful_flops(cfg.B, cfg.L, cfg.n, cfg.Hq, cfg.d, cfg.mode, cfg.window)
        by = 2 * (2 * q.numel() + k.numel() + v.numel())
        return (lambda: hd.hd_sfa_fwd(q, k, v, o, cfg.n, cfg.mode, cfg.window), fl, by)

    if want("intra_n4"):
        comps["intra_n4"] = prefill(I)
    if want("intra_n1"):
        comps["intra_n1"] = prefill(I1)
    if want("cross_n4"):
        comps["cross_n4"] = prefill(X)
    def final(cfg):
        """Final-stream queries (rows t = i*n + n-1 only, compact) of the
        layer's shapes over K/V of every stream; bytes = q, o of the final
        stream + the K/V rows the mask reaches (all for cross, stream n-1's
        for intra)."""
        q, k, v = synth.qkv(cfg.B, cfg.L, cfg.n, cfg.Hq, cfg.Hkv, cfg.d, cfg.dtype, dev)
        qf = q[:, cfg.n - 1::cfg.n].contiguous()
        del q
        o = torch.empty_like(qf)
        fl = useful_flops_final(cfg.B, cfg.L, cfg.n, cfg.Hq, cfg.d, cfg.mode, cfg.window)
        kv = (k.numel() + v.numel()) // (cfg.n if cfg.mode == 0 else 1)
        by = 2 * (2 * qf.numel() + kv)
        return (lambda: hd.hd_sfa_fwd_final(qf, k, v, o, cfg.n, cfg.mode, cfg.window), fl, by)

    if want("final_cross_n4"):
        comps["final_cross_n4"] = final(X)
    if want("final_intra_n4"):
        comps["final_intra_n4"] = final(I)

    def backward(cfg):
        """(callable, useful flops, algorithmic bytes) of one backward call of
        the layer; o and lse come from one forward call outside the timed
        region, dO is a seeded draw like q, k, v."""
        q, k, v = synth.qkv(cfg.B, cfg.L, cfg.n, cfg.Hq, cfg.Hkv, cfg.d, cfg.dtype, dev)
        dout = synth.normal(q.shape, 9, cfg.dtype, dev)
        o, lse = hd.sfa_fwd(q, k, v, cfg.n, cfg.mode, cfg.window, return_lse=True)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(hd.hd_sfa_bwd_workspace_bytes(cfg.B, cfg.L, cfg.n, cfg.Hq, cfg.Hkv, cfg.d),
                         dtype=torch.uint8, device=dev)
        # useful FLOPs: five products of the forward's size over the visible
        # pairs (S recomputed, dP, dV, dK, dQ) = 2.5x the forward's count
        fl = 2.5 * useful_flops(cfg.B, cfg.L, cfg.n, cfg.Hq, cfg.d, cfg.mode, cfg.window)
        # q, o, dO, k, v read; dq, dk, dv written; lse read, D written and read
        by = 2 * (4 * q.numel() + 4 * k.numel()) + 3 * 4 * cfg.B * cfg.Hq * cfg.n * cfg.L
        return (lambda: hd.hd_sfa_bwd(q, k, v, o, dout, lse, dq, dk, dv, cfg.n, cfg.mode, cfg.window,
                                      workspace=ws), fl, by)

    if want("bwd_intra_n4"):
        comps["bwd_intra_n4"] = backward(I)
    if want("bwd_intra_n1"):
        comps["bwd_intra_n1"] = backward(I1)
    def backward_final(cfg):
        """Backward of the final-stream queries of the layer (KV-mirror
        training): dq of the L final rows, dk/dv of all n*L positions."""
        q, k, v = synth.qkv(cfg.B, cfg.L, cfg.n, cfg.Hq, cfg.Hkv, cfg.d, cfg.dtype, dev)
        qf = q[:, cfg.n - 1::cfg.n].contiguous()
        del q
        dof = synth.normal(qf.shape, 9, cfg.dtype, dev)
        of, lsef = hd.sfa_fwd_final(qf, k, v, cfg.n, cfg.mode, cfg.window, return_lse=True)
        dqf, dkf, dvf = torch.empty_like(qf), torch.empty_like(k), torch.empty_like(v)
        wsf = torch.empty(hd.hd_sfa_bwd_final_workspace_bytes(cfg.B, cfg.L, cfg.n, cfg.Hq, cfg.Hkv, cfg.d),
                          dtype=torch.uint8, device=dev)
        fl = 2.5 * useful_flops_final(cfg.B, cfg.L, cfg.n, cfg.Hq, cfg.d, cfg.mode, cfg.window)
        by = 2 * (4 * qf.numel() + 4 * k.numel()) + 3 * 4 * cfg.B * cfg.Hq * cfg.L
        return (lambda: hd.hd_sfa_bwd_final(qf, k, v, of, dof, lsef, dqf, dkf, dvf, cfg.n, cfg.mode, cfg.window,
                                            workspace=wsf), fl, by)

    if want("bwd_final_cross_n4"):
        comps["bwd_final_cross_n4"] = backward_final(X)
    if want("rope_qk"):
        # rotary embedding of the headline layer's q and k at the expanded
        # positions (in place); bytes = read + write of q and k
        q, k, _ = synth.qkv(I.B, I.L, I.n, I.Hq, I.Hkv, I.d, I.dtype, dev)

        def run_rope(q=q, k=k):
            hd.hd_rope(q, q, 10000.0)
            hd.hd_rope(k, k, 10000.0)

        comps["rope_qk"] = (run_rope, 0.0, 2 * 2 * (q.numel() + k.numel()))
    if want("rope_fwd_intra_n4"):
        # the headline layer with RoPE fused: k rotated into k_rot, q rotated
        # inside the prefill kernel (compare rope_qk + intra_n4)
        q, k, v = synth.qkv(I.B, I.L, I.n, I.Hq, I.Hkv, I.d, I.dtype, dev)
        o, k_rot = torch.empty_like(q), torch.empty_like(k)
        fl = useful_flops(I.B, I.L, I.n, I.Hq, I.d, I.mode, I.window)
        by = 2 * (2 * q.numel() + 3 * k.numel() + v.numel())
        comps["rope_fwd_intra_n4"] = (lambda q=q, k=k, v=v, o=o, kr=k_rot: hd.hd_sfa_fwd_rope(q, k, v, o, kr, I.n, I.mode),
                                      fl, by)
    if want("decode_intra") or want("decode_cross") or want("decode_final_intra") or want("decode_final_cross"):
        T_cap = Dc.ctx + 8
        dq, dkn, dvn, dkc, dvc = synth.decode_inputs(Dc.B, Dc.n, Dc.Hq, Dc.Hkv, Dc.d, T_cap, Dc.dtype, dev)
        dcl = torch.full((Dc.B,), Dc.ctx, dtype=torch.int32, device=dev)
        do = torch.empty_like(dq)
        ws = torch.empty(hd.hd_sfa_decode_workspace_bytes(Dc.B, Dc.n, Dc.Hq, Dc.Hkv, Dc.d, T_cap),
                         dtype=torch.uint8, device=dev)
        # algorithmic bytes: cache read for ctx+1 tokens (the new row from
        # k_new/v_new), q read, o written, new rows written to the cache
        tok_bytes = Dc.n * Dc.Hkv * Dc.d * 2
        by = 2 * (Dc.ctx * tok_bytes * Dc.B) + 2 * dq.numel() * 2 + 2 * dkn.numel() * 2 * 2
        for mode, name in ((0, "decode_intra"), (1, "decode_cross")):
            if want(name):
                keys = (Dc.ctx + 1) if mode == 0 else None
                g = Dc.Hq // Dc.Hkv
                if mode == 0:
                    pairs = Dc.B * Dc.n * Dc.Hq * keys
                else:
                    pairs = Dc.B * Dc.Hq * sum(Dc.ctx * Dc.n + s + 1 for s in range(Dc.n))
                fl = 4.0 * Dc.d * pairs
                comps[name] = (lambda mode=mode: hd.hd_sfa_decode(dq, dkn, dvn, dkc, dvc, dcl, do, mode, 0, 0.0, ws),
                               fl, by)
                del g
        # KV-mirror layers: the final stream's query only (intra reads stream
        # n-1's cache rows alone, cross the whole cache)
        dqf = dq[:, Dc.n - 1:Dc.n].contiguous()
        dof = torch.empty_like(dqf)
        for mode, name in ((0, "decode_final_intra"), (1, "decode_final_cross")):
            if want(name):
                rows = Dc.ctx if mode == 0 else Dc.ctx * Dc.n
                by_f = 2 * rows * Dc.Hkv * Dc.d * 2 * Dc.B + 2 * 2 * dqf.numel() + 2 * dkn.numel() * 2 * 2
                pairs = Dc.B * Dc.Hq * ((Dc.ctx + 1) if mode == 0 else (Dc.ctx + 1) * Dc.n)
                comps[name] = (lambda mode=mode: hd.hd_sfa_decode(dqf, dkn, dvn, dkc, dvc, dcl, dof, mode, 0, 0.0, ws,
                                                                  final_only=True), 4.0 * Dc.d * pairs, by_f)
    if want("embed"):
        tabs = synth.tables(E["n"], E["V"], E["D"], E["dtype"], dev)
        # 64 rotating id sets so rows come from HBM rather than the last-level cache
        idsets = [synth.token_ids(E["B"], E["L"], E["V"], seed=1000 + r, device=dev) for r in range(64)]
        eo = torch.empty((E["B"], E["n"] * E["L"], E["D"]), dtype=E["dtype"], device=dev)
        ctr = [0]

        def run_embed():
            hd.hd_expand_embed(idsets[ctr[0] % 64], tabs, eo)
            ctr[0] += 1

        by = 2 * eo.numel() * 2 + E["B"] * E["L"] * 4
        comps["embed"] = (run_embed, 0.0, by)
    if args.long:
        for cfg, name in ((synth.LONG_INTRA_W, "long_intra_w4096"), (synth.LONG_CROSS_W, "long_cross_w4096"),
                          (synth.LONG_CROSS, "long_cross")):
            if want(name):
                comps[name] = prefill(cfg)
    if "copy" in only:
        # calibration only, never part of the step: a plain elementwise copy
        # of 512 MiB, which reads and writes exactly that many bytes; its HBM
        # byte counters scale the counters of the kernels above
        src = torch.randn(256 << 20, device=dev).to(torch.bfloat16)
        dst = torch.empty_like(src)
        comps["copy"] = (lambda: torch.mul(src, 1.0, out=dst), 0.0, 2 * src.numel() * 2)
    torch.cuda.synchronize()

    # The step is one pass over the hot path's rows (gather, prefill n=4 and
    # the n=1 control, cross layer, decode).  With no --only, the extension
    # rows (backward, RoPE, final-stream queries) are timed in a loop of their
    # own after the step, so they neither lengthen nor heat the timed step.
    STEP_ROWS = ("intra_n4", "intra_n1", "cross_n4", "decode_intra", "decode_cross", "embed")
    if only:
        step_comps, extra_comps = comps, {}
    else:
        step_comps = {k: v for k, v in comps.items() if k in STEP_ROWS}
        extra_comps = {k: v for k, v in comps.items() if k not in STEP_ROWS}

    def timed_loop(group, steps, warmup, tm):
        for _ in range(warmup):
            for name, (fn, _, _) in group.items():
                tm.run(name, fn)
        tm.collect()
        tm.ms = {}
        torch.cuda.synchronize()
        s_ev = torch.cuda.Event(enable_timing=True)
        e_ev = torch.cuda.Event(enable_timing=True)
        s_ev.record()
        for _ in range(steps):
            for name, (fn, _, _) in group.items():
                tm.run(name, fn)
        e_ev.record()
        tm.collect()
        return s_ev.elapsed_time(e_ev)

    timer = Timer()
    total_ms = timed_loop(step_comps, args.steps, args.warmup, timer)
    ms_per_step = total_ms / max(args.steps, 1)
    if extra_comps:
        extra_timer = Timer()
        timed_loop(extra_comps, args.steps, args.warmup, extra_timer)
        timer.ms.update(extra_timer.ms)

    report = {}
    for name, (fn, fl, by) in comps.items():
        t = float(np.mean(timer.ms[name]))
        report[name] = {"ms": round(t, 4), "ms_min": round(float(np.min(timer.ms[name])), 4)}
        if fl:
            report[name]["TFLOP/s"] = round(fl / t / 1e9, 2)
        report[name]["GB/s"] = round(by / t / 1e6, 1)

    value = report.get("intra_n4", {}).get("TFLOP/s")
    ratio = None
    if "intra_n4" in report and "intra_n1" in report:
        ratio = round(report["intra_n4"]["ms"] / report["intra_n1"]["ms"], 3)
    roof = None
    if "intra_n4" in report:
        fl = comps["intra_n4"][1]
        ach = fl / report["intra_n4"]["ms"] / 1e9
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic("sfa_fwd_bf16_d128__intra_n4_L4096__hbm_bytes"),
                "kernel": "sfa_fwd_bf16_d128_kernel", "per_launch_flops": fl}
    roof_dec = None
    if "decode_intra" in report:
        by = comps["decode_intra"][2]
        ach = by / report["decode_intra"]["ms"] / 1e6
        roof_dec = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": round(ach / PEAK_HBM_GBPS, 4), "per_launch_bytes": by,
                    "traffic": measured_traffic("sfa_decode_d128__intra_B64_ctx8192__hbm_bytes"),
                    "kernels": "decode_partial_d128_kernel<1> + decode_combine_kernel<128>"}

    line = {
        "metric": "stream-factorized attn TFLOP/s (useful) at n=4 + n4/n1 time ratio; decode GB/s",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "intra-stream prefill n=4 L=4096 (nL=16384) B=1 32q/8kv d=128 bf16, "
                               "plus n=1 control, cross layer, B=64 ctx-8192 decode, 4x160000x7168 gather",
                   "n": 4, "seq_len_tokens": 4096, "expanded_len": 16384, "batch": 1,
                   "heads_q": 32, "heads_kv": 8, "head_dim": 128},
        "n4_n1_time_ratio": ratio,
        # forward + backward of the attention layer (the pages compare training
        # step times); 4.0 would be the FLOP ratio
        "n4_n1_train_time_ratio": (round((report["intra_n4"]["ms"] + report["bwd_intra_n4"]["ms"]) /
                                         (report["intra_n1"]["ms"] + report["bwd_intra_n1"]["ms"]), 3)
                                   if all(c in report for c in ("intra_n4", "bwd_intra_n4", "intra_n1",
                                                                "bwd_intra_n1")) else None),
        "decode_GBps": {m: report[m]["GB/s"] for m in ("decode_intra", "decode_cross") if m in report},
        "components": report,
        "step_components": list(step_comps),
        "roofline": roof,
        "roofline_decode": roof_dec,
        "cpu_baseline": None if args.no_cpu else cpu_baseline(args.cpu_seconds),
        "measured_peaks": None if only else measured_peaks(dev),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
