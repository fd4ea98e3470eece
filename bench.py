"""Benchmark of the Stream-Factorized Attention hot path on one MI355X.

One step = one pass over every step of the hot path on synthetic inputs that
are already resident in HBM:
  expand-embed   64 sequences x 1 token x 4 streams from 4 tables 160000 x 7168 bf16
  intra prefill  n=4, L=4096 (nL=16384), 32 q / 8 kv heads, d=128, bf16   <- headline
  intra prefill  n=1, L=4096 control (for the n=4 / n=1 time ratio)
  cross prefill  same shapes as the headline, dense causal over 16384 positions
  decode         64 sequences, 8192 cached tokens x 4 streams, 32 q / 8 kv heads,
                 intra and cross (one new token, 4 stream queries each)
After the timed steps, the extension rows are timed one row at a time, each
with its own warm-up calls (reported under "components", outside ms_per_step):
  gather         the same tables at prefill size: B=1, L=4096, n=4 -> 16384 rows
                 (0.47 GB moved; 64 rotating id sets so rows come from HBM)
  long context   n=4, L=32768 (nL=131072), 16 q / 4 kv heads: intra-stream with
                 a 4096-token window, local cross-stream with a 4096-token window,
                 and a full cross-stream layer
  final-stream   the final stream's queries of the headline shapes (intra and
                 cross) and the backward of the cross one; decode of the final
                 stream's query (intra and cross)
  rotary embed   q and k of the headline layer at the expanded positions, and
                 the prefill with the rotation of q fused in
  backward       dQ, dK, dV of the headline intra-stream layer (given o, lse, dO)
Each call is timed with HIP events on the stream it is launched on.  The
headline value is useful TFLOP/s of the intra-stream prefill (4*d*Hq FLOPs per
visible query/key pair).  Beside the GPU rows: the CPU oracle timed on a
bounded sample of each step row (and of the gather and long-context rows) on
this host's cores, and the machine's measured matrix-core and HBM-read rates.
Prints one JSON line.
"""
import argparse
import ctypes
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np
import torch

from latent_sequence_length_amd import hd, synth

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E (published)
PROBE_SRC = os.path.join(ROOT, "bench_peaks.hip")
PROBE_LIB = os.path.join(ROOT, "bench_peaks.so")


def build_probe(verbose=False):
    """Compile the measured-peak probes (bench_peaks.hip) for gfx950."""
    arch = os.environ.get("HD_OFFLOAD_ARCH", "gfx950")
    cmd = ["hipcc", f"--offload-arch={arch}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", PROBE_SRC, "-o", PROBE_LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PROBE_SRC}:\n{r.stderr}")
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return PROBE_LIB


_ROCTX = None


def _roctx():
    """The ROCm tools-extension library (range markers a profiler's
    --marker-trace records), or False where it is not installed."""
    global _ROCTX
    if _ROCTX is None:
        _ROCTX = False
        for name in ("librocprofiler-sdk-roctx.so.1", "librocprofiler-sdk-roctx.so"):
            try:
                lib = ctypes.CDLL(name)
            except OSError:
                continue
            lib.roctxRangePushA.argtypes = [ctypes.c_char_p]
            lib.roctxRangePushA.restype = ctypes.c_int
            lib.roctxRangePop.argtypes = []
            lib.roctxRangePop.restype = ctypes.c_int
            _ROCTX = lib
            break
    return _ROCTX


def marker_push(text):
    """Open a named range around a timed loop, so that a kernel trace taken
    with markers attributes each dispatch to its bench row (host-side only;
    two calls per timed loop)."""
    lib = _roctx()
    if lib:
        lib.roctxRangePushA(text.encode())


def marker_pop():
    lib = _roctx()
    if lib:
        lib.roctxRangePop()


def _tri(T, w):
    """Sum over q in [0, T) of min(q + 1, w) (w = 0: no window)."""
    if w <= 0 or w >= T:
        return T * (T + 1) // 2
    return w * (w + 1) // 2 + (T - w) * w


def useful_flops(B, L, n, Hq, d, mode, window=0):
    """4*d*Hq*(number of visible (query, key) pairs): QK^T and PV, 2 flops per
    multiply-add.  Intra: per stream, tokens j <= i within the window; cross:
    positions t_k <= t_q within n*window positions."""
    pairs = n * _tri(L, window) if mode == 0 else _tri(n * L, n * window)
    return 4.0 * d * Hq * B * pairs


def useful_flops_final(B, L, n, Hq, d, mode, window=0):
    """Final-stream queries of a KV-mirror layer: query i sees tokens
    j <= i (within the window) of stream n-1 only (intra) or of all n
    streams (cross)."""
    pairs = _tri(L, window) * (n if mode == 1 else 1)
    return 4.0 * d * Hq * B * pairs


def row_visible_keys(t, n, L, mode, window):
    """Visible keys of query position(s) t of a prefill layer (numpy)."""
    if mode == 0:
        i = t // n + 1
        return np.minimum(i, window) if window else i
    return np.minimum(t + 1, n * window) if window else t + 1


def measured_peaks(dev):
    """The machine's sustained rates, reported beside the published peaks:
    an MFMA-only loop (8 independent bf16 32x32x16 chains per wave, 4 waves
    per SIMD) on constant operands and on random operands that change from
    one MFMA to the next (the chip's clock, and so the rate, depends on the
    operands' switching activity), a read-only stream over 8 GiB (16-byte non-temporal loads; the
    HBM ceiling of a read-dominated kernel such as decode) and, for context,
    a 1 GiB device copy (read + write, torch)."""
    out = {}
    if os.path.exists(PROBE_LIB):
        lib = ctypes.CDLL(PROBE_LIB)
        lib.hd_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        lib.hd_probe_mfma_bf16.restype = ctypes.c_double
        lib.hd_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p]
        lib.hd_probe_hbm_read.restype = ctypes.c_double
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        blocks, iters = 4096, 2048
        sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
        lib.hd_probe_mfma_bf16(blocks, iters, ctypes.c_void_p(sink.data_ptr()), st)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fl = sum(lib.hd_probe_mfma_bf16(blocks, iters, ctypes.c_void_p(sink.data_ptr()), st) for _ in range(5))
        e.record()
        torch.cuda.synchronize()
        if fl > 0:
            out["mfma_bf16_TFLOPs"] = round(fl / s.elapsed_time(e) / 1e9, 1)
        if hasattr(lib, "hd_probe_mfma_bf16_random"):
            lib.hd_probe_mfma_bf16_random.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                                      ctypes.c_void_p, ctypes.c_void_p]
            lib.hd_probe_mfma_bf16_random.restype = ctypes.c_double
            g = torch.Generator(device=dev)
            g.manual_seed(7)
            nops = 1 << 20
            ops = torch.randn(nops, 8, generator=g, device=dev).to(torch.bfloat16)
            rargs = (blocks, iters // 8, ctypes.c_void_p(ops.data_ptr()), nops, ctypes.c_void_p(sink.data_ptr()), st)
            lib.hd_probe_mfma_bf16_random(*rargs)
            s.record()
            fl = sum(lib.hd_probe_mfma_bf16_random(*rargs) for _ in range(5))
            e.record()
            torch.cuda.synchronize()
            if fl > 0:
                out["mfma_bf16_random_TFLOPs"] = round(fl / s.elapsed_time(e) / 1e9, 1)
            del ops
        del sink
        nbytes = 8 << 30
        buf = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device=dev)
        rblocks = 256 * 8
        rsink = torch.empty(rblocks * 256, dtype=torch.int32, device=dev)
        args = (ctypes.c_void_p(buf.data_ptr()), nbytes, rblocks, ctypes.c_void_p(rsink.data_ptr()), st)
        lib.hd_probe_hbm_read(*args)
        s.record()
        by = sum(lib.hd_probe_hbm_read(*args) for _ in range(5))
        e.record()
        torch.cuda.synchronize()
        if by > 0:
            out["hbm_read_GBps"] = round(by / s.elapsed_time(e) / 1e6, 1)
        del buf, rsink
    src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(5):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    out["copy_rw_GBps"] = round(5 * 2 * src.numel() * 2 / s.elapsed_time(e) / 1e6, 1)
    return out


def measured_traffic(name):
    """HBM bytes per launch of a kernel from its committed PMC summary
    (profiles/<name>.md: FETCH_SIZE + WRITE_SIZE scaled by a copy kernel), or
    None when the summary is missing or the kernel source has changed since
    the counters were taken (the summary records the sources' SHA-256)."""
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
    # `source` may list several files (a kernel and the code it includes),
    # comma-separated; the digest is taken over their bytes in that order.
    h = hashlib.sha256()
    for part in src.split(","):
        h.update(open(os.path.join(ROOT, part.strip()), "rb").read())
    digest = h.hexdigest()
    if digest != fields.get("source_sha256"):
        return None
    return int(fields["traffic_bytes_per_launch"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--cpu-seconds", type=float, default=24.0, help="CPU-oracle sample budget over all rows")
    ap.add_argument("--no-extra", action="store_true", help="time the step rows only")
    ap.add_argument("--only", default="", help="comma list of components to run (profiling); 'peaks' runs the "
                                               "measured-peak loops alone")
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


# ---------------------------------------------------------------------------
# CPU-oracle baselines: the oracle as it stands, on a bounded sample of each
# row's workload, on the same inputs as the GPU (host copies), extrapolated to
# the whole row by its share of the work.
# ---------------------------------------------------------------------------

def _cores():
    return int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))


def _time_prefill_rows(q, k, v, cfg, budget_s, seed):
    """Distinct random query rows of a prefill layer through the oracle until
    the budget is spent or every row is done; returns (useful flops done,
    seconds, rows)."""
    import oracle

    nL = cfg.n * cfg.L
    total = cfg.B * nL * cfg.Hq
    rng = np.random.default_rng(seed)
    oracle.sfa_rows(q, k, v, cfg.n, cfg.mode, cfg.window, rows=np.array([0], dtype=np.int64))  # load + warm
    order = rng.permutation(total).astype(np.int64)  # distinct rows, in random order
    flops, rows_done, batch = 0.0, 0, 32
    t0 = time.perf_counter()
    while rows_done < total:
        rows = order[rows_done:rows_done + batch]
        oracle.sfa_rows(q, k, v, cfg.n, cfg.mode, cfg.window, rows=rows)
        t = (rows // cfg.Hq) % nL
        flops += float(4 * cfg.d * row_visible_keys(t, cfg.n, cfg.L, cfg.mode, cfg.window).sum())
        rows_done += rows.size
        spent = time.perf_counter() - t0
        if spent >= budget_s * 0.95:
            break
        # size the next batch to the time that is left, from the rate so far
        batch = int(min(8192, max(16, (budget_s - spent) * rows_done / spent)))
    return flops, time.perf_counter() - t0, rows_done


def cpu_prefill(cfg, budget_s, seed, gpu_inputs=None):
    """CPU-oracle rate on one prefill layer (inputs: host copies of the GPU's)."""
    if gpu_inputs is not None:
        q, k, v = (t.cpu() for t in gpu_inputs)
    else:
        q, k, v = synth.qkv(cfg.B, cfg.L, cfg.n, cfg.Hq, cfg.Hkv, cfg.d, cfg.dtype, "cuda")
        q, k, v = q.cpu(), k.cpu(), v.cpu()
    fl, dt, rows = _time_prefill_rows(q, k, v, cfg, budget_s, seed)
    total_fl = useful_flops(cfg.B, cfg.L, cfg.n, cfg.Hq, cfg.d, cfg.mode, cfg.window)
    rate = fl / dt
    nrows = cfg.B * cfg.n * cfg.L * cfg.Hq
    return {"value": rate / 1e12, "unit": "TFLOP/s", "ms_extrapolated": round(total_fl / rate * 1e3, 1),
            "extrapolated": True,
            "sample": f"{rows} random query rows of {nrows} ({rows / nrows:.2%}), {dt:.1f} s"}


def cpu_decode(dq, dkn, dvn, dkc, dvc, ctx, mode, nseq, by_total):
    """CPU-oracle rate on the decode step, on the first nseq of its sequences
    (each sequence is an independent step); GB/s counts the same bytes per
    sequence as the GPU row."""
    import oracle

    B = dq.shape[0]
    q, kn, vn = dq[:nseq].cpu(), dkn[:nseq].cpu(), dvn[:nseq].cpu()
    kc, vc = dkc[:nseq, :ctx + 1].cpu().contiguous(), dvc[:nseq, :ctx + 1].cpu().contiguous()
    lens = [ctx] * nseq
    t0 = time.perf_counter()
    oracle.sfa_decode(q, kn, vn, kc, vc, lens, mode)
    dt = time.perf_counter() - t0
    ms_full = dt * B / nseq * 1e3
    return {"value": round(by_total * nseq / B / dt / 1e9, 3), "unit": "GB/s", "ms_extrapolated": round(ms_full, 1),
            "extrapolated": True, "sample": f"{nseq} of {B} sequences (whole steps), {dt:.1f} s"}


def cpu_gather(tabs_host, idsets, reps):
    """CPU-oracle rate on the expansion gather: the oracle's row copies from
    host copies of the same tables, over `reps` of the rotating id sets."""
    import oracle

    ids_host = [ids.cpu().numpy() for ids in idsets[:reps]]
    oracle.expand_embed(ids_host[0], tabs_host)
    t0 = time.perf_counter()
    nbytes = 0
    for ids in ids_host:
        out = oracle.expand_embed(ids, tabs_host)
        nbytes += 2 * out.nbytes + ids.nbytes
    dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s",
            "ms_extrapolated": round(dt / len(ids_host) * 1e3, 2), "extrapolated": False,
            "sample": f"{len(ids_host)} whole calls (rotating id sets), {dt:.2f} s"}


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
    EP = synth.EMBED_PREFILL
    extra_on = not args.no_extra

    comps = {}    # name -> (callable, useful flops, algorithmic bytes)
    inputs = {}   # name -> GPU inputs the CPU baseline copies

    def prefill(cfg, name):
        """(callable, useful flops, algorithmic bytes) of one prefill call on
        inputs drawn once; bytes = q, k, v read + o written."""
        q, k, v = synth.qkv(cfg.B, cfg.L, cfg.n, cfg.Hq, cfg.Hkv, cfg.d, cfg.dtype, dev)
        inputs[name] = (q, k, v)
        o = torch.empty_like(q)
        fl = useful_flops(cfg.B, cfg.L, cfg.n, cfg.Hq, cfg.d, cfg.mode, cfg.window)
        by = 2 * (2 * q.numel() + k.numel() + v.numel())
        return (lambda: hd.hd_sfa_fwd(q, k, v, o, cfg.n, cfg.mode, cfg.window), fl, by)

    if want("intra_n4"):
        comps["intra_n4"] = prefill(I, "intra_n4")
    if want("intra_n1"):
        comps["intra_n1"] = prefill(I1, "intra_n1")
    if want("cross_n4"):
        comps["cross_n4"] = prefill(X, "cross_n4")
    dec = None
    if any(want(n) for n in ("decode_intra", "decode_cross", "decode_final_intra", "decode_final_cross")):
        T_cap = Dc.ctx + 8
        dq, dkn, dvn, dkc, dvc = synth.decode_inputs(Dc.B, Dc.n, Dc.Hq, Dc.Hkv, Dc.d, T_cap, Dc.dtype, dev)
        dec = (dq, dkn, dvn, dkc, dvc)
        dcl = torch.full((Dc.B,), Dc.ctx, dtype=torch.int32, device=dev)
        do = torch.empty_like(dq)
        ws = torch.empty(hd.hd_sfa_decode_workspace_bytes(Dc.B, Dc.n, Dc.Hq, Dc.Hkv, Dc.d, T_cap),
                         dtype=torch.uint8, device=dev)
        # algorithmic bytes: cache read for ctx+1 tokens (the new row from
        # k_new/v_new), q read, o written, new rows written to the cache
        tok_bytes = Dc.n * Dc.Hkv * Dc.d * 2
        dec_by = 2 * (Dc.ctx * tok_bytes * Dc.B) + 2 * dq.numel() * 2 + 2 * dkn.numel() * 2 * 2
        for mode, name in ((0, "decode_intra"), (1, "decode_cross")):
            if want(name):
                if mode == 0:
                    pairs = Dc.B * Dc.n * Dc.Hq * (Dc.ctx + 1)
                else:
                    pairs = Dc.B * Dc.Hq * sum(Dc.ctx * Dc.n + s + 1 for s in range(Dc.n))
                comps[name] = (lambda mode=mode: hd.hd_sfa_decode(dq, dkn, dvn, dkc, dvc, dcl, do, mode, 0, 0.0, ws),
                               4.0 * Dc.d * pairs, dec_by)
        # KV-mirror layers: the final stream's query only (intra reads stream
        # n-1's cache rows alone, cross the whole cache)
        dqf = dq[:, Dc.n - 1:Dc.n].contiguous()
        dof = torch.empty_like(dqf)
        for mode, name in ((0, "decode_final_intra"), (1, "decode_final_cross")):
            if want(name) and (extra_on or only):
                rows = Dc.ctx if mode == 0 else Dc.ctx * Dc.n
                by_f = 2 * rows * Dc.Hkv * Dc.d * 2 * Dc.B + 2 * 2 * dqf.numel() + 2 * dkn.numel() * 2 * 2
                pairs = Dc.B * Dc.Hq * ((Dc.ctx + 1) if mode == 0 else (Dc.ctx + 1) * Dc.n)
                comps[name] = (lambda mode=mode: hd.hd_sfa_decode(dqf, dkn, dvn, dkc, dvc, dcl, dof, mode, 0, 0.0, ws,
                                                                  final_only=True), 4.0 * Dc.d * pairs, by_f)
    tabs = None
    if want("embed") or want("embed_prefill"):
        tabs = synth.tables(E["n"], E["V"], E["D"], E["dtype"], dev)
    if want("embed"):
        # 64 rotating id sets so rows come from HBM rather than the last-level cache
        idsets = [synth.token_ids(E["B"], E["L"], E["V"], seed=1000 + r, device=dev) for r in range(64)]
        inputs["embed"] = idsets
        eo = torch.empty((E["B"], E["n"] * E["L"], E["D"]), dtype=E["dtype"], device=dev)
        ctr = [0]

        def run_embed():
            hd.hd_expand_embed(idsets[ctr[0] % 64], tabs, eo)
            ctr[0] += 1

        comps["embed"] = (run_embed, 0.0, 2 * eo.numel() * 2 + E["B"] * E["L"] * 4)
    if want("embed_prefill") and (extra_on or only):
        idsets_p = [synth.token_ids(EP["B"], EP["L"], EP["V"], seed=2000 + r, device=dev) for r in range(64)]
        inputs["embed_prefill"] = idsets_p
        epo = torch.empty((EP["B"], EP["n"] * EP["L"], EP["D"]), dtype=EP["dtype"], device=dev)
        ctrp = [0]

        def run_embed_prefill():
            hd.hd_expand_embed(idsets_p[ctrp[0] % 64], tabs, epo)
            ctrp[0] += 1

        comps["embed_prefill"] = (run_embed_prefill, 0.0, 2 * epo.numel() * 2 + EP["B"] * EP["L"] * 4)

    if extra_on or only:
        for cfg, name in ((synth.LONG_INTRA_W, "long_intra_w4096"), (synth.LONG_CROSS_W, "long_cross_w4096"),
                          (synth.LONG_CROSS, "long_cross")):
            if want(name):
                comps[name] = prefill(cfg, name)

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
            comps["rope_fwd_intra_n4"] = (lambda q=q, k=k, v=v, o=o, kr=k_rot:
                                          hd.hd_sfa_fwd_rope(q, k, v, o, kr, I.n, I.mode), fl, by)
        if want("intra_n4_const_inputs"):
            # the headline layer on constant inputs (every element 0.25): the
            # same instructions and memory traffic as intra_n4, so the rate
            # difference is what the operands' switching costs in power and
            # clock.  Reported beside the headline, never as it.
            q, k, v = (torch.full((I.B, I.n * I.L, hh, I.d), 0.25, dtype=I.dtype, device=dev)
                       for hh in (I.Hq, I.Hkv, I.Hkv))
            o = torch.empty_like(q)
            fl = useful_flops(I.B, I.L, I.n, I.Hq, I.d, I.mode, I.window)
            by = 2 * (2 * q.numel() + k.numel() + v.numel())
            comps["intra_n4_const_inputs"] = (lambda q=q, k=k, v=v, o=o: hd.hd_sfa_fwd(q, k, v, o, I.n, I.mode,
                                                                                        I.window), fl, by)
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
    # rows are timed after the step, one row at a time, so they neither
    # lengthen nor heat the timed step.
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
        marker_push("timed:" + ",".join(group))
        s_ev.record()
        for _ in range(steps):
            for name, (fn, _, _) in group.items():
                tm.run(name, fn)
        e_ev.record()
        marker_pop()
        tm.collect()
        return s_ev.elapsed_time(e_ev)

    timer = Timer()
    total_ms = timed_loop(step_comps, args.steps, args.warmup, timer)
    ms_per_step = total_ms / max(args.steps, 1)
    if extra_comps:
        # each extension row on its own, back to back: its calls see only its
        # own cache state, not the write-back of another row's outputs
        for name, entry in extra_comps.items():
            extra_timer = Timer()
            timed_loop({name: entry}, args.steps, args.warmup, extra_timer)
            timer.ms.update(extra_timer.ms)

    report = {}
    for name, (fn, fl, by) in comps.items():
        t = float(np.mean(timer.ms[name]))
        report[name] = {"ms": round(t, 4), "ms_min": round(float(np.min(timer.ms[name])), 4),
                        "ms_median": round(float(np.median(timer.ms[name])), 4)}
        if fl:
            report[name]["TFLOP/s"] = round(fl / t / 1e9, 2)
        report[name]["GB/s"] = round(by / t / 1e6, 1)

    peaks = None if only else measured_peaks(dev)

    def frac_measured(ach, key):
        return round(ach / peaks[key], 4) if peaks and peaks.get(key) else None

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
                "kernel": "sfa_fwd_bf16_d128_kernel", "per_launch_flops": fl,
                "peak_measured": peaks.get("mfma_bf16_TFLOPs") if peaks else None,
                "frac_measured": frac_measured(ach, "mfma_bf16_TFLOPs"),
                "peak_measured_random": peaks.get("mfma_bf16_random_TFLOPs") if peaks else None,
                "frac_measured_random": frac_measured(ach, "mfma_bf16_random_TFLOPs")}

    def hbm_roof(name, kernels, traffic_profile):
        if name not in report:
            return None
        by = comps[name][2]
        ach = by / report[name]["ms"] / 1e6
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBPS, 4), "per_launch_bytes": by,
                "traffic": measured_traffic(traffic_profile), "kernels": kernels,
                "peak_measured": peaks.get("hbm_read_GBps") if peaks else None,
                "frac_measured": frac_measured(ach, "hbm_read_GBps")}

    roof_dec = hbm_roof("decode_intra", "decode_partial_d128_kernel<1> + decode_combine_kernel<128>",
                        "sfa_decode_d128__intra_B64_ctx8192__hbm_bytes")
    roof_emb = hbm_roof("embed_prefill", "expand_embed_rows", "expand_embed__prefill_16384_rows__hbm_bytes")

    cpu = None
    cpu_rows = None
    if not args.no_cpu and not only:
        budget = args.cpu_seconds
        cpu_rows = {}
        share = {"intra_n4": 0.2, "intra_n1": 0.12, "cross_n4": 0.16, "long_intra_w4096": 0.12,
                 "long_cross": 0.12}
        for name, cfg in (("intra_n4", I), ("intra_n1", I1), ("cross_n4", X),
                          ("long_intra_w4096", synth.LONG_INTRA_W), ("long_cross", synth.LONG_CROSS)):
            if name in inputs:
                cpu_rows[name] = cpu_prefill(cfg, budget * share[name], seed=123, gpu_inputs=inputs[name])
        if dec is not None:
            for mode, name in ((0, "decode_intra"), (1, "decode_cross")):
                cpu_rows[name] = cpu_decode(*dec, Dc.ctx, mode, 8 if mode == 0 else 4, comps[name][2])
        if tabs is not None and ("embed" in inputs or "embed_prefill" in inputs):
            tabs_host = [t.cpu() for t in tabs]
            if "embed" in inputs:
                cpu_rows["embed"] = cpu_gather(tabs_host, inputs["embed"], 64)
            if "embed_prefill" in inputs:
                cpu_rows["embed_prefill"] = cpu_gather(tabs_host, inputs["embed_prefill"], 4)
            del tabs_host
        for name, row in cpu_rows.items():
            row["cores"] = _cores()
            if name in report:
                row["gpu_speedup"] = round(row["ms_extrapolated"] / report[name]["ms"], 1)
        head = cpu_rows.get("intra_n4")
        if head is not None:
            cpu = {"value": head["value"], "unit": head["unit"], "cores": _cores(), "kind": "oracle",
                   "sample": head["sample"] + " of the n=4 L=4096 intra-stream prefill, double-precision C oracle, "
                             "rate extrapolated to the whole layer"}

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
        # the layers' useful-FLOP ratio beside it: a time ratio below it means
        # the n=1 control runs less efficiently (512 items on 256 CUs: two
        # per CU, balanced less finely than the n=4 layer's eight), not that
        # the n=4 layer beats linear cost
        "n4_n1_flop_ratio": (round(comps["intra_n4"][1] / comps["intra_n1"][1], 3)
                             if "intra_n4" in comps and "intra_n1" in comps else None),
        "n4_n1_note": ("time ratio below the useful-FLOP ratio: the n=1 control runs at a lower TFLOP/s "
                       "(components intra_n1 vs intra_n4), not a sub-linear n=4 layer"),
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
        "roofline_embed": roof_emb,
        "cpu_baseline": cpu,
        "cpu_baseline_rows": cpu_rows,
        "cpu_n4_n1_time_ratio": (round(cpu_rows["intra_n4"]["ms_extrapolated"] /
                                       cpu_rows["intra_n1"]["ms_extrapolated"], 3)
                                 if cpu_rows and "intra_n4" in cpu_rows and "intra_n1" in cpu_rows else None),
        "measured_peaks": peaks,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
