"""Writes sfa_fwd_d128_loop.inc: the key-tile loop of the head-dim-128 prefill
kernel as one hand-scheduled gfx950 instruction stream.

The loop is software-pipelined over 32-key sub-tiles i = 0, 1, ...:
iteration i runs the QK^T MFMAs of sub-tile i, the softmax of sub-tile i-1
(vector ALU) and the PV MFMAs of sub-tile i-2, with the softmax instructions
placed one by one between the MFMAs (a cost-aware list schedule, each op at
least one MFMA after its inputs), so that the vector ALU and the matrix core
of a SIMD work at the same time within one wave.  Operands are read from LDS
two MFMAs ahead into small register rings.  64-key K and V tiles are copied
direct to LDS into three-deep rings (K of tile T+2 and V of tile T+1 are
copied while tile T is computed), one barrier per tile, so the first operand
reads of the next tile can be issued before its barrier.

The softmax uses only instructions that issue beside the MFMAs: v_fma_f32,
v_exp_f32, v_cvt_pk_bf16_f32 and v_add_f32 (the row sum adds the fp32
probabilities; the packed bf16 dot instruction stalls the matrix core).  A
sub-tile's probabilities are taken against the running maximum as it stands;
when some row has no maximum yet or a lane's share of its row sum exceeds
2^32, an out-of-line path takes the tile maximum, rescales O and l and
recomputes them.  Band masks (diagonal, sequence end, window start) are
applied to a sub-tile's scores before its softmax, on the sub-tiles that
need them only.  Every hazard the hardware does not check is padded here:
MFMA results are read by vector ops at least eight MFMAs later (or after
s_nop), a transcendental result is not read by the next instruction, VCC
written by a compare is read after s_nop 4.

Run `python gen_fwd_d128_loop.py` after editing; the output is committed.
Register map (per lane):
  v[0:63]    O^T accumulators, dims 32*db .. +31 in v[16db : 16db+15]
  v[64:95]   Q^T operand of k-step ks in v[64+4ks : 67+4ks]
  v96, v97   running max (log2 units) and row sum of this lane's query
  v98, v99   mask: 4*hi - lo and span (key k visible <=> k - lo <= span, unsigned)
  v[100:107] LDS byte address of the K operand of k-step ks (K ring buffer 0, keys 0-31)
  v[108:115] LDS byte address of the V^T half-operand (db, jh) (V ring buffer 0, keys 0-15)
  v[116:119] copy offsets of this lane: K slot 0, K slot 1, V slot 0, V slot 1
  v[120:123] the same for a tile with rows past the end of the sub-sequence
  v[128:159] score accumulators of two sub-tiles (S^T blocks): lane l holds
             query l % 32, register r key 8(r/4) + 4(l/32) + r%4 of the sub-tile
  v[160:175] bf16 probabilities of two sub-tiles
  v[176:191] K operand ring, v[192:207] V^T operand ring
  v[208:213], v[214:219] fma and exp result rings
  v220 row sum of the sub-tile, v221 -max (0 while no max), v222..v224 temps,
  v225, v226 partial row sums, v229 -inf, v230 2^32
Scalar registers s80..s93 are the loop's; the caller passes the rest as operands.
"""
import os

KT_BYTES = 16384          # one 64-key tile of K or V in LDS
V_RING = 3 * KT_BYTES     # V ring starts after the K ring
LOOK = 2                  # LDS operand reads run this many MFMAs ahead
RING = 4                  # operand ring entries
COST = {"fma": 5, "exp": 12, "cvt": 5}  # vector cycles of one wave64 op (measured)
BUDGET = 26               # vector-ALU cycles placed after one MFMA

S_BASE = (128, 144)
P_BASE = (160, 168)
F_RING, E_RING = 208, 214
SGPR = dict(T="s80", j="s81", kt="s82", kdlo="s84", kdhi="s85", vdlo="s86", vdhi="s87",
            tk="s88", tv="s89", m="s[90:91]")


def vr(b, n):
    return f"v[{b}:{b + n - 1}]"


def slot_list(qk, pv):
    """MFMA slots of one iteration: ('qk', ks) x 8 then ('pv', m2, db) x 8.  An
    iteration without QK (the drain) has 'ghost' slots instead: the first LOOK
    of them take the K reads the previous tile issued ahead (unused)."""
    a = [("qk", ks) for ks in range(8)] if qk else [("ghost", ks) for ks in range(8)]
    b = [("pv", m2, db) for m2 in range(2) for db in range(4)] if pv else []
    return a + b


def has_reads(slot):
    return slot[0] != "ghost" or slot[1] < LOOK


def read_texts(slot, kbuf, vbuf, u):
    if slot[0] in ("qk", "ghost"):
        ks = slot[1]
        return "k", [f"ds_read_b128 {{dst}}, v{100 + ks} offset:{kbuf * KT_BYTES + u * 8192}"]
    m2, db = slot[1], slot[2]
    off = vbuf * KT_BYTES + u * 8192 + m2 * 4096
    return "v", [f"ds_read_b64_tr_b16 {{dlo}}, v{108 + db * 2} offset:{off}",
                 f"ds_read_b64_tr_b16 {{dhi}}, v{108 + db * 2 + 1} offset:{off}"]


def softmax_ops(sbuf, pbuf):
    """Vector ops of the softmax of one sub-tile: [kind, text, deps, ring reuse].
    Row sum: v_add_f32 of the fp32 probabilities into two partial sums."""
    ops = []
    fid, eid, cid, aid = {}, {}, {}, {}
    prev_add = {0: None, 1: None}
    for r in range(16):
        fid[r] = len(ops)
        ops.append(["fma", f"v_fma_f32 v{F_RING + r % 6}, v{sbuf + r}, %[sc], v221", [], []])
        eid[r] = len(ops)
        ops.append(["exp", f"v_exp_f32 v{E_RING + r % 6}, v{F_RING + r % 6}", [fid[r]], []])
        aid[r] = len(ops)
        part = 225 + (r % 2)
        if r < 2:
            ops.append(["fma", f"v_mov_b32 v{part}, v{E_RING + r % 6}", [eid[r]], []])
        else:
            ops.append(["fma", f"v_add_f32 v{part}, v{part}, v{E_RING + r % 6}", [eid[r], prev_add[r % 2]], []])
        prev_add[r % 2] = aid[r]
        if r % 2 == 1:
            k = r // 2
            cid[k] = len(ops)
            ops.append(["cvt", f"v_cvt_pk_bf16_f32 v{pbuf + k}, v{E_RING + (r - 1) % 6}, v{E_RING + r % 6}",
                        [eid[r - 1], eid[r]], []])
    ops.append(["fma", "v_add_f32 v220, v225, v226", [prev_add[0], prev_add[1]], []])
    for r in range(6, 16):
        ops[fid[r]][3].append(eid[r - 6])
        ops[eid[r]][3].append(cid[(r - 6) // 2])
        ops[eid[r]][3].append(aid[r - 6])
    return ops


def schedule(ops, nslots, budget=BUDGET):
    """Cost-aware list schedule of ops into nslots slots (a dependence must
    come from an earlier slot; a ring entry is rewritten only after its reader
    is placed).  Whatever does not fit goes to the last slot."""
    where, per = {}, [[] for _ in range(nslots)]
    pending = list(range(len(ops)))
    s = 0
    while pending:
        used, progress = 0, True
        last = s >= nslots - 1
        while progress:
            progress = False
            for o in pending:
                kind, txt, deps, war = ops[o]
                if used + COST[kind] > budget and not last:
                    continue
                ok_dep = all(d in where and (where[d] < s or (last and where[d] <= s)) for d in deps)
                if ok_dep and all(d in where for d in war):
                    where[o] = s
                    per[min(s, nslots - 1)].append(txt)
                    used += COST[kind]
                    pending.remove(o)
                    progress = True
                    break
        s += 1
        if s > 4 * nslots:
            raise RuntimeError("cannot schedule")
    return per


class Gen:
    def __init__(self):
        self.L = []
        self.ring_k = 0   # next K ring entry
        self.ring_v = 0
        self.fifo = []
        self.label_n = 0
        self.slow_blocks = []

    def a(self, s):
        self.L.append(s)

    def label(self, base):
        self.label_n += 1
        return f".Lhd{base}_{self.label_n}_%="

    # ---- LDS read stream -------------------------------------------------
    # fifo: reads issued for slots not yet executed, in order: (n_reads, target)
    def issue_reads(self, slot, kbuf, vbuf, u):
        kind, texts = read_texts(slot, kbuf, vbuf, u)
        if kind == "k":
            b = 176 + 4 * self.ring_k
            self.ring_k = (self.ring_k + 1) % RING
            self.a(texts[0].format(dst=vr(b, 4)))
            self.fifo.append((1, vr(b, 4)))
        else:
            b = 192 + 4 * self.ring_v
            self.ring_v = (self.ring_v + 1) % RING
            self.a(texts[0].format(dlo=vr(b, 2)))
            self.a(texts[1].format(dhi=vr(b + 2, 2)))
            self.fifo.append((2, vr(b, 4)))

    def take(self, wait=True):
        n, target = self.fifo.pop(0)
        if wait:
            later = sum(x[0] for x in self.fifo)
            self.a(f"s_waitcnt lgkmcnt({min(later, 15)})")
        return target

    # ---- pieces ------------------------------------------------------------
    def mask_block(self, sb):
        """Scores of the sub-tile at key %[kt] outside the lane's band -> -inf."""
        skip, do = self.label("nomask"), self.label("mask")
        self.a(f"s_cmp_lt_u32 {SGPR['j']}, %[jw]")
        self.a(f"s_cbranch_scc1 {do}")
        self.a(f"s_cmp_ge_u32 {SGPR['j']}, %[jm]")
        self.a(f"s_cbranch_scc0 {skip}")
        self.a(f"{do}:")
        self.a(f"v_add_u32 v222, {SGPR['kt']}, v98")
        for r in range(16):
            c = 8 * (r >> 2) + (r & 3)
            self.a(f"v_add_u32 v223, {c}, v222")
            self.a("v_cmp_le_u32 vcc, v223, v99")
            self.a("s_nop 4")
            self.a(f"v_cndmask_b32 v{sb + r}, v229, v{sb + r}, vcc")
        self.a(f"{skip}:")

    def slow_path(self, sb, pb, back):
        """The tile max, O and l rescale and the probabilities again (rare)."""
        lab = self.label("slow")
        body = [f"{lab}:", "s_nop 7", "s_nop 7", "s_nop 7"]
        body.append(f"v_max3_f32 v222, v{sb}, v{sb + 1}, v{sb + 2}")
        for r in range(3, 16, 2):
            if r + 1 < 16:
                body.append(f"v_max3_f32 v222, v222, v{sb + r}, v{sb + r + 1}")
            else:
                body.append(f"v_max_f32 v222, v222, v{sb + r}")
        body += ["v_mov_b32 v223, v222", "s_nop 1", "v_permlane32_swap_b32 v222, v223", "s_nop 1",
                 "v_max_f32 v222, v222, v223",
                 "v_mul_f32 v222, %[sc], v222",        # tile max in log2 units
                 "v_max_f32 v223, v96, v222",          # new max
                 "v_sub_f32 v224, v96, v223",
                 "v_exp_f32 v224, v224",
                 "v_cmp_eq_f32 vcc, v96, v223",
                 "s_nop 4",
                 "v_cndmask_b32_e64 v224, v224, 1.0, vcc"]  # alpha
        body += [f"v_mul_f32 v{r}, v{r}, v224" for r in range(64)]
        body += ["v_mul_f32 v97, v97, v224", "v_mov_b32 v96, v223",
                 "v_sub_f32 v221, 0, v223",
                 "v_cmp_eq_f32 vcc, v229, v223",
                 "s_nop 4",
                 "v_cndmask_b32_e64 v221, v221, 0, vcc"]
        # probabilities of the sub-tile against the new max, in program order
        for r in range(16):
            body.append(f"v_fma_f32 v{F_RING + r % 6}, v{sb + r}, %[sc], v221")
            body.append("s_nop 0")
            body.append(f"v_exp_f32 v{E_RING + r % 6}, v{F_RING + r % 6}")
            body.append("s_nop 0")
            if r == 0:
                body.append(f"v_mov_b32 v220, v{E_RING}")
            else:
                body.append(f"v_add_f32 v220, v220, v{E_RING + r % 6}")
            if r % 2 == 1:
                k = r // 2
                body.append(f"v_cvt_pk_bf16_f32 v{pb + k}, v{E_RING + (r - 1) % 6}, v{E_RING + r % 6}")
        body.append("s_nop 4")
        body.append(f"s_branch {back}")
        self.slow_blocks.append(body)
        return lab

    def check(self, sb, pb):
        """Keep the fast probabilities unless some row has no max yet or a
        lane's share of its row sum exceeds 2^32 (or is not a number)."""
        back = self.label("back")
        slow = self.slow_path(sb, pb, back)
        self.a("v_cmp_nge_f32 vcc, v230, v220")
        self.a(f"v_cmp_eq_f32_e64 {SGPR['m']}, v229, v96")
        self.a("s_nop 4")
        self.a(f"s_or_b64 vcc, vcc, {SGPR['m']}")
        self.a("s_and_b64 vcc, vcc, exec")
        self.a(f"s_cbranch_vccnz {slow}")
        self.a(f"{back}:")
        self.a("v_add_f32 v97, v97, v220")

    def iteration(self, u, kbuf, vbuf, qk, sm, pv, nxt, pre_nops=False):
        """One sub-tile iteration i with u = i % 2: QK writes S[u], the softmax
        reads S[1-u] and writes P[1-u], PV reads P[u].  nxt = (kbuf, vbuf, u, qk, pv)
        of the iteration that follows (its first slots' reads are issued here)."""
        sq, ss = S_BASE[u], S_BASE[1 - u]
        ps, pp = P_BASE[1 - u], P_BASE[u]
        slots = slot_list(qk, pv)
        nslots = slot_list(nxt[3], nxt[4])
        stream = [(s, kbuf, vbuf, u) for s in slots] + [(s, nxt[0], nxt[1], nxt[2]) for s in nslots]
        if pre_nops:
            self.a("s_nop 7")
            self.a("s_nop 7")
            self.a("s_nop 7")
        if sm:
            self.mask_block(ss)
        per = schedule(softmax_ops(ss, ps), len(slots)) if sm else [[] for _ in slots]
        first_pv = True
        for n, slot in enumerate(slots):
            target = None
            if has_reads(slot):
                target = self.take(wait=slot[0] != "ghost")
            if slot[0] == "qk":
                ks = slot[1]
                src_c = "0" if ks == 0 else vr(sq, 16)
                self.a(f"v_mfma_f32_32x32x16_bf16 {vr(sq, 16)}, {target}, {vr(64 + 4 * ks, 4)}, {src_c}")
            elif slot[0] == "pv":
                m2, db = slot[1], slot[2]
                if first_pv and not qk:
                    self.a("s_nop 2")
                first_pv = False
                self.a(f"v_mfma_f32_32x32x16_bf16 {vr(16 * db, 16)}, {target}, {vr(pp + 4 * m2, 4)}, {vr(16 * db, 16)}")
            ahead = n + LOOK
            if ahead < len(stream):
                s2, kb2, vb2, u2 = stream[ahead]
                if has_reads(s2):
                    self.issue_reads(s2, kb2, vb2, u2)
            for t in per[n]:
                self.a(t)
        if sm:
            self.check(ss, ps)
            self.a(f"s_add_u32 {SGPR['j']}, {SGPR['j']}, 1")
            self.a(f"s_add_u32 {SGPR['kt']}, {SGPR['kt']}, 32")


def generate():
    g = Gen()
    a = g.a
    # ---- set-up ---------------------------------------------------------------
    a("v_mov_b32 v229, 0xff800000")
    a("v_mov_b32 v230, 0x4f800000")
    a("v_mov_b32 v221, 0")
    a(f"s_mov_b32 {SGPR['T']}, 0")
    a(f"s_mov_b32 {SGPR['j']}, 0")
    a(f"s_mov_b32 {SGPR['kt']}, %[kt0]")
    a(f"s_mov_b64 s[{SGPR['kdlo'][1:]}:{SGPR['kdhi'][1:]}], %[kptr2]")
    a(f"s_mov_b64 s[{SGPR['vdlo'][1:]}:{SGPR['vdhi'][1:]}], %[vptr1]")

    def dma(kind, buf, tail_idx_sgpr):
        """Copy the tile at the running pointer into ring buffer `buf`, then
        advance the pointer.  kind 'k' or 'v'."""
        lo, hi = (SGPR['kdlo'], SGPR['kdhi']) if kind == "k" else (SGPR['vdlo'], SGPR['vdhi'])
        ring = 0 if kind == "k" else V_RING
        offs = (116, 117) if kind == "k" else (118, 119)
        toffs = (120, 121) if kind == "k" else (122, 123)
        normal, done = g.label("dman"), g.label("dmad")
        a(f"s_cmp_eq_u32 {tail_idx_sgpr}, %[tailt]")
        a(f"s_cbranch_scc0 {normal}")
        for i in range(2):
            a(f"s_add_u32 m0, %[ldsw], {ring + buf * KT_BYTES + i * 1024}")
            a("s_nop 0")
            a(f"global_load_lds_dwordx4 v{toffs[i]}, s[{lo[1:]}:{hi[1:]}]")
        a(f"s_branch {done}")
        a(f"{normal}:")
        for i in range(2):
            a(f"s_add_u32 m0, %[ldsw], {ring + buf * KT_BYTES + i * 1024}")
            a("s_nop 0")
            a(f"global_load_lds_dwordx4 v{offs[i]}, s[{lo[1:]}:{hi[1:]}]")
        a(f"{done}:")
        a(f"s_add_u32 {lo}, {lo}, %[tbytes]")
        a(f"s_addc_u32 {hi}, {hi}, 0")

    # The caller has issued the copies of K(0), K(1) (if any) and V(0) and
    # passes the pointers of the next tiles to copy: K(2) and V(1).
    a(f"s_mov_b32 {SGPR['tk']}, 2")
    a(f"s_mov_b32 {SGPR['tv']}, 1")

    def header(p, first=False):
        """Start of tile T (T % 3 == p): wait for the copies issued one tile
        ago, barrier, copy K(T+2) and V(T+1)."""
        nahead = sum(x[0] for x in g.fifo)
        a("s_waitcnt vmcnt(0)")
        a(f"s_waitcnt lgkmcnt({min(nahead, 15)})")
        a("s_barrier")
        nk, nv = g.label("nok"), g.label("nov")
        a(f"s_cmp_lt_u32 {SGPR['tk']}, %[nt]")
        a(f"s_cbranch_scc0 {nk}")
        dma("k", (p + 2) % 3, SGPR['tk'])
        a(f"{nk}:")
        a(f"s_add_u32 {SGPR['tk']}, {SGPR['tk']}, 1")
        a(f"s_cmp_lt_u32 {SGPR['tv']}, %[nt]")
        a(f"s_cbranch_scc0 {nv}")
        dma("v", (p + 1) % 3, SGPR['tv'])
        a(f"{nv}:")
        a(f"s_add_u32 {SGPR['tv']}, {SGPR['tv']}, 1")

    def run_iter(kbuf, vbuf, u, qk, sm, pv, nxt, pre_nops=False):
        g.iteration(u, kbuf, vbuf, qk, sm, pv, nxt, pre_nops=pre_nops)

    def start_reads(kbuf, vbuf, u, qk, pv):
        for s in slot_list(qk, pv)[:LOOK]:
            g.issue_reads(s, kbuf, vbuf, u)

    # The stream of tiles: tile 0 (prologue iterations), then tiles T >= 1
    # with parity T % 3, then the drain after the last tile.  Every tile ends
    # with the reads of the next tile's first QK operands issued (for the drain
    # they read a K buffer nobody uses: harmless).
    drain_labels = {p: g.label(f"drain{p}") for p in range(3)}
    tile_labels = {p: g.label(f"tile{p}") for p in range(3)}

    # tile 0
    header(0, first=True)
    start_reads(0, 0, 0, True, False)
    run_iter(0, 0, 0, True, False, False, (0, 0, 1, True, False))            # i = 0: QK(0)
    run_iter(0, 0, 1, True, True, False, (1, 0, 0, True, True), pre_nops=True)  # i = 1: QK(1), softmax(0)
    # iteration 1 has no PV MFMAs after its QK MFMAs: let them finish before
    # the next softmax reads their scores
    a("s_nop 7")
    a("s_nop 7")
    a("s_nop 7")
    a(f"s_add_u32 {SGPR['T']}, {SGPR['T']}, 1")
    a(f"s_cmp_eq_u32 {SGPR['T']}, %[nt]")
    a(f"s_cbranch_scc1 {drain_labels[0]}")
    # steady tiles, parity 1, 2, 0, 1, ...
    for p in (1, 2, 0):
        a(f"{tile_labels[p]}:")
        header(p)
        kb, vb = p, (p - 1) % 3
        run_iter(kb, vb, 0, True, True, True, (kb, vb, 1, True, True))
        run_iter(kb, vb, 1, True, True, True, ((p + 1) % 3, p, 0, True, True))
        a(f"s_add_u32 {SGPR['T']}, {SGPR['T']}, 1")
        a(f"s_cmp_eq_u32 {SGPR['T']}, %[nt]")
        a(f"s_cbranch_scc1 {drain_labels[p]}")
        a(f"s_branch {tile_labels[(p + 1) % 3]}")
    end = g.label("end")
    # drains: the last tile had parity p; its V is in V buffer p
    saved = (list(g.fifo), g.ring_k, g.ring_v)
    for p in range(3):
        g.fifo, g.ring_k, g.ring_v = list(saved[0]), saved[1], saved[2]
        a(f"{drain_labels[p]}:")
        run_iter((p + 1) % 3, p, 0, False, True, True, ((p + 1) % 3, p, 1, False, True), pre_nops=True)
        run_iter((p + 1) % 3, p, 1, False, False, True, ((p + 1) % 3, p, 0, False, False), pre_nops=True)
        a(f"s_branch {end}")
    for blk in g.slow_blocks:
        g.L.extend(blk)
    a(f"{end}:")
    a("s_waitcnt lgkmcnt(0)")
    a("s_nop 7")
    a("s_nop 7")
    a("s_nop 7")
    return g.L


def trans_gaps(lines):
    """A vector op that reads the result of the transcendental op just before
    it needs one wait state (gfx950): insert s_nop 0 there."""
    out = []
    for ln in lines:
        if out and out[-1].startswith("v_exp_f32"):
            dst = out[-1].split()[1].rstrip(",")
            ops = ln.replace(",", " ").split()[1:]
            if ln.startswith("v_") and dst in ops[1:] if not ln.startswith("v_dot2c") else dst in ops:
                out.append("s_nop 0")
        out.append(ln)
    return out


if __name__ == "__main__":
    lines = trans_gaps(generate())
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "sfa_fwd_d128_loop.inc"), "w") as f:
        f.write("// Generated by gen_fwd_d128_loop.py: the key-tile loop of the head-dim-128\n")
        f.write("// prefill as one instruction stream (see that script for the register map).\n")
        f.write("#define HD_FWD_D128_LOOP \\\n")
        for ln in lines:
            f.write('    "' + ln + '\\n\\t" \\\n')
        f.write('    ""\n')
        clob = ([f'"v{i}"' for i in range(128, 231)] + [f'"s{i}"' for i in range(80, 94)] +
                ['"vcc"', '"m0"', '"scc"', '"memory"'])
        f.write("#define HD_FWD_D128_CLOBBERS " + ", ".join(clob) + "\n")
    print(len(lines), "lines")
