"""Writes sfa_fwd_d128_loop.inc: the key-tile loop of the head-dim-128 prefill
kernel as one hand-scheduled gfx950 instruction stream, for a wave of 64
queries (two 32-query halves) at one wave per SIMD.

The loop is software-pipelined over 32-key sub-tiles i = 0, 1, ...: iteration
i issues the QK^T MFMAs of sub-tile i (8 k-steps x 2 halves; each K fragment
read from LDS feeds both halves), the softmax of sub-tile i-1 (vector ALU, both
halves) and the PV MFMAs of sub-tile i-2 (2 key steps x 4 dim blocks x 2
halves; each V^T fragment feeds both halves).  The softmax instructions are
placed one by one between the MFMAs by a cost-aware list schedule (each op at
least one MFMA after its inputs), so that the vector ALU and the matrix core
work at the same time within the wave; operands are read from LDS two reads
ahead into small register rings.  64-key K and V tiles are copied direct to
LDS into three-deep rings with one barrier per tile: K of tile T+2 and V of
tile T+1 are copied during tile T, from the first MFMA slots of the tile, and
the tile header waits only for the K copies (V is first read two tiles after
its copy starts), so the next tile's first operand reads can be issued before
its barrier.

The softmax uses only instructions that issue beside the MFMAs: v_fma_f32,
v_exp_f32, v_cvt_pk_bf16_f32 and v_add_f32 (the row sum adds the fp32
probabilities; the packed bf16 dot instruction stalls the matrix core).  A
sub-tile's probabilities are taken against the running maximum as it stands;
when some row has no maximum yet or a lane's share of its row sum exceeds
2^32, an out-of-line path takes the sub-tile maximum of both halves, rescales
O and l and recomputes the probabilities.  Band masks (diagonal, sequence
end, window start) are applied to a sub-tile's scores before its softmax, on
the sub-tiles that need them only.  After the loop the block sums l over the
lane pair, scales O by 1/l (hardware reciprocal and one Newton step) and
writes the bf16 rows to LDS, where the caller picks them up for whole-row
stores.  Every hazard the hardware does not check is padded here: MFMA
results are read by vector ops at least eight MFMAs later (or after s_nop),
a transcendental result is not read by the next instruction, a compare's
mask is read after s_nop 1.

Run `python gen_fwd_d128_loop.py` after editing; the output is committed.
Register map (per lane):
  a[0:127]   O^T accumulators of half h, dims 32db..+31: a[64h+16db : +15]
             (MFMA accumulators in AGPRs cost nothing; A / B operands read
             from AGPRs slow the loop down, so Q stays in VGPRs)
  v[0:63]    score accumulators: sub-tile buffer u, half h: v[32u+16h : +15]
  v[64:95]   bf16 probabilities: buffer u, half h: v[64+16u+8h : +7]
  v[96:159]  Q^T operand of half h, k-step ks: v[96+32h+4ks : +3]
  v160, v161 running max of half 0 / 1 (log2 units); v162, v163 row sums
  v[164:171] LDS byte address of the K operand of k-step ks (K buffer 0, keys 0-31)
  v[172:179] LDS byte address of the V^T half-operand (db, jh) (V buffer 0, keys 0-15)
  v[180:183] K copy offsets, v[184:187] V copy offsets (4 per tile per wave)
  v[188:195] the same for a tile with rows past the end of the sub-sequence
  v196, v197 mask base (4*hi - lo) of half 0 / 1; v198, v199 span
  v[200:211] K operand ring, v[212:223] V^T operand ring
  v[224:229] fma ring, v[230:235] exp ring
  v236, v237 sub-tile row sums (1/l after the loop); v[238:241] partial row
             sums; v242, v243 -max; v[244:246] temporaries; v247 -inf;
             v248 2^32; v249 staging address
Scalar registers s80..s93 are the loop's.
"""
import os
import sys

KT_BYTES = 16384
V_RING = 3 * KT_BYTES
LOOK = 4                  # MFMA slots ahead that operand reads are issued (2 reads)
RING = 3                  # operand ring entries (enough for two reads ahead)
COST = {"fma": 5, "exp": 12, "cvt": 5}  # vector cycles of one wave64 op (measured)
BUDGET = 30               # vector-ALU cycles placed after one MFMA
CMPNOP = "s_nop 1"        # wait states between a compare and the reader of its mask

S_AT = lambda u, h: 32 * u + 16 * h
P_AT = lambda u, h: 64 + 16 * u + 8 * h
Q_V = lambda h, ks: 96 + 32 * h + 4 * ks          # Q^T operands in VGPRs (an AGPR B operand is slow)
M = (160, 161)
L = (162, 163)
KADDR, VADDR = 164, 172
CPK, CPV, TPK, TPV = 180, 184, 188, 192
MB, SPAN = (196, 197), (198, 199)
KRING = 200
VRING = KRING + 4 * RING
F_RING = VRING + 4 * RING
NRING = 6
E_RING = F_RING + NRING
RS = (E_RING + NRING, E_RING + NRING + 1)
PART = RS[1] + 1
NM = (PART + 4, PART + 5)
T = PART + 6
NINF, TWO32 = T + 3, T + 4
STG = TWO32 + 1
LAST = STG
assert LAST <= 255, LAST
O_A = lambda h, db: 64 * h + 16 * db
OPITCH = 272
SGPR = dict(T="s80", j="s81", kt="s82", kdlo="s84", kdhi="s85", vdlo="s86", vdhi="s87",
            tk="s88", tv="s89", m="s[90:91]", m2="s[92:93]")


INV = (RS[0], RS[1])   # 1/l after the loop (the sub-tile row sums are dead by then)


def vr(b, n):
    return f"v[{b}:{b + n - 1}]"


def ar(b, n):
    return f"a[{b}:{b + n - 1}]"


def slot_list(qk, pv):
    a = [("qk", ks, h) for ks in range(8) for h in range(2)] if qk else \
        [("ghost", ks, h) for ks in range(8) for h in range(2)]
    b = [("pv", m2, db, h) for m2 in range(2) for db in range(4) for h in range(2)] if pv else []
    return a + b


def has_reads(slot):
    if slot[-1] != 0:
        return False
    return slot[0] != "ghost" or slot[1] < LOOK // 2


def read_texts(slot, kbuf, vbuf, u):
    if slot[0] in ("qk", "ghost"):
        ks = slot[1]
        return "k", [f"ds_read_b128 {{dst}}, v{KADDR + ks} offset:{kbuf * KT_BYTES + u * 8192}"]
    m2, db = slot[1], slot[2]
    off = vbuf * KT_BYTES + u * 8192 + m2 * 4096
    return "v", [f"ds_read_b64_tr_b16 {{dlo}}, v{VADDR + db * 2} offset:{off}",
                 f"ds_read_b64_tr_b16 {{dhi}}, v{VADDR + db * 2 + 1} offset:{off}"]


def softmax_ops(u):
    """Vector ops of the softmax of sub-tile buffer u, both halves."""
    ops = []
    fid, eid, cid, aid = {}, {}, {}, {}
    for h in range(2):
        sb, pb = S_AT(u, h), P_AT(u, h)
        prev = {0: None, 1: None}
        for r in range(16):
            i = 16 * h + r
            fid[i] = len(ops)
            ops.append(["fma", f"v_fma_f32 v{F_RING + i % NRING}, v{sb + r}, %[sc], v{NM[h]}", [], []])
            eid[i] = len(ops)
            ops.append(["exp", f"v_exp_f32 v{E_RING + i % NRING}, v{F_RING + i % NRING}", [fid[i]], []])
            aid[i] = len(ops)
            part = PART + 2 * h + (r % 2)
            if r < 2:
                ops.append(["fma", f"v_mov_b32 v{part}, v{E_RING + i % NRING}", [eid[i]], []])
            else:
                ops.append(["fma", f"v_add_f32 v{part}, v{part}, v{E_RING + i % NRING}", [eid[i], prev[r % 2]], []])
            prev[r % 2] = aid[i]
            if r % 2 == 1:
                cid[i // 2] = len(ops)
                ops.append(["cvt", f"v_cvt_pk_bf16_f32 v{pb + r // 2}, v{E_RING + (i - 1) % NRING}, "
                                   f"v{E_RING + i % NRING}", [eid[i - 1], eid[i]], []])
        ops.append(["fma", f"v_add_f32 v{RS[h]}, v{PART + 2 * h}, v{PART + 2 * h + 1}", [prev[0], prev[1]], []])
    for i in range(NRING, 32):
        ops[fid[i]][3].append(eid[i - NRING])
        ops[eid[i]][3].append(cid[(i - NRING) // 2])
        ops[eid[i]][3].append(aid[i - NRING])
    return ops


def schedule(ops, nslots, budget=BUDGET):
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
        self.ring_k = 0
        self.ring_v = 0
        self.fifo = []
        self.label_n = 0
        self.slow_blocks = []
        self.cur = None

    def a(self, s):
        self.L.append(s)

    def label(self, base):
        self.label_n += 1
        return f".Lhw{base}_{self.label_n}_%="

    def issue_reads(self, slot, kbuf, vbuf, u):
        kind, texts = read_texts(slot, kbuf, vbuf, u)
        if kind == "k":
            b = KRING + 4 * self.ring_k
            self.ring_k = (self.ring_k + 1) % RING
            self.a(texts[0].format(dst=vr(b, 4)))
            self.fifo.append((1, vr(b, 4)))
        else:
            b = VRING + 4 * self.ring_v
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

    def mask_block(self, u):
        skip, do = self.label("nomask"), self.label("mask")
        self.a(f"s_cmp_lt_u32 {SGPR['j']}, %[jw]")
        self.a(f"s_cbranch_scc1 {do}")
        self.a(f"s_cmp_ge_u32 {SGPR['j']}, %[jm]")
        self.a(f"s_cbranch_scc0 {skip}")
        self.a(f"{do}:")
        for h in range(2):
            sb = S_AT(u, h)
            self.a(f"v_add_u32 v{T}, {SGPR['kt']}, v{MB[h]}")
            for r in range(16):
                c = 8 * (r >> 2) + (r & 3)
                self.a(f"v_add_u32 v{T + 1}, {c}, v{T}")
                self.a(f"v_cmp_le_u32 vcc, v{T + 1}, v{SPAN[h]}")
                self.a(CMPNOP)
                self.a(f"v_cndmask_b32 v{sb + r}, v{NINF}, v{sb + r}, vcc")
        self.a(f"{skip}:")

    def slow_path(self, u, back):
        """Tile max, O and l rescale, probabilities again, for both halves (rare)."""
        lab = self.label("slow")
        body = [f"{lab}:", "s_nop 7", "s_nop 7", "s_nop 7"]
        for h in range(2):
            sb, pb = S_AT(u, h), P_AT(u, h)
            t0, t1, t2 = T, T + 1, T + 2
            body.append(f"v_max3_f32 v{t0}, v{sb}, v{sb + 1}, v{sb + 2}")
            for r in range(3, 16, 2):
                if r + 1 < 16:
                    body.append(f"v_max3_f32 v{t0}, v{t0}, v{sb + r}, v{sb + r + 1}")
                else:
                    body.append(f"v_max_f32 v{t0}, v{t0}, v{sb + r}")
            body += [f"v_mov_b32 v{t1}, v{t0}", "s_nop 1", f"v_permlane32_swap_b32 v{t0}, v{t1}", "s_nop 1",
                     f"v_max_f32 v{t0}, v{t0}, v{t1}",
                     f"v_mul_f32 v{t0}, %[sc], v{t0}",            # tile max in log2 units
                     f"v_max_f32 v{t1}, v{M[h]}, v{t0}",          # new max
                     f"v_sub_f32 v{t2}, v{M[h]}, v{t1}",
                     f"v_exp_f32 v{t2}, v{t2}",
                     f"v_cmp_eq_f32 vcc, v{M[h]}, v{t1}",
                     "s_nop 4",
                     f"v_cndmask_b32_e64 v{t2}, v{t2}, 1.0, vcc"]  # alpha
            # O rescale only where a lane has a nonzero sum and alpha != 1
            skip = self.label("norescale")
            body += [f"v_cmp_neq_f32_e64 {SGPR['m']}, 0, v{L[h]}",
                     f"v_cmp_neq_f32 vcc, 1.0, v{t2}",
                     "s_nop 4",
                     f"s_and_b64 vcc, vcc, {SGPR['m']}",
                     "s_and_b64 vcc, vcc, exec",
                     f"s_cbranch_vccz {skip}"]
            for i0 in range(0, 64, 8):
                for k in range(8):
                    body.append(f"v_accvgpr_read_b32 v{F_RING + k}, a{64 * h + i0 + k}")
                for k in range(8):
                    body.append(f"v_mul_f32 v{F_RING + k}, v{F_RING + k}, v{t2}")
                for k in range(8):
                    body.append(f"v_accvgpr_write_b32 a{64 * h + i0 + k}, v{F_RING + k}")
            body.append(f"{skip}:")
            body += [f"v_mul_f32 v{L[h]}, v{L[h]}, v{t2}", f"v_mov_b32 v{M[h]}, v{t1}",
                     f"v_sub_f32 v{NM[h]}, 0, v{t1}",
                     f"v_cmp_eq_f32 vcc, v{NINF}, v{t1}",
                     "s_nop 4",
                     f"v_cndmask_b32_e64 v{NM[h]}, v{NM[h]}, 0, vcc"]
            for r in range(16):
                body.append(f"v_fma_f32 v{F_RING + r % 6}, v{sb + r}, %[sc], v{NM[h]}")
                body.append("s_nop 0")
                body.append(f"v_exp_f32 v{E_RING + r % 6}, v{F_RING + r % 6}")
                body.append("s_nop 0")
                if r == 0:
                    body.append(f"v_mov_b32 v{RS[h]}, v{E_RING}")
                else:
                    body.append(f"v_add_f32 v{RS[h]}, v{RS[h]}, v{E_RING + r % 6}")
                if r % 2 == 1:
                    body.append(f"v_cvt_pk_bf16_f32 v{pb + r // 2}, v{E_RING + (r - 1) % 6}, v{E_RING + r % 6}")
        body += ["s_nop 7", f"s_branch {back}"]
        self.slow_blocks.append(body)
        return lab

    def check(self, u):
        back = self.label("back")
        slow = self.slow_path(u, back)
        self.a(f"v_cmp_nge_f32 vcc, v{TWO32}, v{RS[0]}")
        self.a(f"v_cmp_nge_f32_e64 {SGPR['m']}, v{TWO32}, v{RS[1]}")
        self.a(f"v_cmp_eq_f32_e64 {SGPR['m2']}, v{NINF}, v{M[0]}")
        self.a(CMPNOP)
        self.a(f"s_or_b64 vcc, vcc, {SGPR['m']}")
        self.a(f"s_or_b64 vcc, vcc, {SGPR['m2']}")
        self.a(f"v_cmp_eq_f32_e64 {SGPR['m']}, v{NINF}, v{M[1]}")
        self.a(CMPNOP)
        self.a(f"s_or_b64 vcc, vcc, {SGPR['m']}")
        self.a("s_and_b64 vcc, vcc, exec")
        self.a(f"s_cbranch_vccnz {slow}")
        self.a(f"{back}:")
        self.a(f"v_add_f32 v{L[0]}, v{L[0]}, v{RS[0]}")
        self.a(f"v_add_f32 v{L[1]}, v{L[1]}, v{RS[1]}")

    def iteration(self, u, kbuf, vbuf, qk, sm, pv, nxt, pre_nops=False, extra=None):
        """Sub-tile iteration with u = i % 2: QK writes S[u], the softmax reads
        S[1-u] and writes P[1-u], PV reads P[u]."""
        slots = slot_list(qk, pv)
        nslots = slot_list(nxt[3], nxt[4])
        stream = [(s, kbuf, vbuf, u) for s in slots] + [(s, nxt[0], nxt[1], nxt[2]) for s in nslots]
        if pre_nops:
            self.a("s_nop 7")
            self.a("s_nop 7")
            self.a("s_nop 7")
        if sm:
            self.mask_block(1 - u)
        per = schedule(softmax_ops(1 - u), len(slots)) if sm else [[] for _ in slots]
        first_pv = True
        for n, slot in enumerate(slots):
            if has_reads(slot):
                self.cur = self.take(wait=slot[0] != "ghost")
            target = self.cur
            if slot[0] == "qk":
                ks, h = slot[1], slot[2]
                d = vr(S_AT(u, h), 16)
                src_c = "0" if ks == 0 else d
                self.a(f"v_mfma_f32_32x32x16_bf16 {d}, {target}, {vr(Q_V(h, ks), 4)}, {src_c}")
            elif slot[0] == "pv":
                m2, db, h = slot[1], slot[2], slot[3]
                if first_pv and not qk:
                    self.a("s_nop 2")
                first_pv = False
                o = ar(O_A(h, db), 16)
                self.a(f"v_mfma_f32_32x32x16_bf16 {o}, {target}, {vr(P_AT(u, h) + 4 * m2, 4)}, {o}")
            ahead = n + LOOK
            if ahead < len(stream):
                s2, kb2, vb2, u2 = stream[ahead]
                if has_reads(s2):
                    self.issue_reads(s2, kb2, vb2, u2)
            if extra and n in extra:
                for t in extra[n]:
                    self.a(t)
            for t in per[n]:
                self.a(t)
        if sm:
            self.check(1 - u)
            self.a(f"s_add_u32 {SGPR['j']}, {SGPR['j']}, 1")
            self.a(f"s_add_u32 {SGPR['kt']}, {SGPR['kt']}, 32")


def generate():
    g = Gen()
    a = g.a
    # ---- set-up: O = 0, constants --------------------------------------------------
    for i in range(128):
        a(f"v_accvgpr_write_b32 a{i}, 0")
    a(f"v_mov_b32 v{NINF}, 0xff800000")
    a(f"v_mov_b32 v{TWO32}, 0x4f800000")
    a(f"v_mov_b32 v{NM[0]}, 0")
    a(f"v_mov_b32 v{NM[1]}, 0")
    a(f"s_mov_b32 {SGPR['T']}, 0")
    a(f"s_mov_b32 {SGPR['j']}, 0")
    a(f"s_mov_b32 {SGPR['kt']}, %[kt0]")
    a(f"s_mov_b64 s[{SGPR['kdlo'][1:]}:{SGPR['kdhi'][1:]}], %[kptr2]")
    a(f"s_mov_b64 s[{SGPR['vdlo'][1:]}:{SGPR['vdhi'][1:]}], %[vptr1]")

    def dma(kind, buf, tail_idx_sgpr, out):
        """Copy the tile at the running pointer into ring buffer `buf` (lines
        appended to `out`), then advance the pointer.  kind 'k' or 'v'."""
        a = out.append
        lo, hi = (SGPR['kdlo'], SGPR['kdhi']) if kind == "k" else (SGPR['vdlo'], SGPR['vdhi'])
        ring = 0 if kind == "k" else V_RING
        offs = CPK if kind == "k" else CPV
        toffs = TPK if kind == "k" else TPV
        normal, done = g.label("dman"), g.label("dmad")
        a(f"s_cmp_eq_u32 {tail_idx_sgpr}, %[tailt]")
        a(f"s_cbranch_scc0 {normal}")
        for i in range(4):
            a(f"s_add_u32 m0, %[ldsw], {ring + buf * KT_BYTES + i * 1024}")
            a("s_nop 0")
            a(f"global_load_lds_dwordx4 v{toffs + i}, s[{lo[1:]}:{hi[1:]}]")
        a(f"s_branch {done}")
        a(f"{normal}:")
        for i in range(4):
            a(f"s_add_u32 m0, %[ldsw], {ring + buf * KT_BYTES + i * 1024}")
            a("s_nop 0")
            a(f"global_load_lds_dwordx4 v{offs + i}, s[{lo[1:]}:{hi[1:]}]")
        a(f"{done}:")
        a(f"s_add_u32 {lo}, {lo}, %[tbytes]")
        a(f"s_addc_u32 {hi}, {hi}, 0")

    # The caller has issued the copies of K(0), K(1) (if any) and V(0) and
    # passes the pointers of the next tiles to copy: K(2) and V(1).
    a(f"s_mov_b32 {SGPR['tk']}, 2")
    a(f"s_mov_b32 {SGPR['tv']}, 1")

    def header(p):
        """Start of tile T (T % 3 == p): wait for the K copies issued one
        tile ago (the last 4 copies, of V, may stay in flight: V(T+1) is first
        read in tile T+2), barrier; returns the copies of K(T+2) and V(T+1),
        which the tile's first iteration issues after its MFMA slots 1 and 5."""
        a = g.a
        nahead = sum(x[0] for x in g.fifo)
        a("s_waitcnt vmcnt(4)")
        a(f"s_waitcnt lgkmcnt({min(nahead, 15)})")
        a("s_barrier")
        nk, nv = g.label("nok"), g.label("nov")
        kl, vl = [], []
        kl.append(f"s_cmp_lt_u32 {SGPR['tk']}, %[nt]")
        kl.append(f"s_cbranch_scc0 {nk}")
        dma("k", (p + 2) % 3, SGPR['tk'], kl)
        kl.append(f"{nk}:")
        kl.append(f"s_add_u32 {SGPR['tk']}, {SGPR['tk']}, 1")
        vl.append(f"s_cmp_lt_u32 {SGPR['tv']}, %[nt]")
        vl.append(f"s_cbranch_scc0 {nv}")
        dma("v", (p + 1) % 3, SGPR['tv'], vl)
        vl.append(f"{nv}:")
        vl.append(f"s_add_u32 {SGPR['tv']}, {SGPR['tv']}, 1")
        return {1: kl, 5: vl}

    def run_iter(kbuf, vbuf, u, qk, sm, pv, nxt, pre_nops=False, extra=None):
        g.iteration(u, kbuf, vbuf, qk, sm, pv, nxt, pre_nops=pre_nops, extra=extra)

    def start_reads(kbuf, vbuf, u, qk, pv):
        for s in slot_list(qk, pv)[:LOOK]:
            if has_reads(s):
                g.issue_reads(s, kbuf, vbuf, u)

    drain_labels = {p: g.label(f"drain{p}") for p in range(3)}
    tile_labels = {p: g.label(f"tile{p}") for p in range(3)}

    a("s_nop 7")   # AGPR writes before the first MFMA accumulates into them
    ex0 = header(0)
    start_reads(0, 0, 0, True, False)
    run_iter(0, 0, 0, True, False, False, (0, 0, 1, True, False), extra=ex0)
    run_iter(0, 0, 1, True, True, False, (1, 0, 0, True, True), pre_nops=True)
    a("s_nop 7")
    a("s_nop 7")
    a("s_nop 7")
    a(f"s_add_u32 {SGPR['T']}, {SGPR['T']}, 1")
    a(f"s_cmp_eq_u32 {SGPR['T']}, %[nt]")
    a(f"s_cbranch_scc1 {drain_labels[0]}")
    for p in (1, 2, 0):
        a(f"{tile_labels[p]}:")
        ex = header(p)
        kb, vb = p, (p - 1) % 3
        run_iter(kb, vb, 0, True, True, True, (kb, vb, 1, True, True), extra=ex)
        run_iter(kb, vb, 1, True, True, True, ((p + 1) % 3, p, 0, True, True))
        a(f"s_add_u32 {SGPR['T']}, {SGPR['T']}, 1")
        a(f"s_cmp_eq_u32 {SGPR['T']}, %[nt]")
        a(f"s_cbranch_scc1 {drain_labels[p]}")
        a(f"s_branch {tile_labels[(p + 1) % 3]}")
    end = g.label("end")
    saved = (list(g.fifo), g.ring_k, g.ring_v)
    for p in range(3):
        g.fifo, g.ring_k, g.ring_v = list(saved[0]), saved[1], saved[2]
        a(f"{drain_labels[p]}:")
        a("s_waitcnt vmcnt(0)")   # V of the last tile
        a("s_barrier")
        run_iter((p + 1) % 3, p, 0, False, True, True, ((p + 1) % 3, p, 1, False, True), pre_nops=True)
        run_iter((p + 1) % 3, p, 1, False, False, True, ((p + 1) % 3, p, 0, False, False), pre_nops=True)
        a(f"s_branch {end}")
    for blk in g.slow_blocks:
        g.L.extend(blk)
    a(f"{end}:")
    # ---- epilogue: row sums over the lane pair, O / l to LDS staging ---------------
    a("s_waitcnt lgkmcnt(0)")
    a("s_nop 7")
    a("s_nop 7")
    a("s_nop 7")
    for h in range(2):
        a(f"v_mov_b32 v{T}, v{L[h]}")
        a(f"v_mov_b32 v{T + 1}, v{L[h]}")
        a("s_nop 1")
        a(f"v_permlane32_swap_b32 v{T}, v{T + 1}")
        a("s_nop 1")
        a(f"v_add_f32 v{L[h]}, v{T}, v{T + 1}")
        # 1/l: hardware reciprocal and one Newton step
        a(f"v_rcp_f32 v{INV[h]}, v{L[h]}")
        a("s_nop 0")
        a(f"v_fma_f32 v{T}, -v{L[h]}, v{INV[h]}, 1.0")
        a(f"v_fma_f32 v{INV[h]}, v{T}, v{INV[h]}, v{INV[h]}")
    a("s_barrier")   # every wave has left the loop: the rings are free
    n = 0
    for h in range(2):
        for db in range(4):
            for r4 in range(4):
                t = 4 * (n % 16)
                n += 1
                for e in range(4):
                    a(f"v_accvgpr_read_b32 v{t + e}, a{O_A(h, db) + 4 * r4 + e}")
                for e in range(4):
                    a(f"v_mul_f32 v{t + e}, v{t + e}, v{INV[h]}")
                a(f"v_cvt_pk_bf16_f32 v{t}, v{t}, v{t + 1}")
                a(f"v_cvt_pk_bf16_f32 v{t + 1}, v{t + 2}, v{t + 3}")
                a(f"ds_write_b64 v{STG}, v[{t}:{t + 1}] offset:{h * 32 * OPITCH + db * 64 + r4 * 16}")
    a("s_waitcnt lgkmcnt(0)")
    return g.L


def trans_gaps(lines):
    out = []
    for ln in lines:
        if out and (out[-1].startswith("v_exp_f32") or out[-1].startswith("v_rcp_f32")):
            dst = out[-1].split()[1].rstrip(",")
            ops = ln.replace(",", " ").split()[1:]
            if ln.startswith("v_") and (dst in ops[1:] or ("-" + dst) in ops[1:]):
                out.append("s_nop 0")
        out.append(ln)
    return out


if __name__ == "__main__":
    out_path = sys.argv[sys.argv.index("--out") + 1] if "--out" in sys.argv else \
        os.path.join(os.path.dirname(os.path.abspath(__file__)), "sfa_fwd_d128_loop.inc")
    lines = trans_gaps(generate())
    with open(out_path, "w") as f:
        f.write("// Generated by gen_fwd_d128_loop.py: the key-tile loop of the head-dim-128\n")
        f.write("// prefill as one instruction stream (see that script for the register map).\n")
        f.write("#define HD_FWD_D128_LOOP \\\n")
        for ln in lines:
            f.write('    "' + ln + '\\n\\t" \\\n')
        f.write('    ""\n')
        clob = ([f'"v{i}"' for i in list(range(0, 96)) + list(range(KRING, STG))] +
                [f'"a{i}"' for i in range(128)] +
                [f'"s{i}"' for i in range(80, 94)] +
                ['"vcc"', '"m0"', '"scc"', '"memory"'])
        f.write("#define HD_FWD_D128_CLOBBERS " + ", ".join(clob) + "\n")
    print(len(lines), "lines")
