"""Writes attn_bwd_dq_w64_loop.h: the key loop of the one-wave-per-SIMD dQ
kernel of the attention backward (bf16, D = 128) as one inline-asm statement
with a fixed instruction schedule and a fixed register plan.

A wave owns 64 query rows in two 32-row blocks; Q and dO of both blocks stay
in AGPRs. The key block is walked in 32-key sub-tiles j (two per 64-key
tile). With p = exp2(S c - lse2) and dS = p (dP - delta):
  phase A(j): the S^T = K Q^T and dP^T = V dO^T MFMAs of sub-tile j+1 (each
              K or V row read from LDS feeds the MFMA of both blocks) with
              the dS arithmetic of sub-tile j of both blocks between them;
  phase B(j): dQ^T += K^T dS^T of sub-tile j (each K^T read feeds both
              blocks), with p of block 0 of sub-tile j+1 between them
              (written over its S), so both phases carry vector work.
The last pairs of each phase issue the first operand reads of the next one.
The backward's probabilities use the saved lse ("Sequence Parallelism in
Large Language Models ...", section "The Activation Memory Wall":
recomputation instead of stored activations), so there is no running max
and no rescale; the causal mask is applied out of line to the sub-tiles
from the wave's first partly visible one.

Tiles reach LDS through direct global->LDS loads: K and V row tiles (64 keys,
padded rows) rotate through three buffers, K^T tiles (D rows of 64 keys)
through two. One barrier per 64-key tile t publishes the loads of the
previous tile and frees the buffers it refills; a wave's thirteen loads of K
and V rows of tile t+2 and K^T of tile t+1 are spread over the MFMA pairs of
that tile's first phase A. Tiles past the last one repeat the last one (into
a buffer nobody reads), so no wave branches around its loads.

Register plan (one wave per SIMD: 256 VGPRs + 256 AGPRs):
  a[0:63]     dQ^T of block 0, four 32-wide d tiles of 16 registers
  a[64:127]   dQ^T of block 1
  a[128:191]  Q of blocks 0 and 1 (eight k-steps of 4 registers each)
  a[192:255]  dO of blocks 0 and 1
  v[40:55]    minus delta of block 1, 16 copies (the first dP^T MFMA's
              accumulator input, so dP - delta comes out of the chain)
  v56 row-tile read address, v57 K^T read address, v[58:61] temporaries
  v[64:79]    LDS operand ring, four 16-byte reads in flight
  v[80:95]    dS_x: bf16 dS^T of blocks 0 / 1 (even sub-tiles)
  v[96:111]   dS_y (odd sub-tiles)
  v[112:175]  set x: S^T and dP^T of blocks 0 and 1 (even sub-tiles)
  v[176:239]  set y (odd sub-tiles)
  v[240:255]  minus delta of block 0, 16 copies
  s[80:81], s[82:83], s[84:85]: global addresses of the next K rows, V rows
  and K^T tiles
The compiler keeps everything else in v[0:39] and the other SGPRs.

Hazards the statement respects by construction, and check_hazards verifies
on the executed paths (several trip counts, each out-of-line mask) before
the header is written: a transcendental result is read no earlier than the
second instruction after it; MFMA results are read by vector instructions
only a phase later, or by the out-of-line mask and after the statement, each
behind s_nop 7 x 3 (at least 19 wait states); an M0 write is not directly
followed by the LDS-DMA load that reads it; an MFMA operand read from LDS
has returned when the MFMA issues (LDS reads return in order; each pair's
lgkmcnt wait sits right after the previous pair's first MFMA, and no other
LGKM operation is in flight). An MFMA accumulator is reused no sooner than three MFMAs later.

Run: python gen_bwd_dq_w64.py  (writes the header next to this file)
"""
import os
import re

D = 128
KS = D // 16            # k-steps of the S / dP products
DT = D // 32            # d tiles of dQ
ROW = (D // 8 + 1) * 16     # padded K / V row in LDS, bytes
TROW = 9 * 16               # padded K^T row (64 keys + pad), bytes
RBUF = 64 * ROW             # one 64-row tile
RT = 2 * RBUF               # K rows then V rows
TBUF = D * TROW             # one K^T tile
RBUFS = 3
HALF_R = 32 * ROW           # second 32-key half of a row tile
HALF_T = 64                 # second 32-key half of a K^T tile (bytes)
NA, NB = 2 * KS, 2 * DT     # operand reads of phase A / B
PF = 4
NEG_INF = "0xff800000"

DQ_ = (0, 64)
Q_ = (128, 160)
DO_ = (192, 224)
V_RADDR, V_TADDR = 56, 57
T0, T1, T2, T3 = 58, 59, 60, 61
RING = 64
DS_ = {0: (80, 88), 1: (96, 104)}                  # per parity: block 0, block 1
SET_ = {0: (112, 128, 144, 160), 1: (176, 192, 208, 224)}   # S0, S1, dP0, dP1
NDL_ = (240, 40)        # minus delta of block 0 / 1, 16 copies: the dP^T accumulators' start
PAD = ["s_nop 7", "s_nop 7", "s_nop 7"]
KG_S, VG_S, TG_S = 80, 82, 84


def vr(base, n):
    return f"v[{base}:{base + n - 1}]"


def ar(base, n):
    return f"a[{base}:{base + n - 1}]"


def ring(i):
    return vr(RING + 4 * (i % PF), 4)


def row_off(i):
    """Phase A read i: even = K row (k-step i/2), odd = V row."""
    return (i & 1) * RBUF + 32 * (i >> 1)


def kt_off(i):
    """Phase B read i: d tile T = i % DT, 16-key step u = i // DT."""
    return 32 * (i % DT) * TROW + 32 * (i // DT)


def a_mfmas(par):
    """S^T / dP^T of both blocks into the set of parity `par`; the first
    k-step starts S^T from 0 and dP^T from minus delta."""
    S0, S1, P0, P1 = SET_[par]

    def f(i):
        s = i >> 1
        if i & 1:
            d0, d1, b0, b1 = P0, P1, DO_[0], DO_[1]
        else:
            d0, d1, b0, b1 = S0, S1, Q_[0], Q_[1]
        if s > 0:
            c0, c1 = vr(d0, 16), vr(d1, 16)
        elif i & 1:     # dP^T - delta comes out of the chain
            c0, c1 = vr(NDL_[0], 16), vr(NDL_[1], 16)
        else:
            c0 = c1 = "0"
        return (f"v_mfma_f32_32x32x16_bf16 {vr(d0, 16)}, {ring(i)}, {ar(b0 + 4 * s, 4)}, {c0}",
                f"v_mfma_f32_32x32x16_bf16 {vr(d1, 16)}, {ring(i)}, {ar(b1 + 4 * s, 4)}, {c1}")
    return f


def b_mfmas(par):
    """dQ^T of both blocks from dS of parity `par`."""
    ds0, ds1 = DS_[par]

    def f(i):
        T, u = i % DT, i // DT
        return (f"v_mfma_f32_32x32x16_bf16 {ar(DQ_[0] + 16 * T, 16)}, {ring(i)}, "
                f"{vr(ds0 + 4 * u, 4)}, {ar(DQ_[0] + 16 * T, 16)}",
                f"v_mfma_f32_32x32x16_bf16 {ar(DQ_[1] + 16 * T, 16)}, {ring(i)}, "
                f"{vr(ds1 + 4 * u, 4)}, {ar(DQ_[1] + 16 * T, 16)}")
    return f


def p_early(k, par):
    """p = exp2(S c - lse2) of block 0, elements 2k, 2k+1 of the set of
    parity `par`, written over S: the work of phase B pair k of the sub-tile
    before, whose MFMAs carry no vector work of their own."""
    S0 = SET_[par][0]
    e = 2 * k
    return [f"v_fma_f32 v{T0}, v{S0 + e}, %[c], %[nl20]",
            f"v_fma_f32 v{T1}, v{S0 + e + 1}, %[c], %[nl20]",
            f"v_exp_f32 v{S0 + e}, v{T0}",
            f"v_exp_f32 v{S0 + e + 1}, v{T1}"]


def ds_pair(i, par):
    """dS of elements 2k, 2k+1 (k = i % 8) of block b = i // 8 from the set
    of parity `par`, in two parts (one after each MFMA of a pair); block 0
    finds p already in place of S (p_early)."""
    b, k = i // 8, i % 8
    S0, S1, P0, P1 = SET_[par]
    S, P = (S0, P0) if b == 0 else (S1, P1)
    e = 2 * k
    dst = DS_[par][b] + 4 * (e >> 3) + ((e & 7) >> 1)
    if b == 0:
        return [], [f"v_mul_f32 v{T0}, v{S + e}, v{P + e}",
                    f"v_mul_f32 v{T1}, v{S + e + 1}, v{P + e + 1}",
                    f"v_cvt_pk_bf16_f32 v{dst}, v{T0}, v{T1}"]
    first = [f"v_fma_f32 v{T0}, v{S + e}, %[c], %[nl2{b}]",
             f"v_fma_f32 v{T1}, v{S + e + 1}, %[c], %[nl2{b}]",
             f"v_exp_f32 v{T0}, v{T0}",
             f"v_exp_f32 v{T1}, v{T1}"]
    second = [f"v_mul_f32 v{T0}, v{T0}, v{P + e}",
              f"v_mul_f32 v{T1}, v{T1}, v{P + e + 1}",
              f"v_cvt_pk_bf16_f32 v{dst}, v{T0}, v{T1}"]
    return first, second


def phase(n, mfmas, addr, off, work=None, pre_in=False, nxt=None, extra=()):
    """n MFMA pairs; pair i reads one operand (address register `addr`,
    offset off(i)) through the ring; work(i) = (first, second) vector work
    after the pair's two MFMAs; pre_in: the first PF reads were issued by the
    previous phase; nxt = (addr, off): the last PF pairs issue the first PF
    reads of the next phase; extra[i]: more instructions after pair i."""
    lines = [] if pre_in else ["s_waitcnt lgkmcnt(0)"]
    if not pre_in:
        for i in range(PF):
            lines.append(f"ds_read_b128 {ring(i)}, v{addr} offset:{off(i)}")
    for i in range(n):
        # reads 0 .. issued-1 are in flight or done, in order. Pair 0 waits
        # for its read before its first MFMA; every other pair's read is
        # waited for right after the previous pair's first MFMA, in the
        # slot where the wave could not issue vector work anyway
        issued = i + PF if nxt else min(n, i + PF)
        if i == 0:
            lines.append(f"s_waitcnt lgkmcnt({issued - 1})")
        first, second = work(i) if work else ([], [])
        ma, mb = mfmas(i)
        lines += [ma]
        if i + 1 < n:
            lines.append(f"s_waitcnt lgkmcnt({issued - (i + 2)})")
        lines += first + [mb]
        if i + PF < n:
            lines.append(f"ds_read_b128 {ring(i)}, v{addr} offset:{off(i + PF)}")
        elif nxt:
            lines.append(f"ds_read_b128 {ring(i)}, v{nxt[0]} offset:{nxt[1](i + PF - n)}")
        lines += second
        if i < len(extra):
            lines += extra[i]
    return lines


LOOP_CLOBBER = ([f'"v{r}"' for r in range(NDL_[1], NDL_[1] + 16)] +
                [f'"v{r}"' for r in range(V_RADDR, 256)] +
                ['"vcc"', '"scc"', '"m0"', '"exec"', '"memory"'])


class Loop:
    def __init__(self):
        self.lines = []
        self.ool = []

    def add(self, lines):
        self.lines += lines

    def lab(self, name):
        return f".L{name}_%="

    def place(self, name):
        self.lines.append(f"{self.lab(name)}:")

    def mask(self, par, jj_lines, site):
        """Causal mask of the sub-tile whose index jj_lines leave in %[sy]
        (SCC = 1 when it is at or past %[fmask]), on the set of parity par,
        out of line."""
        S0, S1, _, _ = SET_[par]
        self.add(jj_lines + ["s_cmp_ge_u32 %[sy], %[fmask]",
                             f"s_cbranch_scc1 {self.lab('mask' + site)}"])
        self.place("mback" + site)
        body = [f"{self.lab('mask' + site)}:"] + PAD + [
                "s_lshl_b32 %[sy], %[sy], 5",
                f"v_subrev_u32 v{T1}, %[sy], %[nalh0]",
                f"v_subrev_u32 v{T2}, %[sy], %[nalh1]",
                f"v_mov_b32 v{T0}, {NEG_INF}"]
        for S, lim in ((S0, T1), (S1, T2)):
            for e in range(16):
                k = 16 * (e >> 3) + (e & 7)
                body += [f"v_cmp_lt_i32 vcc, {k}, v{lim}",
                         f"v_cndmask_b32 v{S + e}, v{T0}, v{S + e}, vcc"]
        self.ool += body + [f"s_branch {self.lab('mback' + site)}"]


def load_groups():
    """The thirteen loads of tile t (three more under an all-or-nothing exec
    mask: the fifth chunk load of K, V and K^T, one of which a wave issues):
    K and V rows of tile min(t+2, n_kt-1) into row buffer %[rw], K^T of tile
    min(t+1, n_kt-1) into K^T buffer %[kto] ^ TBUF; then the global addresses
    advance (by a tile while the next one exists)."""
    g = []
    for name, dst, src, x5 in (("ko", "%[sx]", "kg", "%[x5k]"), ("vo", "%[sy]", "vg", "%[x5v]"),
                               ("to", "%[sz]", "tg", "%[x5t]")):
        for j in range(4):
            g.append([f"s_add_u32 m0, {dst}, {4096 * j}", "s_nop 0",
                      f"global_load_lds_dwordx4 %[{name}{j}], %[{src}]"])
        g.append([f"s_add_u32 m0, {dst}, 16384", f"s_mov_b64 exec, {x5}",
                  f"global_load_lds_dwordx4 %[{name}4], %[{src}]", "s_mov_b64 exec, -1"])
    g[-1] += ["s_add_u32 %[sx], %[t], 3", "s_cmp_lt_u32 %[sx], %[nkt]",
              f"s_cselect_b32 %[sx], {64 * D * 2}, 0",
              f"s_add_u32 s{KG_S}, s{KG_S}, %[sx]", f"s_addc_u32 s{KG_S + 1}, s{KG_S + 1}, 0",
              f"s_add_u32 s{VG_S}, s{VG_S}, %[sx]", f"s_addc_u32 s{VG_S + 1}, s{VG_S + 1}, 0",
              "s_add_u32 %[sx], %[t], 2", "s_cmp_lt_u32 %[sx], %[nkt]",
              "s_cselect_b32 %[sx], 128, 0",
              f"s_add_u32 s{TG_S}, s{TG_S}, %[sx]", f"s_addc_u32 s{TG_S + 1}, s{TG_S + 1}, 0"]
    return g


def loop_asm():
    L = Loop()
    L.add([f"v_accvgpr_write_b32 a{r}, 0" for r in range(128)])
    L.add([f"v_mov_b32 v{NDL_[b] + r}, %[ndl{b}]" for b in (0, 1) for r in range(16)])
    # prologue: S^T / dP^T of sub-tile 0 (row buffer 0, first half), whose
    # last pairs start the reads of sub-tile 1 (second half)
    L.add([f"v_mov_b32 v{V_RADDR}, %[rbase]"])
    L.add(phase(NA, a_mfmas(0), V_RADDR, row_off, nxt=(V_RADDR, lambda i: row_off(i) + HALF_R)))
    L.add(PAD + ["s_mov_b32 %[t], 0"])
    L.mask(0, ["s_mov_b32 %[sy], 0"], "pro")
    for k in range(8):
        L.add(p_early(k, 0))
    L.place("loop")
    # ---- even sub-tile j = 2t
    L.add(["s_waitcnt vmcnt(0)", "s_barrier",
           "s_add_u32 %[sx], %[kd], %[rw]", "s_add_u32 %[sy], %[vd], %[rw]",
           "s_xor_b32 %[sz], %[kto], " + str(TBUF), "s_add_u32 %[sz], %[td], %[sz]",
           f"v_add_u32 v{V_TADDR}, %[kto], %[tbase]"])
    L.add(phase(NA, a_mfmas(1), V_RADDR, lambda i: row_off(i) + HALF_R,
                work=lambda i: ds_pair(i, 0), pre_in=True, nxt=(V_TADDR, kt_off),
                extra=load_groups()))
    L.mask(1, ["s_lshl_b32 %[sy], %[t], 1", "s_add_u32 %[sy], %[sy], 1"], "e")
    L.add([f"v_add_u32 v{V_RADDR}, %[rn], %[rbase]"])
    L.add(phase(NB, b_mfmas(0), V_TADDR, kt_off, pre_in=True, nxt=(V_RADDR, row_off),
                work=lambda i: (p_early(i, 1), [])))
    # ---- odd sub-tile j = 2t+1
    L.add(["s_add_u32 %[sx], %[t], 1", "s_cmp_ge_u32 %[sx], %[nkt]",
           f"s_cbranch_scc1 {L.lab('last')}"])
    L.add(phase(NA, a_mfmas(0), V_RADDR, row_off, work=lambda i: ds_pair(i, 1), pre_in=True,
                nxt=(V_TADDR, lambda i: kt_off(i) + HALF_T)))
    L.mask(0, ["s_lshl_b32 %[sy], %[t], 1", "s_add_u32 %[sy], %[sy], 2"], "o")
    L.add([f"v_add_u32 v{V_RADDR}, %[rn], %[rbase]"])
    L.add(phase(NB, b_mfmas(1), V_TADDR, lambda i: kt_off(i) + HALF_T, pre_in=True,
                nxt=(V_RADDR, lambda i: row_off(i) + HALF_R),
                work=lambda i: (p_early(i, 0), [])))
    # next tile: rotate the row buffers and flip the K^T buffer
    L.add(["s_add_u32 %[t], %[t], 1", "s_mov_b32 %[sx], %[rt]", "s_mov_b32 %[rt], %[rn]",
           "s_mov_b32 %[rn], %[rw]", "s_mov_b32 %[rw], %[sx]",
           f"s_xor_b32 %[kto], %[kto], {TBUF}",
           f"s_branch {L.lab('loop')}"])
    # ---- the last (odd) sub-tile: its dS, then its dQ; no load is left in
    # flight when the statement ends
    L.place("last")
    L.add(["s_waitcnt vmcnt(0)", "s_waitcnt lgkmcnt(0)"])
    for i in range(16):
        first, second = ds_pair(i, 1)
        L.add(first + second)
    L.add(phase(NB, b_mfmas(1), V_TADDR, lambda i: kt_off(i) + HALF_T))
    L.add([f"s_branch {L.lab('done')}"])
    L.add(L.ool)
    L.place("done")
    L.add(PAD)
    return L.lines


XDL_WAIT = 19    # wait states between an MFMA and a vector access of its result
REG = re.compile(r"\b([va])(?:(\d+)\b|\[(\d+):(\d+)\])")


def regs(text):
    out = set()
    for m in REG.finditer(text):
        if m.group(2):
            out.add(m.group(1) + m.group(2))
        else:
            out.update(f"{m.group(1)}{r}" for r in range(int(m.group(3)), int(m.group(4)) + 1))
    return out


def trace(lines, policy, limit=40000):
    """The instructions one wave executes, branches decided by policy(label,
    count of earlier decisions at that label) -> taken."""
    where = {ln[:-1]: i for i, ln in enumerate(lines) if ln.endswith(":")}
    seen = {}
    out, i = [], 0
    while i < len(lines) and len(out) < limit:
        ln = lines[i]
        op, _, rest = ln.partition(" ")
        if ln.endswith(":"):
            if ln == ".Ldone_%=:":
                break
            i += 1
            continue
        out.append(ln)
        if op == "s_branch":
            i = where[rest.strip()]
            continue
        if op.startswith("s_cbranch"):
            lab = rest.strip()
            k = seen.get(lab, 0)
            seen[lab] = k + 1
            if policy(lab, k):
                i = where[lab]
                continue
        i += 1
    assert len(out) < limit, "trace did not reach the end"
    return out


def check_trace(tr):
    """Along one executed path: vector accesses of MFMA results at least
    XDL_WAIT wait states after the MFMA; no read of a transcendental result
    by the next instruction; no LDS-DMA load right after an M0 write; every
    register an LDS read is still writing left alone until a wait covers it."""
    last, trans, ws, pending, prev = {}, set(), 0, [], ""
    for ln in tr:
        op, _, rest = ln.partition(" ")
        if op == "s_nop":
            ws += int(rest) + 1
            trans, prev = set(), ln
            continue
        ops = [o.strip() for o in rest.split(",")]
        if op == "s_waitcnt" and "lgkmcnt" in rest:
            k = int(re.search(r"lgkmcnt\((\d+)\)", rest).group(1))
            pending = pending[len(pending) - k:] if len(pending) > k else pending
        if op.startswith("global_load_lds"):
            assert "m0" not in prev.split(" ", 1)[-1].split(",")[0], (prev, ln)
        if op.startswith("v_mfma"):
            for r in regs(",".join(ops[1:])):
                assert all(r not in p for p in pending), ("LDS read not waited for", ln)
            for r in regs(",".join(ops[1:3])):
                assert ws - last.get(r, -99) >= XDL_WAIT, ln
            for r in regs(ops[0]):
                last[r] = ws
        elif op.startswith("ds_"):
            for r in regs(",".join(ops[1:])):
                assert ws - last.get(r, -99) >= XDL_WAIT, ln
                assert all(r not in p for p in pending), ("LDS result", ln)
            pending.append(regs(ops[0]))
        elif op.startswith("v_"):
            for r in regs(rest):
                assert ws - last.get(r, -99) >= XDL_WAIT, (ln, ws - last.get(r, -99))
                assert all(r not in p for p in pending), ("LDS result", ln)
            assert not (regs(",".join(ops[1:])) & trans), ln
        trans = regs(ops[0]) if op == "v_exp_f32" else set()
        prev = ln
        ws += 1


def check_hazards(lines):
    """check_trace over the common path for several trip counts and over
    paths through each out-of-line mask."""
    for n_it in range(0, 4):
        check_trace(trace(lines, lambda lab, k, n_it=n_it: lab == ".Llast_%=" and k >= n_it))
    for fam in ("maskpro", "maske", "masko"):
        for when in (0, 1):
            def pol(lab, k, fam=fam, when=when):
                if lab == ".Llast_%=":
                    return k >= 2
                return lab == f".L{fam}_%=" and k == when
            check_trace(trace(lines, pol))


def main():
    lines = loop_asm()
    check_hazards(lines)
    outs = ([f'"={{{ar(DQ_[b] + 16 * T, 16)}}}"(dq{b}[{T}])' for b in (0, 1) for T in range(DT)] +
            ['[t] "=&s"(t)', '[sx] "=&s"(sx)', '[sy] "=&s"(sy)', '[sz] "=&s"(sz)',
             f'[kg] "+{{s[{KG_S}:{KG_S + 1}]}}"(kgv)', f'[vg] "+{{s[{VG_S}:{VG_S + 1}]}}"(vgv)',
             f'[tg] "+{{s[{TG_S}:{TG_S + 1}]}}"(tgv)',
             '[rt] "+s"(rt)', '[rn] "+s"(rn)', '[rw] "+s"(rw)', '[kto] "+s"(kto)'])
    ins = (['[nkt] "s"(n_kt)', '[fmask] "s"(first_mask)', '[kd] "s"(kd)', '[vd] "s"(vd)',
            '[td] "s"(td)', '[x5k] "s"(x5k)', '[x5v] "s"(x5v)', '[x5t] "s"(x5t)', '[c] "s"(c)',
            '[rbase] "v"(rbase)', '[tbase] "v"(tbase)', '[nl20] "v"(nl20)', '[nl21] "v"(nl21)',
            '[ndl0] "v"(ndl0)', '[ndl1] "v"(ndl1)', '[nalh0] "v"(nalh0)', '[nalh1] "v"(nalh1)'] +
           [f'[ko{j}] "v"(koff[{j}])' for j in range(5)] +
           [f'[vo{j}] "v"(voff[{j}])' for j in range(5)] +
           [f'[to{j}] "v"(toff[{j}])' for j in range(5)] +
           [f'"{{{ar(Q_[b] + 4 * s, 4)}}}"(q{b}[{s}])' for b in (0, 1) for s in range(KS)] +
           [f'"{{{ar(DO_[b] + 4 * s, 4)}}}"(do{b}[{s}])' for b in (0, 1) for s in range(KS)])
    body = "\n".join(f'      "{ln}\\n\\t"' for ln in lines)
    out = f'''// Generated by gen_bwd_dq_w64.py -- do not edit by hand.
//
// The key loop of attn_bwd_dq_w64 (D = {D}) as one inline-asm statement with
// a fixed schedule and fixed registers; gen_bwd_dq_w64.py documents the
// register plan, the schedule and the hazards it respects.
#pragma once

namespace ra {{
namespace dqw64 {{

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kRowBufs = {RBUFS};        // K / V row tile buffers ({RT} bytes each)
constexpr int kRowTileBytes = {RT};
constexpr int kKtBufBytes = {TBUF};      // one K^T tile; two buffers

// The key loop of one wave: n_kt >= 1 tiles of 64 keys. K / V row tiles 0
// and 1 (those the block has) are in row buffers 0 and 1, K^T tile 0 in K^T
// buffer 0. rbase: this lane's S / dP operand address in row buffer 0 (K
// rows, kperm'd, +16 bytes for the upper half of the wave); tbase: its dQ
// operand address in K^T buffer 0; kd / vd / td: this wave's first load
// destination in row buffer 0 (K part, V part) and K^T buffer 0; kg / vg:
// global address of the K / V row tile min(2, n_kt - 1), tg: of K^T tile
// min(1, n_kt - 1); koff / voff / toff: the lane's load offsets; x5k / x5v
// / x5t: whether the wave issues the fifth load of a K, V, K^T tile;
// first_mask: first 32-key sub-tile needing the causal mask; nalh0 / nalh1:
// keys visible to the lane's row of block 0 / 1, minus 8 for the upper half
// of the wave; nl20 / nl21: minus the rows' lse in exp2 units; ndl0 / ndl1:
// minus the rows' delta. Returns dQ^T of both blocks (unscaled).
__device__ __forceinline__ void dq_loop(
    int n_kt, int first_mask, unsigned kd, unsigned vd, unsigned td, int k5, int v5, int t5,
    float c, unsigned rbase, unsigned tbase, float nl20, float nl21, float ndl0, float ndl1,
    int nalh0, int nalh1, const void* kg, const void* vg, const void* tg,
    const unsigned (&koff)[5], const unsigned (&voff)[5], const unsigned (&toff)[5],
    const bf16x8 (&q0)[8], const bf16x8 (&q1)[8], const bf16x8 (&do0)[8],
    const bf16x8 (&do1)[8], floatx16 (&dq0)[4], floatx16 (&dq1)[4]) {{
  int t, sx, sy, sz;
  const long long x5k = k5 ? -1ll : 0ll, x5v = v5 ? -1ll : 0ll, x5t = t5 ? -1ll : 0ll;
  unsigned long long kgv = (unsigned long long)(size_t)kg, vgv = (unsigned long long)(size_t)vg;
  unsigned long long tgv = (unsigned long long)(size_t)tg;
  unsigned rt = 0, rn = {RT}, rw = {2 * RT}, kto = 0;  // row buffers of tiles t, t+1, t+2; K^T of t
  asm volatile(
{body}
      : {", ".join(outs)}
      : {", ".join(ins)}
      : {", ".join(LOOP_CLOBBER)});
}}

}}  // namespace dqw64
}}  // namespace ra
'''
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "attn_bwd_dq_w64_loop.h")
    with open(path, "w") as f:
        f.write(out)
    return path


if __name__ == "__main__":
    print(main())
