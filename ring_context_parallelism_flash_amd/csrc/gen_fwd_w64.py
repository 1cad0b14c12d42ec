"""Writes attn_fwd_w64_phases.h: the key-tile loop of the one-wave-per-SIMD
bf16 forward kernel (D = 128) as one inline-asm statement with a fixed
instruction schedule and a fixed register plan.

A wave owns 64 query rows in two 32-row blocks. Each iteration (key tile t)
runs two phases. Phase A issues the 32 score MFMAs of tile t+1 (each K
operand read from LDS feeds the MFMA of both blocks) with the softmax of
block 1 of tile t between them; phase B issues the 32 P*V MFMAs of tile t
(each V^T read feeds both blocks) with the softmax of block 0 of tile t+1
between them. Every MFMA is followed by part of one step's vector work, so
the wave's vector and LDS instructions issue while its matrix pipe runs, and
the last pairs of each phase already issue the first operand reads of the
next one, so no phase starts by waiting for LDS.

Tiles reach LDS through direct global->LDS loads: K tiles rotate through
three buffers, V^T tiles through two. One barrier per iteration publishes
the loads of the previous iteration and frees the buffers it refills; the
ten loads of a wave (five contiguous 1 KiB chunks of K tile t+3, five of
V^T tile t+1, each five placed from one M0 by the instructions' offsets; the
waves' ranges overlap on a few chunks, loaded twice with the same data) are
then spread over the first ten MFMA pairs of phase A, where their issue
overlaps the matrix pipe instead of stalling all four waves at once behind
the barrier. A K tile past the last one repeats the last one (into a buffer
nobody reads), so no wave branches around its loads.

Online softmax with a lazy reference (the pages' running max / sum /
rescaled output, "Algorithmic Mechanics"): probabilities are taken against a
per-row reference m that moves only when a lane's probabilities of one tile
sum past 2^8 (or it has none yet); then the row max is taken, O and l are
rescaled by exp2((m_old - m_new) * c) and the tile's probabilities redone.
l and O always share the reference, so the result is the same. A row with
no reference yet (m = -inf) takes exponent offset -m*c = +inf on the common
path, so its probabilities come out +inf (or NaN where masked) and the sum
test alone sends it to the slow path, which redoes the tile with offset 0
for such rows (their p are then exp2 of -inf scores: 0). That slow path and
the causal mask (tiles from the wave's first partly visible one) are placed
out of line, so the common path has no taken branch but the loop's back
edge.

With one wave per SIMD the wave's own instruction issue sets the pace (an
MFMA pair of the common path takes about as long as the two MFMAs, one
softmax pair and its operand read take to issue; after an MFMA the wave
issues no vector instruction for about 12 cycles, other instructions after
about 8), so the common path keeps vector instructions out: one running row
sum started by a move, one offset instruction per phase, a four-instruction
sum test; each pair's LDS wait sits right after the previous pair's first
MFMA, where it costs no vector issue slot.

Register plan (one wave per SIMD: 256 VGPRs + 256 AGPRs):
  a[0:63]    O of block 0, four 32-wide d tiles of 16 registers (O^T layout)
  a[64:127]  O of block 1
  a[128:159] Q of block 0, eight k-steps of 4 registers (bf16x8)
  a[160:191] Q of block 1
  v52 m0, v53 l0, v54 m1, v55 l1: reference and running sum of each block
  v57 K read address, v58 minus the exponent offset of the block in hand,
  v59 V^T read address, v[60:61] temporaries, v62 the tile's row sum,
  v63 the slow path's exponent offset
  v[64:79]   LDS operand ring, four 16-byte reads in flight
  v[80:95]   P0a  bf16 probabilities of block 0 (tile parity 0)
  v[96:111]  P0b  (tile parity 1)
  v[112:127] P1   bf16 probabilities of block 1
  v[128:159] SA0  scores of block 0, two 32-key halves of 16 registers
  v[160:191] SA1  scores of block 1
  v[192:223] SB0, v[224:255] SB1: the other score buffer pair
  s[80:81], s[82:83]: global addresses of the next K and V^T tiles
The compiler keeps everything else (the load offsets, the lane addresses,
its own values) in v[0:51], v56, a[192:255] and the other SGPRs.

Hazards the statement respects by construction, and check_hazards verifies
on the executed paths (the common path for several trip counts, and paths
through each out-of-line branch) before the header is written: a
transcendental result is read no earlier than the second instruction after
it; an MFMA result is read by a vector instruction only after at least 19
wait states (phase A's scores are first read two MFMA pairs into phase B,
or by the out-of-line mask, which starts with s_nop 7 x 3; O is read only by
the out-of-line slow path, which starts the same way, and after the
statement, which ends with the same pad); an M0 write is not directly
followed by the LDS-DMA load that reads it; an MFMA operand read from LDS
has returned when the MFMA issues (LDS reads return in order; lgkmcnt
counts them, and no other LGKM operation is in flight on the common path).
An MFMA accumulator is reused no sooner than three MFMAs later.

Run: python gen_fwd_w64.py  (writes the header next to this file)
"""
import os
import re

D = 128
KS = D // 16           # score k-steps
DT = D // 32           # output d tiles
KROW = (D // 8 + 1) * 16   # padded K row in LDS, bytes
VROW = 9 * 16              # padded V^T row in LDS, bytes
KBUF, VBUF = 64 * KROW, D * VROW   # bytes per K / V^T tile buffer
KBUFS = 3              # K tile buffers (V^T: two)
N = 16                 # operand reads per phase (2*KS score reads, 4*DT P*V reads)
PF = 4                 # reads in flight
assert 2 * KS == N and 4 * DT == N
FAST_SUM = 256.0       # 2^8: the lazy-rescale bound on a lane's tile sum
NEG_INF = "0xff800000"

O_ = (0, 64)                     # O of block 0 / 1 (AGPR base)
Q_ = (128, 160)                  # Q of block 0 / 1 (AGPR base)
M_ = (52, 54)
L_ = (53, 55)
V_KADDR, V_NMOFF, V_VADDR = 57, 58, 59
T0, T1, T2, T3 = 60, 61, 62, 63
RING = 64
P0A, P0B, P1 = 80, 96, 112
SA0, SA1, SB0, SB1 = 128, 160, 192, 224
PAD = ["s_nop 7", "s_nop 7", "s_nop 7"]   # 24 wait states after an MFMA
KG_S, VG_S = 80, 82              # SGPR pairs of the global K / V^T tile addresses


def vr(base, n):
    return f"v[{base}:{base + n - 1}]"


def ar(base, n):
    return f"a[{base}:{base + n - 1}]"


def ring(i):
    return vr(RING + 4 * (i % PF), 4)


def elem(S, e):
    """VGPR of probability element e (= 8u + j of P[u]) of a 32-score block."""
    u, j = e >> 3, e & 7
    return S + 16 * (u >> 1) + 8 * (u & 1) + j


def nmoff_lines(m, dst):
    """dst = -m * c, or 0 where m = -inf (the slow path's redo: a row with no
    visible key yet gets p = 0 from its -inf scores)."""
    return [f"v_mul_f32 v{dst}, %[c], v{m}",
            f"v_sub_f32 v{dst}, 0, v{dst}",
            f"v_cmp_class_f32_e64 vcc, v{m}, 4",
            f"v_cndmask_b32_e64 v{dst}, v{dst}, 0, vcc"]


def fast_off(m):
    """The common path's exponent offset: v58 = -m * c, which is +inf where m
    = -inf, so a row without a reference gets +inf (or NaN) probabilities
    and fails the sum test below."""
    return [f"v_mul_f32_e64 v{V_NMOFF}, -%[c], v{m}"]


def softmax_pair(i, S, P, nm=V_NMOFF):
    """Vector work for scores e = 2i, 2i+1 in two parts, one after each MFMA
    of a pair: the exponentials, then the row sum (v62, started by the first
    pair) and the bf16 packing."""
    s0 = elem(S, 2 * i)
    u, j = (2 * i) >> 3, (2 * i) & 7
    first = [f"v_fma_f32 v{T0}, v{s0}, %[c], v{nm}",
             f"v_fma_f32 v{T1}, v{s0 + 1}, %[c], v{nm}",
             f"v_exp_f32 v{T0}, v{T0}",
             f"v_exp_f32 v{T1}, v{T1}"]
    second = [f"v_mov_b32 v{T2}, v{T0}" if i == 0 else f"v_add_f32 v{T2}, v{T2}, v{T0}",
              f"v_cvt_pk_bf16_f32 v{P + 4 * u + j // 2}, v{T0}, v{T1}",
              f"v_add_f32 v{T2}, v{T2}, v{T1}"]
    return first, second


def score_off(i):
    return (i % 2) * 32 * KROW + (i // 2) * 32


def pv_off(i):
    return (i % DT) * 32 * VROW + (i // DT) * 32


def phase(mfmas, addr, off, work, pre_in=False, nxt=None, extra=()):
    """16 MFMA pairs; pair i reads one LDS operand (address register `addr`,
    byte offset off(i)) through the read ring. `work` = (S, P, block): the
    softmax of S between the MFMAs. pre_in: the first PF reads were issued
    by the previous phase; nxt = (addr, off): issue the first PF reads of
    the next phase in the last PF pairs (LDS reads return in order, so every
    pair waits until at most PF - 1 reads are outstanding); extra[i]: more
    instructions after pair i."""
    lines = [] if pre_in else ["s_waitcnt lgkmcnt(0)"]
    if work:
        lines += fast_off(M_[work[2]])
    if not pre_in:
        for i in range(PF):
            lines.append(f"ds_read_b128 {ring(i)}, v{addr} offset:{off(i)}")
    for i in range(N):
        # reads 0 .. issued-1 are in flight or done, in order. Pair 0 waits
        # for its read before its first MFMA; every other pair's read is
        # waited for right after the previous pair's first MFMA, in the
        # slot where the wave could not issue vector work anyway
        issued = i + PF if nxt else min(N, i + PF)
        if i == 0:
            lines.append(f"s_waitcnt lgkmcnt({issued - 1})")
        first, second = softmax_pair(i, work[0], work[1]) if work else ([], [])
        ma, mb = mfmas(i)
        lines += [ma]
        if i + 1 < N:
            lines.append(f"s_waitcnt lgkmcnt({issued - (i + 2)})")
        lines += first + [mb]
        if i + PF < N:
            lines.append(f"ds_read_b128 {ring(i)}, v{addr} offset:{off(i + PF)}")
        elif nxt:
            lines.append(f"ds_read_b128 {ring(i)}, v{nxt[0]} offset:{nxt[1](i + PF - N)}")
        lines += second
        if i < len(extra):
            lines += extra[i]
    return lines


def score_mfmas(S0, S1):
    """Pair i: half h = i % 2 (32 keys) at k-step s = i // 2, block 0 then 1."""
    def f(i):
        h, s = i % 2, i // 2
        c0 = "0" if s == 0 else vr(S0 + 16 * h, 16)
        c1 = "0" if s == 0 else vr(S1 + 16 * h, 16)
        return (f"v_mfma_f32_32x32x16_bf16 {vr(S0 + 16 * h, 16)}, {ring(i)}, "
                f"{ar(Q_[0] + 4 * s, 4)}, {c0}",
                f"v_mfma_f32_32x32x16_bf16 {vr(S1 + 16 * h, 16)}, {ring(i)}, "
                f"{ar(Q_[1] + 4 * s, 4)}, {c1}")
    return f


def pv_mfmas(P0, P1_):
    """Pair i: d tile T = i % DT, probability k-step u = i // DT."""
    def f(i):
        u, T = i // DT, i % DT
        return (f"v_mfma_f32_32x32x16_bf16 {ar(O_[0] + 16 * T, 16)}, {ring(i)}, "
                f"{vr(P0 + 4 * u, 4)}, {ar(O_[0] + 16 * T, 16)}",
                f"v_mfma_f32_32x32x16_bf16 {ar(O_[1] + 16 * T, 16)}, {ring(i)}, "
                f"{vr(P1_ + 4 * u, 4)}, {ar(O_[1] + 16 * T, 16)}")
    return f


LOOP_CLOBBER = ([f'"v{r}"' for r in range(V_KADDR, 256)] +
                ['"vcc"', '"scc"', '"m0"', '"exec"', '"memory"'])


class Loop:
    """The whole key-tile loop as one asm statement. Rarely taken code (the
    slow path, the causal mask) is placed out of line after the loop, so the
    common path runs without taken branches."""

    def __init__(self):
        self.lines = []
        self.ool = []

    def add(self, lines):
        self.lines += lines

    def lab(self, name):
        return f".L{name}_%="

    def place(self, name):
        self.lines.append(f"{self.lab(name)}:")

    def set_addr(self, reg, reg_operand, const):
        self.lines.append(f"v_add_u32 v{reg}, {const}, {reg_operand}")

    def check_and_slow(self, b, S, P, site):
        """Row sum check of block b; the fast path adds it to l, the slow
        path (out of line) redoes the tile's softmax."""
        m, l = M_[b], L_[b]
        # (a row without a reference has +inf or NaN probabilities and fails)
        self.add([f"v_cmp_ge_f32 vcc, {FAST_SUM}, v{T2}",
                  "s_cmp_eq_u64 vcc, exec",
                  f"s_cbranch_scc0 {self.lab('slow' + site)}",
                  f"v_add_f32 v{l}, v{l}, v{T2}"])
        self.place("cont" + site)
        self.ool += [f"{self.lab('slow' + site)}:"] + PAD
        self.ool += slow_path_body(S, P, b, self.lab("keep" + site))
        self.ool += [f"s_branch {self.lab('cont' + site)}"]

    def mask(self, S0, S1, kt_sgpr, site, cond):
        """Causal mask of the tile whose index is in kt_sgpr, on both blocks,
        out of line; `cond` = instructions leaving SCC = 1 when it is needed."""
        self.add(cond + [f"s_cbranch_scc1 {self.lab('mask' + site)}"])
        self.place("mback" + site)
        body = [f"{self.lab('mask' + site)}:"] + PAD + [
                f"s_lshl_b32 %[sx], {kt_sgpr}, 6",
                f"v_subrev_u32 v{T1}, %[sx], %[nal0]",
                f"v_subrev_u32 v{T2}, %[sx], %[nal1]",
                f"v_mov_b32 v{T0}, {NEG_INF}"]
        for S, lim in ((S0, T1), (S1, T2)):
            for t in range(2):
                for i in range(16):
                    k = 32 * t + 16 * (i >> 3) + (i & 7)
                    r = S + 16 * t + i
                    body += [f"v_cmp_lt_i32 vcc, {k}, v{lim}",
                             f"v_cndmask_b32 v{r}, v{T0}, v{r}, vcc"]
        self.ool += body + [f"s_branch {self.lab('mback' + site)}"]


def slow_path_body(S, P, b, keep_label):
    """Row max of S; where it exceeds the reference, O and l of block b are
    scaled by exp2((m - m_new) c) and m moves up; then P and the row sum are
    redone from S against the reference and l += sum. The O rescale uses P
    (about to be redone) as temporaries: the operand ring may hold reads of
    the next phase."""
    m, l, Ob = M_[b], L_[b], O_[b]
    regs = [elem(S, e) for e in range(32)]
    lines = [f"v_max_f32 v{T0}, v{regs[0]}, v{regs[1]}",
             f"v_max_f32 v{T1}, v{regs[2]}, v{regs[3]}"]
    for k in range(4, 32, 2):
        t = T0 if (k // 2) % 2 == 0 else T1
        lines.append(f"v_max3_f32 v{t}, v{t}, v{regs[k]}, v{regs[k + 1]}")
    lines += [f"v_max_f32 v{T0}, v{T0}, v{T1}",
              f"ds_bpermute_b32 v{T1}, %[perm], v{T0}",
              "s_waitcnt lgkmcnt(0)",
              f"v_max_f32 v{T0}, v{T0}, v{T1}",            # row max (both lane halves)
              f"v_cmp_gt_f32 vcc, v{T0}, v{m}",             # grow
              "s_cmp_eq_u64 vcc, 0",
              f"s_cbranch_scc1 {keep_label}",
              f"v_cndmask_b32 v{T1}, v{m}, v{T0}, vcc",     # m_new
              f"v_sub_f32 v{T2}, v{m}, v{T1}",
              f"v_mul_f32 v{T2}, %[c], v{T2}",
              f"v_exp_f32 v{T2}, v{T2}",
              "s_nop 1",
              f"v_cndmask_b32_e64 v{T2}, 1.0, v{T2}, vcc",   # alpha
              f"v_mov_b32 v{m}, v{T1}",
              f"v_mul_f32 v{l}, v{l}, v{T2}"]
    for r in range(64):
        t = P + (r % 8)
        lines += [f"v_accvgpr_read_b32 v{t}, a{Ob + r}",
                  f"v_mul_f32 v{t}, v{t}, v{T2}",
                  f"v_accvgpr_write_b32 a{Ob + r}, v{t}"]
    lines.append(f"{keep_label}:")
    # the redo takes offset 0 where m is still -inf (no key of the row
    # visible yet: every p is 0)
    lines += nmoff_lines(m, T3)
    for i in range(16):
        first, second = softmax_pair(i, S, P, T3)
        lines += first + second
    lines += [f"v_add_f32 v{l}, v{l}, v{T2}"]
    return lines


def rotate(sreg):
    """Next K buffer offset: + KBUF, wrapping after the last buffer."""
    return [f"s_add_u32 {sreg}, {sreg}, {KBUF}", f"s_cmp_eq_u32 {sreg}, {KBUFS * KBUF}",
            f"s_cselect_b32 {sreg}, 0, {sreg}"]


def loads(L, p):
    """Barrier, then the tile loads of iteration t (parity p) as groups for
    the MFMA pairs of phase A: K(min(t+3, n_kt-1)) into K buffer %[kw] and
    V(t+1) into V^T buffer 1-p; the global tile addresses advance after them.
    Every wave loads five contiguous 1 KiB chunks of each tile (the four
    waves' chunk ranges overlap on a few chunks, loaded twice with the same
    data), all placed from one M0 value by the instructions' own offsets."""
    L.add(["s_waitcnt vmcnt(0)", "s_barrier", "s_add_u32 m0, %[kdst], %[kw]"] + rotate("%[kw]"))
    groups = []
    for j in range(5):
        groups.append([f"global_load_lds_dwordx4 %[ko{j}], %[kg] offset:{(j - 4) * 1024}"])
    groups[4].append(f"s_add_u32 m0, %[vdst], {(1 - p) * VBUF}")
    for j in range(5):
        groups.append([f"global_load_lds_dwordx4 %[vo{j}], %[vg] offset:{(j - 4) * 1024}"])
    groups[9] += [
                   # the next K tile, t+4, if it exists; else the last one again
                   f"s_add_u32 %[sx], %[t], {KBUFS + 1}", "s_cmp_lt_u32 %[sx], %[nkt]",
                   f"s_cselect_b32 %[sx], {64 * D * 2}, 0",
                   f"s_add_u32 s{KG_S}, s{KG_S}, %[sx]", f"s_addc_u32 s{KG_S + 1}, s{KG_S + 1}, 0",
                   f"s_add_u32 s{VG_S}, s{VG_S}, 128", f"s_addc_u32 s{VG_S + 1}, s{VG_S + 1}, 0"]
    return groups


def loop_asm():
    S = {0: (SA0, SA1, SB0, SB1), 1: (SB0, SB1, SA0, SA1)}
    P0 = {0: (P0A, P0B), 1: (P0B, P0A)}
    L = Loop()
    L.add([f"v_accvgpr_write_b32 a{O_[b] + r}, 0" for b in (0, 1) for r in range(64)])
    # prologue: scores of tile 0 (K buffer 0), whose last pairs start the
    # reads of tile 1 (K buffer 1); mask; block 0 softmax
    L.set_addr(V_KADDR, "%[krb]", 0)
    L.set_addr(V_VADDR, "%[krb]", KBUF)
    L.add(phase(score_mfmas(SA0, SA1), V_KADDR, score_off, None, nxt=(V_VADDR, score_off)) + PAD)
    L.set_addr(V_KADDR, "%[krb]", KBUF)
    L.add(["s_mov_b32 %[t], 0"])
    L.mask(SA0, SA1, "%[t]", "pro", ["s_cmp_eq_u32 %[fmask], 0"])
    L.add(fast_off(M_[0]))
    for i in range(16):
        first, second = softmax_pair(i, SA0, P0A)
        L.add(first + second)
    L.check_and_slow(0, SA0, P0A, "pro")
    L.add(["s_mov_b32 %[t], 0"])
    L.place("loop")
    for p in (0, 1):
        c0, c1, n0, n1 = S[p]
        pc, pn = P0[p]
        # t + 1 < n_kt, else the last tile of this parity
        L.add(["s_add_u32 %[t1], %[t], 1", "s_cmp_ge_u32 %[t1], %[nkt]",
               f"s_cbranch_scc1 {L.lab(f'last{p}')}"])
        groups = loads(L, p)
        L.set_addr(V_VADDR, "%[vrb]", p * VBUF)
        L.add(phase(score_mfmas(n0, n1), V_KADDR, score_off, (c1, P1, 1), pre_in=True,
                    nxt=(V_VADDR, pv_off), extra=groups))
        L.check_and_slow(1, c1, P1, f"a{p}")
        L.mask(n0, n1, "%[t1]", f"{p}", ["s_cmp_ge_u32 %[t1], %[fmask]"])
        # K tile t+2 (buffer %[kr]) for the reads started at the end of phase B
        L.add([f"v_add_u32 v{V_KADDR}, %[kr], %[krb]"] + rotate("%[kr]"))
        L.add(phase(pv_mfmas(pc, P1), V_VADDR, pv_off, (n0, pn, 0), pre_in=True,
                    nxt=(V_KADDR, score_off)))
        L.check_and_slow(0, n0, pn, f"b{p}")
        L.add(["s_mov_b32 %[t], %[t1]"])
    L.add([f"s_branch {L.lab('loop')}"])
    for p in (0, 1):
        c0, c1, n0, n1 = S[p]
        pc, pn = P0[p]
        L.place(f"last{p}")
        L.add(["s_waitcnt vmcnt(0)", "s_barrier", "s_waitcnt lgkmcnt(0)"] + fast_off(M_[1]))
        for i in range(16):
            first, second = softmax_pair(i, c1, P1)
            L.add(first + second)
        L.check_and_slow(1, c1, P1, f"l{p}")
        L.set_addr(V_VADDR, "%[vrb]", p * VBUF)
        L.add(phase(pv_mfmas(pc, P1), V_VADDR, pv_off, None))
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


def trace(lines, policy, limit=20000):
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
    """Along one executed path: a vector access of an MFMA result is at least
    XDL_WAIT wait states after the MFMA; no instruction reads a
    transcendental result right after it; an M0 write is not followed
    directly by an LDS-DMA load; every MFMA operand read from LDS has
    returned (LDS reads return in order) at the MFMA."""
    last, trans, ws = {}, set(), 0
    pending = []          # destination register sets of LDS reads in flight, oldest first
    prev = ""
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
            src = regs(",".join(ops[1:]))
            for r in src:
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
    """check_trace over paths through the loop: the common path for several
    trip counts, and paths that take each out-of-line branch."""
    for n_it in range(0, 4):
        for lastp in (0, 1):
            def pol(lab, k, n_it=n_it, lastp=lastp, extra=None):
                if lab.startswith(".Llast"):
                    return lab == f".Llast{lastp}_%=" and k >= n_it
                return False
            check_trace(trace(lines, pol))
    fams = ["slowpro", "maskpro", "slowa0", "slowb0", "slowa1", "slowb1", "mask0", "mask1",
            "slowl0", "slowl1", "keeppro", "keepa0", "keepb0", "keepa1", "keepb1", "keepl0", "keepl1"]
    for fam in fams:
        for when in (0, 1):
            def pol(lab, k, fam=fam, when=when):
                if lab.startswith(".Llast"):
                    return lab == ".Llast1_%=" and k >= 2
                return lab == f".L{fam}_%=" and k == when
            check_trace(trace(lines, pol))


def main():
    out = [f'''// Generated by gen_fwd_w64.py -- do not edit by hand.
//
// The key-tile loop of attn_fwd_bf16_w64 (D = {D}) as one inline-asm
// statement with a fixed schedule and fixed registers; gen_fwd_w64.py
// documents the register plan, the schedule and the hazards it respects.
#pragma once

namespace ra {{
namespace w64 {{

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// LDS buffers of K tiles the loop rotates through.
constexpr int kKBufs = {KBUFS};
''']
    lines = loop_asm()
    check_hazards(lines)
    outs = ([f'"={{{ar(O_[b] + 16 * T, 16)}}}"(o{b}[{T}])' for b in (0, 1) for T in range(DT)] +
            [f'"+{{v{M_[b]}}}"(m{b})' for b in (0, 1)] +
            [f'"+{{v{L_[b]}}}"(l{b})' for b in (0, 1)] +
            ['[t] "=&s"(t)', '[t1] "=&s"(t1)', '[sx] "=&s"(sx)', '[stmp] "=&s"(stmp)',
             f'[kg] "+{{s[{KG_S}:{KG_S + 1}]}}"(kgv)', f'[vg] "+{{s[{VG_S}:{VG_S + 1}]}}"(vgv)',
             '[kw] "+s"(kw)', '[kr] "+s"(kr)'])
    ins = (['[nkt] "s"(n_kt)', '[fmask] "s"(first_mask)', '[kdst] "s"(kdst)',
            '[vdst] "s"(vdst)', '[c] "s"(c)',
            '[krb] "v"(krb)', '[vrb] "v"(vrb)', '[nal0] "v"(nal0)', '[nal1] "v"(nal1)',
            '[perm] "v"(perm)'] +
           [f'[ko{j}] "v"(koff[{j}])' for j in range(5)] +
           [f'[vo{j}] "v"(voff[{j}])' for j in range(5)] +
           [f'"{{{ar(Q_[0] + 4 * s, 4)}}}"(q0[{s}])' for s in range(KS)] +
           [f'"{{{ar(Q_[1] + 4 * s, 4)}}}"(q1[{s}])' for s in range(KS)])
    body = "\n".join(f'      "{ln}\\n\\t"' for ln in lines)
    out.append(f"""// The key-tile loop of one wave: n_kt >= 1 tiles; K tiles 0 .. kKBufs-1
// (those the block has) are in K buffers 0 .. kKBufs-1 and V^T tile 0 in
// V^T buffer 0. krb / vrb: this lane's operand read address in K buffer 0 /
// V^T buffer 0; kdst / vdst: the LDS address of the last of this wave's five
// chunks in K / V^T buffer 0 (the M0 of its loads); kg: global address of K
// tile min(kKBufs, n_kt - 1), vg: of V^T tile 1 (both advanced by the loop);
// koff / voff: the lane's byte offsets in a tile of its five chunks, load j
// plus (4 - j) KiB (the loads' instruction offsets take that off); first_mask: first
// tile needing the causal mask; nal0 / nal1: keys visible to the lane's row
// of block 0 / 1, minus 8 for the upper half of the wave; perm: byte address
// of lane ^ 32. Returns O, m and l of both blocks (O^T layout, exponent
// reference m, sum l).
__device__ __forceinline__ void attn_loop(
    int n_kt, int first_mask, unsigned kdst, unsigned vdst, float c,
    unsigned krb, unsigned vrb, int nal0, int nal1, unsigned perm, const void* kg,
    const void* vg, const unsigned (&koff)[5], const unsigned (&voff)[5],
    const bf16x8 (&q0)[8], const bf16x8 (&q1)[8], floatx16 (&o0)[4], floatx16 (&o1)[4],
    float& m0, float& l0, float& m1, float& l1) {{
  int t, t1, sx;
  long long stmp;
  unsigned long long kgv = (unsigned long long)(size_t)kg, vgv = (unsigned long long)(size_t)vg;
  unsigned kw = 0, kr = {(KBUFS - 1) * KBUF};  // K buffer offsets: next load, next prefetch
  asm volatile(
{body}
      : {", ".join(outs)}
      : {", ".join(ins)}
      : {", ".join(LOOP_CLOBBER)});
}}
""")
    out.append("}  // namespace w64\n}  // namespace ra\n")
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "attn_fwd_w64_phases.h")
    with open(path, "w") as f:
        f.write("\n".join(out))
    return path


if __name__ == "__main__":
    print(main())
