"""Writes attn_bwd_dkdv_loop.h: the query loop of the dK / dV kernel of the
attention backward (bf16, D = 128) as one inline-asm statement with a fixed
instruction schedule and a fixed register plan.

A wave owns 32 keys of one KV head: their K and V rows and the dK^T / dV^T
accumulators stay in AGPRs. The workgroup's four waves walk one stream of
64-query tiles (every query head of the group, latest tile first) in 32-query
sub-tiles j. With p = exp2(S c - lse2) and dS = p (dP - delta):
  phase A(j): the S = Q K^T and dP = dO V^T MFMAs of sub-tile j+1 (Q and dO
              rows from LDS) with dS of sub-tile j between them;
  phase B(j): dV^T += dO^T P, then dK^T += Q^T dS of sub-tile j (dO^T and
              Q^T tiles from LDS), with p of sub-tile j+1 between them.
Each MFMA thus carries about a third of its shadow in vector work (the exp
is a quarter-rate instruction), and no phase waits on its own arithmetic.
The probabilities use the saved lse ("Sequence Parallelism in Large Language
Models ...", section "The Activation Memory Wall": recomputation instead of
stored activations), so there is no running max; the causal mask is applied
out of line to the sub-tiles from the stream's first partly visible one.

Every LDS operand read goes through one ring of four 4-register slots; the
last four reads of each phase are the next phase's first. The lse2 of sub-tile j+1 is
read during phase A(j), minus its delta (stored negated) during phase B(j-1):
it is the starting accumulator of the dP chain, which so ends at dP - delta. The generator tracks
every LDS read it emits and gives each use the exact lgkmcnt wait it needs
(LDS reads return in order, and the statement issues no other LGKM
operation); one wait serves a pair of MFMAs and sits right after the
previous pair's second MFMA, where the wave could not issue a vector
instruction anyway. It checks the wait states between each MFMA and the
vector instructions that read its result.

LDS holds two row buffers [Q rows | dO rows | lse2 | delta] and two
transposed buffers [Q^T | dO^T], filled by direct global->LDS loads, each
placed after one MFMA of a phase A: the even sub-tile 2t loads the transposed
tile t+1, the odd one the rows (with lse2 / delta) of tile t+2; a tile past
the stream's end repeats the last one. Two barriers per tile:
  even barrier (after MFMA 0 of phase A(2t)): publishes the transposed tile
    t and frees the other transposed buffer (phase B(2t-1) is done);
  odd barrier (after MFMA 12 of phase B(2t)): publishes the rows of tile t+1
    and frees the rows of tile t (both of its phases A and its lse2 / delta
    reads, waited for right before that MFMA, are done); the last four steps
    of phase B(2t) then issue the first reads of tile t+1. (Placed as late as
    the ring allows: the rows loads it waits for get the most time.)
Each barrier follows an MFMA issue, so the matrix pipe has work while the
wave waits.
Each barrier waits only for the loads before the latest batch (vmcnt(8):
every batch gives each wave at least eight loads), so a batch has about two
sub-tiles to land.

Register plan (one wave per SIMD):
  a[0:63] dV^T, a[64:127] dK^T (four 32-wide d tiles of 16 registers each)
  a[128:159] K, a[160:191] V of the wave's keys (eight k-steps of 4)
  v56 rows read address, v57 Q^T read address, v58 lse2 / delta read address,
  v[59:62] temporaries, v[64:79] operand ring
  v[80:95] lse2, v[96:111] minus delta, v[112:127] fp32 p, each of one sub-tile
  v[144:175], v[176:207]: S (16) then dP (16), per parity
  v[208:223], v[224:239]: bf16 P (8) then dS (8), per parity
  v[240:244]: row offsets of the row tile loads
  s[80:81], s[82:83], s[84:85]: global bases of the loads in flight
The compiler keeps everything else in v[0:55], v[245:255], a[192:255] and the
other SGPRs.

Hazards the statement respects by construction: a transcendental result is
read no earlier than the second instruction after it; MFMA results are read
by vector instructions only a phase later, or by the out-of-line mask and
after the statement, each behind s_nop 7 x 3; S and dP accumulate in two
alternating chains, each dV^T / dK^T tile every fourth MFMA; P / dS are
written a phase before the MFMAs that read them and rewritten only after
them; an M0 write is followed by
one wait state (the step's MFMA) before the LDS-DMA load that reads it; an
SALU write of the lane select is four wait states before the v_readlane
that uses it.

Run: python gen_bwd_dkdv_w32.py  (writes the header next to this file)
"""
import os
import re

D = 128
KS = D // 16                # k-steps of the S / dP products
DT = D // 32                # d tiles of dK / dV
ROW = (D // 8 + 1) * 16     # padded Q / dO row, bytes
TROW = 9 * 16               # padded row of a transposed tile (64 queries + pad)
RBUF = 64 * ROW
TBUF = D * TROW
OFF_L = RBUF                # rows buffer: [Q rows | lse2 | dO rows | minus delta],
OFF_DO = RBUF + 1024        # 36 chunks of 1 KiB, nine loaded by each wave
OFF_DL = OFF_DO + RBUF
ROWS_BUF = OFF_DL + 1024
TRANS_BUF = 2 * TBUF        # Q^T, dO^T: 36 chunks, nine per wave
CHUNKS = 9                  # tile loads per wave and batch
assert ROWS_BUF == TRANS_BUF == 4 * CHUNKS * 1024
HALF_R = 32 * ROW           # second 32-query half of a row tile
HALF_T = 64                 # ... of a transposed tile (bytes)
HALF_L = 128                # ... of lse2 / delta (bytes)
N = 2 * KS                  # MFMAs (and operand reads) per phase
assert N == 4 * DT == 16
PF = 4                      # operand reads in flight
NEG_INF = "0xff800000"

DV_, DK_, K_, V_ = 0, 64, 128, 160
V_RADDR, V_TADDR, V_LADDR = 56, 57, 58
T0, T1, T2, T3 = 59, 60, 61, 62
RING, RING2 = 64, 128         # operand ring: slots 0-3 (4-7 if PF = 8)
LX = 80                      # lse2 of the sub-tile whose p is next
DX = 96                      # delta of the sub-tile whose dS is next
P32 = 112                    # fp32 p of that sub-tile
XDL_WAIT = 19                # wait states between an MFMA and a vector read of its result
SD_ = {0: 144, 1: 176}       # S at +0..15, dP at +16..31
PD_ = {0: 208, 1: 224}       # P at +0..7, dS at +8..15
VOFF = 240                   # v[240:248]: row-load offsets (ragged blocks)
SB_A, SB_T, SB_L = 80, 82, 84   # rows (Q / dO), transposed, ninth rows load
PAD = ["s_nop 7", "s_nop 7", "s_nop 7"]
BARRIER_STEP = N - PF        # phase B(2t): the odd barrier follows this MFMA


def vr(base, n):
    return f"v[{base}:{base + n - 1}]"


def ar(base, n):
    return f"a[{base}:{base + n - 1}]"


def ring(i):
    slot = i % PF
    return vr(RING + 4 * slot if slot < 4 else RING2 + 4 * (slot - 4), 4)


def a_off(i):
    """Phase A read i: even = Q row (k-step i/2), odd = dO row."""
    return (i & 1) * OFF_DO + 32 * (i >> 1)


def b_kind(i):
    """Phase B MFMA i: (dK?, 16-query half u, d tile T); the dV MFMAs (both
    halves) come first."""
    return i >= 2 * DT, (i // DT) % 2, i % DT


def b_off(i):
    """Phase B read i: dO^T (dV) or Q^T (dK) rows of d tile T, half u."""
    dk, u, T = b_kind(i)
    return (0 if dk else TBUF) + 32 * T * TROW + 32 * u


class Gen:
    """The statement's lines (in order) and its out-of-line blocks, plus the
    wave's outstanding LDS reads in issue order (they return in order)."""

    def __init__(self):
        self.lines = []
        self.ool = []
        self.q = []          # outstanding reads: (id, tag)
        self.n = 0
        self.ring_id = [None] * PF
        self.lx_id = {}      # register base -> read id of an lse2 / delta read

    def add(self, lines):
        self.lines += lines

    def lab(self, name):
        return f".L{name}_%="

    def place(self, name):
        self.lines.append(f"{self.lab(name)}:")

    def issue(self, tag):
        self.n += 1
        self.q.append((self.n, tag))
        assert len(self.q) <= 15, "more LDS reads in flight than lgkmcnt counts"
        return self.n

    def wait(self, x):
        """s_waitcnt that retires read x (nothing if it already is)."""
        ids = [i for i, _ in self.q]
        if x not in ids:
            return []
        k = len(ids) - 1 - ids.index(x)
        self.q = self.q[ids.index(x) + 1:]
        assert k <= 15
        return [f"s_waitcnt lgkmcnt({k})"]

    def shape(self):
        """The outstanding reads as tags: the loop's entry and back edge
        must agree, since the same waits serve both."""
        return [tag for _, tag in self.q]

    def read(self, slot, addr, off):
        self.ring_id[slot] = self.issue(("ring", slot))
        return [f"ds_read_b128 {ring(slot)}, v{addr} offset:{off}"]

    def lse_read(self, k, half):
        """Read k (0..7) of a sub-tile's lse2 (k < 4, into LX) / delta (into
        DX), four floats: rows 16w + 4m' .. +3 of the sub-tile for k % 4 =
        2w + m' (element e of a lane is register e)."""
        base = (DX if k >= 4 else LX) + 4 * (k % 4)
        off = (OFF_DL if k >= 4 else OFF_L) + [0, 16, 64, 80][k % 4] + (HALF_L if half else 0)
        self.lx_id[base] = self.issue(("lx", base))
        return [f"ds_read_b128 {vr(base, 4)}, v{V_LADDR} offset:{off}"]

    def need_all(self, bases):
        """One wait for the youngest of several lse2 / delta reads."""
        ids = [self.lx_id.pop(b) for b in bases if b in self.lx_id]
        return self.wait(max(ids)) if ids else []

    def need(self, base):
        """Waits before a use of the four registers at base (an lse2 or
        delta read)."""
        x = self.lx_id.pop(base, None)
        return self.wait(x) if x is not None else []

    def phase(self, mfma, addr, off, work=None, pre_in=False, nxt=None, extra=None,
              pre=None, mid=None):
        """N MFMAs; MFMA i reads operand i (address register addr, offset
        off(i)) through the ring. Step i: pre(i), MFMA i, mid(i), the read of
        operand i + PF (the last PF steps issue the first reads of the next phase:
        nxt() gives (addr, off) then, after the extras before it), work(i)
        (instruction strings, or the register base of an lse2 / delta read
        the next ones use) and extra(i)."""
        if not pre_in:
            for i in range(PF):
                self.add(self.read(i, addr, off(i)))
        for i in range(N):
            # one wait serves a pair of MFMAs (an instruction slot is the
            # scarce resource with one wave per SIMD); the pair after this
            # one is waited for right after this pair's second MFMA, where
            # the wave could not issue vector work anyway
            if i % 2 == 0:
                self.add(self.wait(self.ring_id[(i + 1) % PF]))
            else:
                self.add(self.wait(self.ring_id[i % PF]))
            if pre:
                self.add(pre(i))
            self.add([mfma(i)])
            if i % 2 == 1 and (i + 2 < N or nxt):
                self.add(self.wait(self.ring_id[(i + 2) % PF]))
            if mid:
                self.add(mid(i))
            if i + PF < N:
                self.add(self.read(i % PF, addr, off(i + PF)))
            elif nxt:
                a, o = nxt()
                self.add(self.read(i % PF, a, o(i + PF - N)))
            if work:
                for item in work(i):
                    self.add(self.need(item) if isinstance(item, int) else [item])
            if extra:
                self.add(extra(i))


def a_mfma(par):
    """S (even i) and dP (odd i) of parity par, k-step i / 2. S starts from
    0, dP from minus delta (DX), so the chain ends at dP - delta."""
    S, P = SD_[par], SD_[par] + 16

    def f(i):
        s = i >> 1
        dst, b = (P, V_) if i & 1 else (S, K_)
        c = vr(dst, 16) if s else (vr(DX, 16) if i & 1 else "0")
        return f"v_mfma_f32_32x32x16_bf16 {vr(dst, 16)}, {ring(i)}, {ar(b + 4 * s, 4)}, {c}"
    return f


def b_mfma(par):
    """dV^T / dK^T MFMA i (b_kind), from P / dS of parity par."""
    P, dS = PD_[par], PD_[par] + 8

    def f(i):
        dk, u, T = b_kind(i)
        acc, b = (DK_ + 16 * T, dS + 4 * u) if dk else (DV_ + 16 * T, P + 4 * u)
        return f"v_mfma_f32_32x32x16_bf16 {ar(acc, 16)}, {ring(i)}, {vr(b, 4)}, {ar(acc, 16)}"
    return f


def p_pair(par, k):
    """p = exp2(S c - lse2) of elements 2k, 2k+1 of the sub-tile of parity
    par, into P32, in two parts: (fma, fma, exp) and (exp, packing of pair
    k - 1), so both steps of a pair carry a similar share of the issue slots
    (a transcendental result is not read by the next instruction). Element e
    of a lane is query 16(e/8) + 8hh + e%8 of the sub-tile; bf16 pairs pack
    as register 4(e/8) + (e%8)/2."""
    S, e = SD_[par], 2 * k
    first = [LX + 4 * (e // 4),
             f"v_fma_f32 v{P32 + e}, v{S + e}, %[c], -v{LX + e}",
             f"v_fma_f32 v{P32 + e + 1}, v{S + e + 1}, %[c], -v{LX + e + 1}",
             f"v_exp_f32 v{P32 + e}, v{P32 + e}"]
    return first, [f"v_exp_f32 v{P32 + e + 1}, v{P32 + e + 1}"] + ([p_pack(par, k - 1)] if k else [])


def p_pack(par, k):
    e = 2 * k
    return f"v_cvt_pk_bf16_f32 v{PD_[par] + 4 * (e >> 3) + ((e & 7) >> 1)}, v{P32 + e}, v{P32 + e + 1}"


def p_work(par):
    """p of the sub-tile of parity par over the 16 steps of a phase B; the
    last pair's packing is left to the next phase A."""
    def f(i):
        first, second = p_pair(par, i // 2)
        return first if i % 2 == 0 else second
    return f


def ds_work(par):
    """dS = p (dP - delta) of the sub-tile of parity par, bf16, over the 16
    steps of its phase A (dP - delta comes out of the MFMA chain): elements
    2k, 2k+1 after MFMA 2k, their packing after MFMA 2k+1; step 1 also packs
    the last pair of p."""
    dP, dSr = SD_[par] + 16, PD_[par] + 8

    def f(i):
        e = 2 * (i // 2)
        if i % 2 == 0:
            return [f"v_mul_f32 v{T2}, v{P32 + e}, v{dP + e}",
                    f"v_mul_f32 v{T3}, v{P32 + e + 1}, v{dP + e + 1}"]
        return ([p_pack(par, 7)] if i == 1 else []) + [
            f"v_cvt_pk_bf16_f32 v{dSr + 4 * (e >> 3) + ((e & 7) >> 1)}, v{T2}, v{T3}"]
    return f


def mask(G, par, q_sgpr, site):
    """Causal mask of the S of parity par, out of line: the sub-tile's
    index is in %[js], its first query in q_sgpr; a query offset below the
    lane's limit (%[lmin] - q) does not see the lane's key."""
    S = SD_[par]
    G.add(["s_cmp_ge_u32 %[js], %[jfree]", f"s_cbranch_scc1 {G.lab('mask' + site)}"])
    G.place("mback" + site)
    body = [f"{G.lab('mask' + site)}:"] + PAD + [
            f"v_subrev_u32 v{T1}, {q_sgpr}, %[lmin]",
            f"v_mov_b32 v{T0}, {NEG_INF}"]
    for e in range(16):
        k = 16 * (e >> 3) + (e & 7)
        body += [f"v_cmp_lt_i32 vcc, {k}, v{T1}",
                 f"v_cndmask_b32 v{S + e}, v{S + e}, v{T0}, vcc"]
    G.ool += body + [f"s_branch {G.lab('mback' + site)}"]


def tile_loads(sb, vaddr):
    """The nine 1 KiB loads of a wave's share of a tile: its chunks are
    contiguous in LDS, so one M0 value (%[sz] = chunk 4, then %[sz] + 4 KiB
    = chunk 8) and the load's own offset, which moves the global address and
    the LDS destination alike, place loads 0-4 and 5-8. The lane offsets
    vaddr(j) include minus that offset. sb(j): the SGPR pair of load j's
    source. Each is (instructions before the step's MFMA, after it)."""
    g = []
    for j in range(CHUNKS):
        off = (j - 4) * 1024 if j < 5 else (j - 8) * 1024
        pre = ["s_mov_b32 m0, %[sz]"] if j == 0 else (["s_add_u32 m0, %[sz], 4096"] if j == 5 else [])
        b = sb(j)
        g.append((pre, [f"global_load_lds_dwordx4 {vaddr(j)}, s[{b}:{b + 1}] offset:{off}"]))
    return g


# phase A steps of the nine loads, in load order (the M0 change between
# loads 4 and 5 must fall between them): the light (odd) steps first
LOAD_STEPS = [1, 3, 5, 7, 9, 11, 13, 15, 14]


def place_loads(loads):
    at = {LOAD_STEPS[k]: g for k, g in enumerate(loads)}
    return (lambda i: at[i][0] if i in at else []), (lambda i: at[i][1] if i in at else [])


def trans_setup():
    """Source and destination of the transposed tile t+1 (the last one past
    the end): s[SB_T] = this wave's tensor (Q^T or dO^T) at the tile, %[sz] =
    its chunk 4 in the other transposed buffer."""
    return ["s_add_u32 %[sx], %[t], 1", "s_cmp_lt_u32 %[sx], %[nt]",
            "s_cselect_b32 %[sh], %[hn], %[hlast]", "s_cselect_b32 %[sq], %[q0n], %[q0last]",
            "s_mul_i32 %[sx], %[sh], %[qths]", "s_lshl_b32 %[sy], %[sq], 1",
            "s_add_u32 %[sx], %[sx], %[sy]",
            f"s_add_u32 s{SB_T}, %[tb_lo], %[sx]", f"s_addc_u32 s{SB_T + 1}, %[tb_hi], 0",
            f"s_xor_b32 %[sz], %[tb], {TRANS_BUF}", "s_add_u32 %[sz], %[sz], %[tdst]"]


def rows_setup(ragged):
    """Sources and destination of the row tile t+2 (the last one past the
    end), in pieces (one per MFMA after the odd barrier): s[SB_A] = this
    wave's tensor (Q or dO) at the tile, s[SB_L] = its ninth load's (the
    same tensor, or lse2 / minus delta: per-wave head stride %[lhsw] and
    query shift %[shw]), %[sz] = its chunk 4. Ragged blocks: rows past the
    block re-read its last row (their lse2 is +inf), so the lane offsets are
    rebuilt per tile."""
    pieces = [
        ["s_add_u32 %[sx], %[t], 2", "s_cmp_lt_u32 %[sx], %[nt]",
         "s_cselect_b32 %[sh], %[hf], %[hlast]", "s_cselect_b32 %[sq], %[q0f], %[q0last]",
         "s_mul_i32 %[sx], %[sh], %[qhs]", "s_lshl_b32 %[sy], %[sq], 8",
         "s_add_u32 %[sx], %[sx], %[sy]"],
        [f"s_add_u32 s{SB_A}, %[mb_lo], %[sx]", f"s_addc_u32 s{SB_A + 1}, %[mb_hi], 0",
         "s_mul_i32 %[sx], %[sh], %[lhsw]", "s_lshl_b32 %[sy], %[sq], %[shw]",
         "s_add_u32 %[sx], %[sx], %[sy]",
         f"s_add_u32 s{SB_L}, %[lb_lo], %[sx]", f"s_addc_u32 s{SB_L + 1}, %[lb_hi], 0",
         "s_add_u32 %[sz], %[rb], %[rdst]"]]
    if ragged:
        pieces += [["s_sub_u32 %[sx], %[cqm1], %[sq]"] +
                   [f"v_min_u32 v{VOFF + j}, %[sx], %[rv{j}]" for j in range(CHUNKS)],
                   [f"v_lshl_add_u32 v{VOFF + j}, v{VOFF + j}, 8, %[rc{j}]" for j in range(CHUNKS)]]
    return pieces


def advance():
    """Next tile: tile t+1 becomes current, t+2 next, and the tile after
    them (stream order: every head of the group, then the tile row below)
    becomes the far one; the buffers flip. In pieces, one per MFMA."""
    return [
        ["s_add_u32 %[t], %[t], 1", "s_mov_b32 %[q0c], %[q0n]", "s_mov_b32 %[hn], %[hf]",
         "s_mov_b32 %[q0n], %[q0f]"],
        ["s_add_u32 %[hi], %[hi], 1", "s_cmp_eq_u32 %[hi], %[ng]",
         "s_cselect_b32 %[hi], 0, %[hi]", "s_cselect_b32 %[sx], 64, 0",
         "s_sub_u32 %[q0f], %[q0f], %[sx]", "s_nop 3"],
        ["v_readlane_b32 %[hf], %[vhead], %[hi]",
         f"s_xor_b32 %[rb], %[rb], {ROWS_BUF}", f"s_xor_b32 %[tb], %[tb], {TRANS_BUF}"],
    ]


def loop_asm(ragged):
    G = Gen()
    G.add(["s_waitcnt lgkmcnt(0)"] + [f"v_accvgpr_write_b32 a{r}, 0" for r in range(128)])
    LXB = [LX + 4 * m for m in range(4)]
    DXB = [DX + 4 * m for m in range(4)]

    def lx_reads(half):
        """lse2 of a sub-tile: one read at each of steps 1, 3, 5, 7."""
        return lambda i: G.lse_read(i // 2, half) if i % 2 and i < 8 else []

    def dx_reads(half, first):
        """minus delta of a sub-tile: one read at each of steps first..first+3."""
        return lambda i: G.lse_read(4 + i - first, half) if first <= i < first + 4 else []

    def dx_wait(pre=None):
        """Before MFMA 1 (the first dP MFMA, which starts from minus delta):
        wait for the delta reads."""
        return lambda i: (G.need_all(DXB) if i == 1 else []) + (pre(i) if pre else [])

    # prologue: lse2 / delta of sub-tile 0, its S / dP (the last steps start
    # the reads of sub-tile 1; delta of sub-tile 1 is read once the first dP
    # MFMA has taken sub-tile 0's) and its p. V_LADDR stays at the rows
    # buffer of tile t+1 from the middle of sub-tile 2t on.
    G.add([f"v_mov_b32 v{V_RADDR}, %[rbase]", f"v_mov_b32 v{V_LADDR}, %[lbase]",
           f"v_mov_b32 v{V_TADDR}, %[tbase]"])
    for k in range(8):
        G.add(G.lse_read(k, False))
    G.add(G.need_all(LXB + DXB))
    G.phase(a_mfma(0), V_RADDR, a_off, nxt=lambda: (V_RADDR, lambda i: a_off(i) + HALF_R),
            extra=dx_reads(True, 3))
    G.add(PAD + ["s_mov_b32 %[js], 0"])
    mask(G, 0, "%[q0c]", "pro")
    for k in range(8):
        first, second = p_pair(0, k)
        for item in first + ["s_nop 0"] + second + ["s_nop 0"]:
            G.add(G.need(item) if isinstance(item, int) else [item])
    G.add(["s_mov_b32 %[t], 0"] + trans_setup())
    entry = G.shape()
    G.place("loop")

    def work(a, b):
        return lambda i: a(i) + b(i)

    # ================= even sub-tile 2t (tile t, first half)
    pre, post = place_loads(tile_loads(lambda j: SB_T, lambda j: f"%[tv{j}]"))
    # the even barrier right behind MFMA 0, which keeps the matrix pipe busy
    # while the wave waits there
    bar_e = lambda i: [f"s_waitcnt vmcnt({CHUNKS})", "s_barrier"] if i == 0 else []
    # S / dP of sub-tile 2t+1, dS of 2t; lse2 of 2t+1 (this tile's second half)
    G.phase(a_mfma(1), V_RADDR, lambda i: a_off(i) + HALF_R,
            work=work(ds_work(0), lx_reads(True)), pre_in=True,
            nxt=lambda: (V_TADDR, b_off), pre=dx_wait(pre), extra=post, mid=bar_e)
    G.add(["s_add_u32 %[js], %[js], 1", "s_add_u32 %[sq], %[q0c], 32"])
    mask(G, 1, "%[sq]", "e")
    G.add(["s_nop 1",   # wait states before phase B's first read of S
           f"s_xor_b32 %[sx], %[rb], {ROWS_BUF}", f"v_add_u32 v{V_LADDR}, %[sx], %[lbase]"])
    rs = rows_setup(ragged)
    dxr = dx_reads(False, BARRIER_STEP)

    def even_b_pre(i):
        # the rows of tile t are read for the last time: this wave's lse2 /
        # delta reads of them are waited for before the odd barrier
        return G.need_all(LXB + DXB) if i == BARRIER_STEP else []

    def even_b_mid(i):
        # the odd barrier right behind an MFMA; the first reads of tile t+1
        # follow it
        if i != BARRIER_STEP:
            return []
        return [f"s_waitcnt vmcnt({CHUNKS})", "s_barrier", f"s_xor_b32 %[sx], %[rb], {ROWS_BUF}",
                f"v_add_u32 v{V_RADDR}, %[sx], %[rbase]"]

    def even_b_extra(i):
        out = rs[i - BARRIER_STEP] if BARRIER_STEP <= i < BARRIER_STEP + len(rs) else []
        return out + dxr(i)   # delta of sub-tile 2t+2 (tile t+1, just published)
    # dV / dK of sub-tile 2t, p of 2t+1
    G.phase(b_mfma(0), V_TADDR, b_off, work=p_work(1), pre_in=True,
            nxt=lambda: (V_RADDR, a_off), extra=even_b_extra, pre=even_b_pre, mid=even_b_mid)

    # ================= odd sub-tile 2t+1 (tile t, second half)
    pre, post = place_loads(tile_loads(lambda j: SB_L if j == CHUNKS - 1 else SB_A,
                                       (lambda j: f"v{VOFF + j}") if ragged else
                                       (lambda j: f"%[rv{j}]")))
    # S / dP of sub-tile 2t+2, dS of 2t+1; lse2 of 2t+2 (tile t+1, first half)
    G.phase(a_mfma(0), V_RADDR, a_off, work=work(ds_work(1), lx_reads(False)),
            pre_in=True, nxt=lambda: (V_TADDR, lambda i: b_off(i) + HALF_T), pre=dx_wait(pre),
            extra=post)
    G.add(["s_add_u32 %[js], %[js], 1"])
    mask(G, 0, "%[q0n]", "o")
    G.add(["s_nop 3"])   # wait states before phase B's first read of S
    adv = advance()
    ts = trans_setup()
    dxr1 = dx_reads(True, 0)

    def odd_b_extra(i):
        out = dxr1(i)   # delta of sub-tile 2t+3 (tile t+1, second half)
        if 8 <= i < 8 + len(adv):
            out += adv[i - 8]
        if i == 12:  # the last read of the transposed tile t went out earlier
            out += [f"v_add_u32 v{V_TADDR}, %[tb], %[tbase]"] + ts
        return out
    # dV / dK of sub-tile 2t+1, p of 2t+2. V_RADDR stays at tile t+1's rows:
    # the next phase A reads their second half
    G.phase(b_mfma(1), V_TADDR, lambda i: b_off(i) + HALF_T, work=p_work(0), pre_in=True,
            nxt=lambda: (V_RADDR, lambda i: a_off(i) + HALF_R), extra=odd_b_extra)
    assert G.shape() == entry, (G.shape(), entry)
    G.add(["s_cmp_lt_u32 %[t], %[nt]", f"s_cbranch_scc1 {G.lab('loop')}"])
    body = G.lines[G.lines.index(f"{G.lab('loop')}:"):]
    check_hazards(G.lines[:G.lines.index(f"{G.lab('loop')}:")] + body + body)
    # no load or read is left in flight when the statement ends
    G.add(["s_waitcnt vmcnt(0)", "s_waitcnt lgkmcnt(0)", f"s_branch {G.lab('done')}"])
    G.add(G.ool)
    G.place("done")
    G.add(PAD)
    return G.lines


REG = re.compile(r"\bv(\d+)\b|\bv\[(\d+):(\d+)\]")


def regs(text):
    out = set()
    for m in REG.finditer(text):
        if m.group(1):
            out.add(int(m.group(1)))
        else:
            out.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def check_hazards(lines):
    """The straight-line path (prologue, then the loop body twice): every
    vector instruction that reads or writes an MFMA result register is at
    least XDL_WAIT wait states after that MFMA, and no instruction reads a
    transcendental result right after it is written."""
    last = {}       # register -> wait-state index of the MFMA that writes it
    trans = set()   # registers written by the previous instruction, if a transcendental
    ws = 0
    for ln in lines:
        if ln.endswith(":"):
            continue
        op, _, rest = ln.partition(" ")
        if op == "s_nop":
            ws += int(rest) + 1
            trans = set()
            continue
        ops = rest.split(",")
        if op.startswith("v_mfma"):
            for r in regs(",".join(ops[1:3])):   # A, B operands: no result reads
                assert ws - last.get(r, -99) >= XDL_WAIT, ln
            for r in regs(ops[0]):
                last[r] = ws
        elif op.startswith("v_") and not op.startswith("v_accvgpr"):
            used = regs(rest)
            for r in used:
                assert ws - last.get(r, -99) >= XDL_WAIT, (ln, ws - last[r])
            assert not (regs(",".join(ops[1:])) & trans), ln
        trans = regs(ops[0]) if op in ("v_exp_f32",) else set()
        ws += 1


def asm_function(name, ragged):
    lines = loop_asm(ragged)
    outs = ([f'"={{{ar(DV_ + 16 * T, 16)}}}"(dv[{T}])' for T in range(DT)] +
            [f'"={{{ar(DK_ + 16 * T, 16)}}}"(dk[{T}])' for T in range(DT)] +
            ['[t] "=&s"(t)', '[js] "=&s"(js)', '[sx] "=&s"(sx)', '[sy] "=&s"(sy)',
             '[sz] "=&s"(sz)', '[sh] "=&s"(sh)', '[sq] "=&s"(sq)',
             '[q0c] "+s"(q0c)', '[q0n] "+s"(q0n)', '[q0f] "+s"(q0f)', '[hn] "+s"(hn)',
             '[hf] "+s"(hf)', '[hi] "+s"(hi)', '[rb] "+s"(rb)', '[tb] "+s"(tb)'])
    ins = (['[nt] "s"(n_t)', '[jfree] "s"(j_free)', '[ng] "s"(ng)', '[hlast] "s"(h_last)',
            '[q0last] "s"(q0_last)', '[rdst] "s"(rdst)', '[tdst] "s"(tdst)',
            '[qhs] "s"(qhs)', '[qths] "s"(qths)', '[lhsw] "s"(lhsw)', '[shw] "s"(shw)',
            '[c] "s"(c)', '[mb_lo] "s"(mb_lo)', '[mb_hi] "s"(mb_hi)', '[lb_lo] "s"(lb_lo)',
            '[lb_hi] "s"(lb_hi)', '[tb_lo] "s"(tb_lo)', '[tb_hi] "s"(tb_hi)',
            '[rbase] "v"(rbase)', '[tbase] "v"(tbase)', '[lbase] "v"(lbase)', '[lmin] "v"(lmin)',
            '[vhead] "v"(vhead)'] +
           [f'[rv{j}] "v"(rv[{j}])' for j in range(CHUNKS)] +
           [f'[tv{j}] "v"(tv[{j}])' for j in range(CHUNKS)] +
           (['[cqm1] "s"(cq_m1)'] + [f'[rc{j}] "v"(rc[{j}])' for j in range(CHUNKS)]
            if ragged else []) +
           [f'"{{{ar(K_ + 4 * s, 4)}}}"(kr[{s}])' for s in range(KS)] +
           [f'"{{{ar(V_ + 4 * s, 4)}}}"(vr_[{s}])' for s in range(KS)])
    last_v = (VOFF + CHUNKS - 1) if ragged else PD_[1] + 15
    clob = ([f'"v{r}"' for r in range(V_RADDR, last_v + 1)] +
            [f'"s{r}"' for r in range(SB_A, SB_L + 2)] +
            ['"vcc"', '"scc"', '"m0"', '"memory"'])
    body = "\n".join(f'      "{ln}\\n\\t"' for ln in lines)
    return f'''__device__ __forceinline__ void {name}(
    int n_t, int j_free, int ng, int h_last, int q0_last, int cq_m1, unsigned rdst, unsigned tdst,
    unsigned qhs, unsigned qths, unsigned lhsw, unsigned shw, float c, const void* mb,
    const void* lb, const void* tbp, unsigned rbase, unsigned tbase, unsigned lbase, int lmin,
    int vhead, const unsigned (&rv)[{CHUNKS}], const unsigned (&rc)[{CHUNKS}],
    const unsigned (&tv)[{CHUNKS}], const bf16x8 (&kr)[8], const bf16x8 (&vr_)[8], int q0c,
    int q0n, int q0f, int hn, int hf, int hi, floatx16 (&dv)[4], floatx16 (&dk)[4]) {{
  int t, js, sx, sy, sz, sh, sq;
  int rb = 0, tb = 0;
  const unsigned mb_lo = lo32(mb), mb_hi = hi32(mb), lb_lo = lo32(lb), lb_hi = hi32(lb);
  const unsigned tb_lo = lo32(tbp), tb_hi = hi32(tbp);
  asm volatile(
{body}
      : {", ".join(outs)}
      : {", ".join(ins)}
      : {", ".join(clob)});
}}
'''


def main():
    out = f'''// Generated by gen_bwd_dkdv_w32.py -- do not edit by hand.
//
// The query loop of attn_bwd_dkdv_w32 (D = {D}) as one inline-asm statement
// with a fixed schedule and fixed registers; gen_bwd_dkdv_w32.py documents
// the register plan, the schedule and the hazards it respects.
#pragma once

namespace ra {{
namespace dkdvw {{

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// A rows buffer is [Q rows | lse2 | dO rows | minus delta] (lse2 and minus
// delta: 1 KiB each, the first 256 bytes used), a transposed buffer [Q^T |
// dO^T]; two of each. A wave loads nine contiguous 1 KiB chunks of each.
constexpr int kRowsBuf = {ROWS_BUF};
constexpr int kTransBuf = {TRANS_BUF};
constexpr int kOffL = {OFF_L};
constexpr int kOffDO = {OFF_DO};
constexpr int kOffDL = {OFF_DL};
constexpr int kChunks = {CHUNKS};

__device__ __forceinline__ unsigned lo32(const void* p) {{
  return (unsigned)(unsigned long long)(size_t)p;
}}
__device__ __forceinline__ unsigned hi32(const void* p) {{
  return (unsigned)((unsigned long long)(size_t)p >> 32);
}}

// The query-tile stream of one wave: n_t >= 1 tiles of 64 queries. The rows
// (with lse2 / minus delta) of tiles 0 and min(1, n_t - 1) are in rows
// buffers 0 and 1, the transposed tile 0 in transposed buffer 0. Tile T is
// query head lane (T % ng) of vhead, first query q0(T) (the tiles of each
// query range for every head, ranges from the last down); the caller passes
// q0 of tiles 0, 1, 2 (q0c, q0n, q0f), the heads of tiles 1, 2 (hn, hf), hi
// = 2 % ng, and head and q0 of the last tile (h_last, q0_last). rbase /
// tbase / lbase: this lane's read addresses in rows / transposed / lse2 of
// buffer 0; rdst / tdst: this wave's chunk 4 in rows / transposed buffer 0.
// mb: the batch base of this wave's rows tensor (q for waves 0 and 1, dout
// for 2 and 3); lb: of its ninth rows load (q, lse2, dout, minus delta by
// wave), lhsw / shw that one's head stride (bytes) and query shift; tbp: of
// its transposed tensor (q^T, q^T, dout^T, dout^T); qhs / qths: head strides
// of q / dout and of q^T / dout^T in bytes. rv / tv: the lane's byte offset
// of each of its nine rows / transposed loads within the tile, minus the
// load's own offset; in the ragged form rv holds the rows and rc the byte
// offsets within the row (minus the same), and rows are clamped to cq_m1,
// the block's last one. j_free: the first sub-tile that needs the causal
// mask; lmin: the first row that sees the lane's key, minus 8 for the upper
// half of the wave. Returns dV^T and dK^T (unscaled).
{asm_function("dkdv_loop", False)}
{asm_function("dkdv_loop_ragged", True)}
}}  // namespace dkdvw
}}  // namespace ra
'''
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "attn_bwd_dkdv_loop.h")
    with open(path, "w") as f:
        f.write(out)
    return path


if __name__ == "__main__":
    print(main())
