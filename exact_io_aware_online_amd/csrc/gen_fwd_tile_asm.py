"""Generates fa_fwd_tile_asm.h: the hand-scheduled tile body of the 64-row
prefill shape (head dim 128, 64-key tiles, one wavefront per SIMD, two
32-row query blocks A and B per wavefront).

Run from this directory: ``python gen_fwd_tile_asm.py`` (the header is
committed; a CPU test checks that it matches this script's output).

Why assembly. Each wavefront owns 64 query rows, so every K and V^T operand
read from LDS feeds two MFMAs (half the LDS bytes per flop of the 32-row
shape), but the state needs about 450 registers and leaves one wavefront per
SIMD: the wavefront must overlap its own softmax with its own MFMAs. One
tile runs as four phases of 16 MFMAs each (S^T = K Q^T, then O^T += V^T P^T,
FlashAttention: Part 2, section 6.2), the vector work of the other block
interleaved one MFMA at a time (section 1.5: overlap the softmax of one part
of the work with the matrix products of another):

  1. S_A = K Q_A^T                  (K operands read in the previous tile)
  2. S_B = K Q_B^T   | softmax of A, V^T operands read from LDS
  3. O_A += V^T P_A^T | row sum of A, softmax of B
     wait for the next tile's loads, barrier, next-but-one tile's loads issued
  4. O_B += V^T P_B^T | row sum of B, next tile's K operands read

Register map (fixed; no compiled code between these statements uses these
registers, which a CPU test checks on the compiled kernel):
  a[0:63]    O^T of block A (four 32-row d blocks of 16), a[64:127] block B
  a[128:159] Q^T operands of A (eight k-steps of 4), a[160:191] block B
  a[192:255] V^T operands, (d block dt, 16-key step kk) at 192 + 16 dt + 4 kk
  v[40:47]   K operand LDS addresses per k-step (inputs)
  v[48:55]   V^T operand LDS addresses per (dt, half) (inputs)
  v[56:63]   per-thread byte offsets of the eight tile loads (inputs)
  v[72:95]   temporaries, v[96:127] P^T of A and B, v[128:191] S^T of A, B
  v[192:255] K operands (nb, ks) at 192 + 32 nb + 4 ks, carried to the next tile

Online softmax in base 2 with the lazy reference move of the default kernel
(a row's reference moves only when its maximum grew by more than 8);
probabilities are rounded to bf16 for the PV product and summed in fp32.

Hazards. The generator counts wait states: a VALU read of an MFMA result
waits MFMA_VALU wait states after the MFMA's issue, an MFMA read of a VALU
result VALU_MFMA; LDS results are waited for with exact lgkmcnt counts.
Every statement ends with no LDS read in flight.
"""

import os

D, BN = 128, 64
TILE = BN * D * 2           # bytes of one K (or V) tile
MFMA_VALU = 18              # wait states between an MFMA and a VALU read of its result
VALU_MFMA = 4               # between a VALU write and an MFMA operand read
NINF = "0xff800000"
NEG_MAX = "0xff7fffff"      # -FLT_MAX: a finite stand-in for an unset reference
SLACK = "0x41000000"        # 8.0


def vr(base, n):
    return [f"v{base + i}" for i in range(n)]


def ar(base, n):
    return [f"a{base + i}" for i in range(n)]


class Emitter:
    def __init__(self):
        self.out = []
        self.t = 0                  # wait-state clock
        self.ready_valu = {}        # reg -> clock from which a VALU may read it
        self.ready_mfma = {}        # reg -> clock from which an MFMA may read it
        self.lds_seq = {}           # reg -> sequence number of the LDS read writing it
        self.lds_issued = 0
        self.lds_done = -1          # reads with sequence <= this have completed

    def raw(self, s, ws=1):
        self.out.append(s)
        self.t += ws

    def nop_until(self, t):
        while self.t < t:
            k = min(t - self.t, 8)
            self.raw(f"s_nop {k - 1}", k)

    def wait_lds(self, regs):
        need = max((self.lds_seq[r] for r in regs if r in self.lds_seq and self.lds_seq[r] > self.lds_done),
                   default=None)
        if need is None:
            return
        n = min(self.lds_issued - 1 - need, 15)
        self.raw(f"s_waitcnt lgkmcnt({n})")
        self.lds_done = self.lds_issued - 1 - n

    def valu(self, s, reads=(), writes=()):
        self.wait_lds(reads)
        self.nop_until(max((self.ready_valu.get(r, 0) for r in reads), default=0))
        self.raw(s)
        for r in writes:
            self.ready_mfma[r] = self.t + VALU_MFMA
            self.ready_valu.pop(r, None)
            self.lds_seq.pop(r, None)

    def salu(self, s):
        self.raw(s)

    def mfma(self, dst, a, b, c):
        """v_mfma_f32_32x32x16_bf16 dst(16), a(4), b(4), c(16 regs or '0')."""
        reads = a + b + (c if c != "0" else [])
        self.wait_lds(reads)
        self.nop_until(max((self.ready_mfma.get(r, 0) for r in reads), default=0))
        rng = lambda regs: f"{regs[0][0]}[{regs[0][1:]}:{regs[-1][1:]}]"
        # the matrix pipe takes one 8-pass MFMA at a time: consecutive issues
        # lie at least 4 cycles apart
        self.raw(f"v_mfma_f32_32x32x16_bf16 {rng(dst)}, {rng(a)}, {rng(b)}, {rng(c) if c != '0' else '0'}", 4)
        for r in dst:
            self.ready_valu[r] = self.t + MFMA_VALU
            self.ready_mfma.pop(r, None)

    def lds(self, s, writes):
        self.raw(s)
        for r in writes:
            self.lds_seq[r] = self.lds_issued
        self.lds_issued += 1

    def wait_all_lds(self):
        if self.lds_done < self.lds_issued - 1:
            self.raw("s_waitcnt lgkmcnt(0)")
            self.lds_done = self.lds_issued - 1

    def text(self):
        return "\n".join(self.out)


# ---- register map
O = [[ar(64 * x + 16 * dt, 16) for dt in range(4)] for x in range(2)]
Q = [[ar(128 + 32 * x + 4 * ks, 4) for ks in range(8)] for x in range(2)]
V = [[ar(192 + 16 * dt + 4 * kk, 4) for kk in range(4)] for dt in range(4)]
S = [[vr(128 + 32 * x + 16 * nb, 16) for nb in range(2)] for x in range(2)]
K = [[vr(192 + 32 * nb + 4 * ks, 4) for ks in range(8)] for nb in range(2)]
P = [[vr(96 + 16 * x + 4 * kk, 4) for kk in range(4)] for x in range(2)]
KADDR = [f"v{40 + ks}" for ks in range(8)]
VADDR = [[f"v{48 + 2 * dt + h}" for h in range(2)] for dt in range(4)]
DMAOFF = [f"v{56 + j}" for j in range(8)]
TMP = vr(72, 24)             # v72..v95
MNAME = ["%[mA]", "%[mB]"]
LNAME = ["%[lA]", "%[lB]"]
LONAME = ["%[loA]", "%[loB]"]
RGNAME = ["%[rgA]", "%[rgB]"]


def k_reads(e, stage):
    """The 16 K operands of a tile from ring stage `stage`, in the order the
    S^T MFMAs use them."""
    for ks in range(8):
        for nb in range(2):
            e.lds(f"ds_read_b128 v[{K[nb][ks][0][1:]}:{K[nb][ks][-1][1:]}], {KADDR[ks]} "
                  f"offset:{stage * TILE + nb * 32 * D * 2}", K[nb][ks])


def v_read_items(stage):
    """The 32 transposing reads of a tile's V^T operands, in PV order."""
    items = []
    for kk in range(4):
        for dt in range(4):
            for h in range(2):
                regs = V[dt][kk][2 * h:2 * h + 2]
                items.append(("lds", f"ds_read_b64_tr_b16 a[{regs[0][1:]}:{regs[1][1:]}], {VADDR[dt][h]} "
                                     f"offset:{stage * TILE + kk * 16 * D * 2}", regs))
    return items


def s_mfmas(x):
    # the two key blocks' accumulation chains alternate, so no MFMA waits
    # on the one just issued
    out = []
    for ks in range(8):
        for nb in range(2):
            out.append((S[x][nb], K[nb][ks], Q[x][ks], "0" if ks == 0 else S[x][nb]))
    return out


def pv_mfmas(x):
    out = []
    for kk in range(4):
        for dt in range(4):
            out.append((O[x][dt], V[dt][kk], P[x][kk], O[x][dt]))
    return out


def softmax_items(x, masked):
    """Vector work of block x's softmax up to its packed P^T (row sum apart),
    as a list of items: ("v", text, reads, writes), ("s", text) or
    ("rescale",) for the reference-move branch."""
    s = S[x][0] + S[x][1]
    it = []
    if masked:
        # key 4 g + o of the tile, o = 32 nb + 8 (i / 4) + i % 4, is visible
        # iff 0 <= o - lo <= range (unsigned compare: o < lo wraps)
        it.append(("v", f"v_mov_b32 v95, {NINF}", [], ["v95"]))
        for e_ in range(32):
            nb, i = divmod(e_, 16)
            o = 32 * nb + 8 * (i // 4) + i % 4
            it.append(("v", f"v_sub_u32 v94, {o}, {LONAME[x]}", [], ["v94"]))
            it.append(("v", f"v_cmp_gt_u32_e64 %[sp], v94, {RGNAME[x]}", ["v94"], []))
            it.append(("s", "s_nop 1"))
            it.append(("v", f"v_cndmask_b32_e64 {s[e_]}, {s[e_]}, v95, %[sp]", [s[e_], "v95"], [s[e_]]))
    # row maximum: two chains of v_max3 (alternating, so neither waits on
    # its previous step), then the halves of the wavefront
    chains = []
    for regs, dst in ((s[:16], "v88"), (s[16:], "v89")):
        ch = [("v", f"v_max3_f32 {dst}, {regs[0]}, {regs[1]}, {regs[2]}", regs[:3], [dst])]
        k = 3
        while k + 1 < 16:
            ch.append(("v", f"v_max3_f32 {dst}, {dst}, {regs[k]}, {regs[k + 1]}", [dst, regs[k], regs[k + 1]], [dst]))
            k += 2
        ch.append(("v", f"v_max_f32 {dst}, {dst}, {regs[15]}", [dst, regs[15]], [dst]))
        chains.append(ch)
    for a_, b_ in zip(*chains):
        it += [a_, b_]
    it.append(("v", "v_max_f32 v88, v88, v89", ["v88", "v89"], ["v88"]))
    it.append(("v", "v_mov_b32 v89, v88", ["v88"], ["v89"]))
    it.append(("s", "s_nop 1"))
    it.append(("v", "v_permlane32_swap_b32 v88, v89", ["v88", "v89"], ["v88", "v89"]))
    it.append(("v", "v_max_f32 v88, v88, v89", ["v88", "v89"], ["v88"]))
    it.append(("v", "v_mul_f32 v88, %[c], v88", ["v88"], ["v88"]))               # row max in base-2 units
    it.append(("v", f"v_max_f32 v88, {MNAME[x]}, v88", ["v88"], ["v88"]))         # candidate reference
    it.append(("v", f"v_add_f32 v89, {SLACK}, {MNAME[x]}", [], ["v89"]))
    it.append(("v", "v_cmp_gt_f32_e64 %[sp], v88, v89", ["v88", "v89"], []))
    it.append(("rescale",))
    # probabilities 2^(t - m) against the (possibly moved) reference
    it.append(("v", f"v_max_f32 v90, {NEG_MAX}, {MNAME[x]}", [], ["v90"]))
    # each exponential four steps behind its argument
    LAG = 4
    for e_ in range(32 + LAG):
        if e_ < 32:
            it.append(("v", f"v_fma_f32 {s[e_]}, {s[e_]}, %[c], -v90", [s[e_], "v90"], [s[e_]]))
        if e_ >= LAG:
            r = s[e_ - LAG]
            it.append(("v", f"v_exp_f32 {r}, {r}", [r], [r]))
    # P^T packed to bf16: step kk takes registers 8 (kk % 2) .. +7 of S[kk / 2]
    for kk in range(4):
        nb, h = kk >> 1, (kk & 1) * 8
        for e2 in range(4):
            lo, hi = S[x][nb][h + 2 * e2], S[x][nb][h + 2 * e2 + 1]
            it.append(("v", f"v_cvt_pk_bf16_f32 {P[x][kk][e2]}, {lo}, {hi}", [lo, hi], [P[x][kk][e2]]))
    return it


def rowsum_items(x):
    """This lane's sum of block x's 32 probabilities, added to its l."""
    s = S[x][0] + S[x][1]
    t = TMP[:16]
    it = [("v", f"v_add_f32 {t[i]}, {s[i]}, {s[i + 16]}", [s[i], s[i + 16]], [t[i]]) for i in range(16)]
    w = 8
    while w >= 1:
        it += [("v", f"v_add_f32 {t[i]}, {t[i]}, {t[i + w]}", [t[i], t[i + w]], [t[i]]) for i in range(w)]
        w //= 2
    it.append(("v", f"v_add_f32 {LNAME[x]}, {LNAME[x]}, {t[0]}", [t[0]], []))
    return it


def emit_rescale(e, x, label):
    """Branch over the reference move of block x (taken by no row: skipped).
    v88 = candidate reference, %[sp] = rows whose maximum grew past the slack."""
    e.salu("s_cmp_lg_u64 %[sp], 0")
    e.salu(f"s_cbranch_scc0 {label}f")
    t_branch = e.t
    e.valu(f"v_max_f32 v90, {NEG_MAX}, v88", ["v88"], ["v90"])          # mu: finite stand-in for -inf
    e.valu(f"v_sub_f32 v90, {MNAME[x]}, v90", ["v90"], ["v90"])
    e.valu("v_exp_f32 v90, v90", ["v90"], ["v90"])                      # alpha = 2^(m - mu)
    e.salu("s_nop 1")
    e.valu(f"v_mul_f32 {LNAME[x]}, {LNAME[x]}, v90", ["v90"], [])
    e.valu(f"v_mov_b32 {MNAME[x]}, v88", ["v88"], [])
    regs = [r for dt in range(4) for r in O[x][dt]]
    for g in range(0, 64, 8):
        grp = regs[g:g + 8]
        for j, a in enumerate(grp):
            e.valu(f"v_accvgpr_read_b32 {TMP[j]}, {a}", [a], [TMP[j]])
        e.salu("s_nop 1")
        for j in range(8):
            e.valu(f"v_mul_f32 {TMP[j]}, {TMP[j]}, v90", [TMP[j], "v90"], [TMP[j]])
        e.salu("s_nop 1")
        for j, a in enumerate(grp):
            e.valu(f"v_accvgpr_write_b32 {a}, {TMP[j]}", [TMP[j]], [a])
    e.salu("s_nop 1")
    e.raw(f"{label}:", 0)
    # the path that skips the block has only the wait states before it; on
    # the path through it, the block's last writes lie at least the final
    # s_nop behind the label
    e.t = t_branch
    for a in regs:
        e.ready_mfma[a] = e.t + VALU_MFMA


def interleave(e, mfmas, items, x_rescale=None):
    """Issue the phase's MFMAs one at a time with an even share of the
    items (vector work, LDS reads) between them."""
    n = len(mfmas)
    items = list(items)
    for j, (dst, a, b, c) in enumerate(mfmas):
        e.mfma(dst, a, b, c)
        share = -(-len(items) // (n - j)) if items else 0
        for _ in range(share):
            emit_item(e, items.pop(0), x_rescale)
    while items:
        emit_item(e, items.pop(0), x_rescale)


def emit_item(e, it, x_rescale):
    kind = it[0]
    if kind == "v":
        e.valu(it[1], it[2], it[3])
    elif kind == "s":
        e.salu(it[1])
    elif kind == "lds":
        e.lds(it[1], it[2])
    elif kind == "rescale":
        emit_rescale(e, x_rescale, 1 if x_rescale == 0 else 2)


def tile_body(stage, masked):
    """One tile from ring stage `stage` (0 or 1); the next tile's stage is
    1 - stage. Flags in %[fl]: bit 0 wait for the next tile and barrier,
    bit 1 issue the next-but-one tile's loads into this stage, bit 2 read the
    next tile's K operands."""
    e = Emitter()
    # the K operands of this tile were read by the previous statement
    # phase 1: S_A
    for dst, a, b, c in s_mfmas(0):
        e.mfma(dst, a, b, c)
    # phase 2: S_B | softmax A, V^T reads
    sm_a = softmax_items(0, masked)
    vreads = v_read_items(stage)
    merged = []
    # V^T reads spread over the phase, two per MFMA, after the first few
    # softmax steps
    for i, it in enumerate(sm_a):
        merged.append(it)
        if i % 4 == 3 and vreads:
            merged.append(vreads.pop(0))
            if vreads:
                merged.append(vreads.pop(0))
    merged += vreads
    interleave(e, s_mfmas(1), merged, x_rescale=0)
    # phase 3: PV_A | row sum A, softmax B
    interleave(e, pv_mfmas(0), rowsum_items(0) + softmax_items(1, masked), x_rescale=1)
    # next tile: its loads landed everywhere, its successor's loads issued
    e.salu("s_bitcmp1_b32 %[fl], 0")
    e.salu("s_cbranch_scc0 3f")
    e.raw("s_waitcnt vmcnt(0)")
    e.raw("s_barrier")
    e.salu("s_bitcmp1_b32 %[fl], 1")
    e.salu("s_cbranch_scc0 3f")
    # an LDS-bound global load reads M0 one wait state after the SALU write
    # of M0 at the earliest
    for j in range(8):
        e.salu(f"s_add_u32 m0, %[dl], {stage * TILE + j * 128 * 16}")
        e.raw("s_nop 0")
        e.raw(f"global_load_lds_dwordx4 {DMAOFF[j]}, %[kb]")
    for j in range(8):
        e.salu(f"s_add_u32 m0, %[dl], {2 * TILE + stage * TILE + j * 128 * 16}")
        e.raw("s_nop 0")
        e.raw(f"global_load_lds_dwordx4 {DMAOFF[j]}, %[vb]")
    e.raw("3:", 0)
    e.wait_all_lds()   # (the V^T reads: already waited for by the PV_A phase)
    e.salu("s_bitcmp1_b32 %[fl], 2")
    e.salu("s_cbranch_scc0 4f")
    t0, seq0 = e.t, e.lds_issued
    k_reads(e, 1 - stage)
    e.raw("4:", 0)
    e.t = t0
    # phase 4: PV_B | row sum B
    interleave(e, pv_mfmas(1), rowsum_items(1))
    # no LDS read may be in flight when the statement ends
    e.raw("s_waitcnt lgkmcnt(0)")
    return e.text()


def k_read_only(stage):
    e = Emitter()
    k_reads(e, stage)
    e.wait_all_lds()
    return e.text()


def q_to_agpr():
    return "\n".join(f"v_accvgpr_write_b32 a{128 + i}, v{72 + i}" for i in range(64))


def o_zero():
    return "\n".join(f"v_accvgpr_write_b32 a{i}, 0" for i in range(128))


def o_read():
    # the last PV MFMAs may still be running: wait before reading
    return "\n".join(["s_nop 7"] * 4 + [f"v_accvgpr_read_b32 v{72 + i}, a{i}" for i in range(128)])


def c_string(name, text):
    lines = text.split("\n")
    body = "\n".join(f'  "{ln}\\n\\t"' for ln in lines)
    return f"#define {name} \\\n" + " \\\n".join(f'  "{ln}\\n\\t"' for ln in lines) + "\n"


def header():
    parts = ["// Generated by gen_fwd_tile_asm.py: do not edit.",
             "// Tile body of the 64-row prefill shape (head dim 128, 64-key tiles);",
             "// register map and phases are described in the generator.",
             "#pragma once", ""]
    for stage in (0, 1):
        for masked in (0, 1):
            parts.append(c_string(f"FA_TILE_ASM_S{stage}_{'M' if masked else 'U'}", tile_body(stage, masked)))
        parts.append(c_string(f"FA_KREAD_ASM_S{stage}", k_read_only(stage)))
    parts.append(c_string("FA_Q_TO_AGPR_ASM", q_to_agpr()))
    parts.append(c_string("FA_O_ZERO_ASM", o_zero()))
    parts.append(c_string("FA_O_READ_ASM", o_read()))
    regs_v = ", ".join(f'"v{i}"' for i in range(72, 256))
    regs_a = ", ".join(f'"a{i}"' for i in range(256))
    parts.append(f"#define FA_TILE_ASM_CLOBBERS {regs_v}, {regs_a}, \"m0\", \"vcc\", \"memory\"\n")
    parts.append(f"#define FA_AGPR_CLOBBERS {regs_a}\n")
    parts.append(f"#define FA_KREAD_ASM_CLOBBERS {', '.join(repr(f'v{i}').replace(chr(39), chr(34)) for i in range(192, 256))}, \"memory\"\n")
    return "\n".join(parts)


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fa_fwd_tile_asm.h")
    with open(out, "w") as f:
        f.write(header())
    print("wrote", out)
