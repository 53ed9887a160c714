"""Writes gemm_w4_steps.inc: the instruction sequences of one 16-deep K-step of the main GEMM.

A K-step is 16 v_mfma_f32_32x32x16_bf16 (8 row tiles x 2 column tiles of one wave) with the work for
the next K-step spread between them: LDS reads of the next A operand (and codes / scales), and the
decode of the next 4-bit B operand (E2M1 codes -> fp32 via v_cvt_scalef32_pk_f32_fp4 with scale 1,
times the E4M3 block scale, packed to bf16 by v_perm_b32). Written as one asm block per step so the
compiler cannot gather the decode into a run that leaves the matrix core idle.

Registers v108..v111 and v120..v127 are private to each block (declared clobbered): v120..v127 are
decode temporaries, v110/v111 the code dwords, v108/v109 the block scales of a new tile. The running step's W4
B operand comes in as two 4-register tuples %[bq0], %[bq1] (the previous block's eight decoded
outputs, which the compiler allocates in place).

A step can also carry global->LDS copies of a later K-tile (buffer_load_dwordx4 ... lds, M0 = LDS
address), spread between its MFMAs so that the copies of a tile trickle out over the steps between
two stage handovers instead of leaving every wave at once. Copy j takes operands %[cmj] (M0 value),
%[cvj] (per-lane offset), %[csj] (uniform offset) and %[crj] (buffer descriptor); a masked copy runs
on lanes 0..15 only (exec saved in %[ex]). M0 is saved in %[msv] and restored at the end. The copies
of a step go after evenly spaced MFMAs.

Run `python gen_gemm_steps.py` after editing; tests/test_abi_cpu.py checks the .inc is current.
"""
import os

RT = 8          # row tiles (of 32) per wave
SCL = (108, 109)   # block scales of a new tile (fp32)
CODE = (110, 111)  # code dwords of the two column tiles
TMP = 120          # v120..v127: decode temporaries
SEL = {0: "", 1: " op_sel:[1,0,0]", 2: " op_sel:[0,1,0]", 3: " op_sel:[1,1,0]"}


def mf(i, j, b):
    return f"v_mfma_f32_32x32x16_bf16 %[c{i}{j}], %[a{i}], {b}, %[c{i}{j}]"


def decode_groups(scale_regs):
    """Decode code dword CODE[0] (scale scale_regs[0]) -> m0..m3 and CODE[1] (scale_regs[1]) -> m4..m7."""
    dec = []
    for j, (w, s) in enumerate([(f"v{CODE[0]}", scale_regs[0]), (f"v{CODE[1]}", scale_regs[1])]):
        for half in range(2):
            b0, b1 = 2 * half, 2 * half + 1
            t0, t1 = TMP + 4 * half, TMP + 2 + 4 * half
            dec.append([f"v_cvt_scalef32_pk_f32_fp4 v[{t0}:{t0+1}], {w}, 1.0{SEL[b0]}",
                        f"v_cvt_scalef32_pk_f32_fp4 v[{t1}:{t1+1}], {w}, 1.0{SEL[b1]}",
                        f"v_mul_f32 v{t0}, {s}, v{t0}",
                        f"v_mul_f32 v{t0+1}, {s}, v{t0+1}",
                        f"v_mul_f32 v{t1}, {s}, v{t1}",
                        f"v_mul_f32 v{t1+1}, {s}, v{t1+1}",
                        f"v_perm_b32 %[m{4*j+b0}], v{t0+1}, v{t0}, %[sel]",
                        f"v_perm_b32 %[m{4*j+b1}], v{t1+1}, v{t1}, %[sel]"])
    return dec


def copy_at(n):
    """MFMA positions (0 .. 2 RT - 1) after which the n copies of a step go: evenly spaced."""
    nm = 2 * RT
    return [(q * nm) // n + (nm // n) // 2 for q in range(n)]


def copy_lines(j, masked):
    body = [f"s_mov_b32 m0, %[cm{j}]", "s_nop 0", f"buffer_load_dwordx4 %[cv{j}], %[cr{j}], %[cs{j}] offen lds"]
    if not masked:
        return body
    return ["s_mov_b64 %[ex], exec", "s_mov_b32 exec_lo, 0xffff", "s_mov_b32 exec_hi, 0"] + body + \
           ["s_mov_b64 exec, %[ex]"]


def step(kind, copies=""):
    """kind: src ('b' base W4 operand %[bq0],%[bq1] | 'l' LoRA bf16 operand %[l0],%[l1]) +
    next ('b' next K-step of a base tile | 'B' first K-step of a new base tile (scales read here) |
          'l' a LoRA K-step | 'n' none); copies: one letter per copy, 'c' plain, 'm' lanes 0..15."""
    src, nxt = kind[0], kind[1]
    L = ["s_waitcnt lgkmcnt(0)", "s_nop 3"]
    if copies:
        L.append("s_mov_b32 %[msv], m0")
    n_mfma = 2 * RT
    extras = [[] for _ in range(n_mfma)]
    if nxt in 'bB':
        if nxt == 'B':
            L += ["ds_read_b32 %[d0], %[saddr]", "ds_read_b32 %[d1], %[saddr] offset:128"]
        L += [f"ds_read_b32 v{CODE[0]}, %[caddr]", f"ds_read_b32 v{CODE[1]}, %[caddr] offset:128"]
        for i in range(RT):
            extras[i].append(f"ds_read_b128 %[n{i}], %[aaddr] offset:{i*4096}")
        extras[RT - 1].append(f"s_waitcnt lgkmcnt({RT})")
        if nxt == 'B':
            extras[RT - 1] += [f"v_cvt_f32_fp8_sdwa v{SCL[0]}, %[d0] src0_sel:BYTE_0",
                               f"v_cvt_f32_fp8_sdwa v{SCL[1]}, %[d1] src0_sel:BYTE_0"]
            scales = (f"v{SCL[0]}", f"v{SCL[1]}")
        else:
            scales = ("%[s0]", "%[s1]")
        for k, grp in enumerate(decode_groups(scales)):
            extras[RT + k] += grp
    elif nxt == 'l':
        for i in range(RT):
            extras[i].append(f"ds_read_b128 %[n{i}], %[aaddr] offset:{i*2048}")
        extras[RT].append("ds_read_b128 %[k0], %[baddr]")
        extras[RT + 1].append("ds_read_b128 %[k1], %[baddr] offset:2048")
    for j, (at, kind_c) in enumerate(zip(copy_at(len(copies)), copies)):
        extras[at] += copy_lines(j, kind_c == 'm')
    L.append("s_nop 1")
    for s in range(n_mfma):
        i, j = s // 2, s % 2
        L.append(mf(i, j, f"%[bq{j}]" if src == 'b' else f"%[l{j}]"))
        L += extras[s]
    if nxt != 'n':
        L.append("s_waitcnt lgkmcnt(0)")
    if copies:
        L.append("s_mov_b32 m0, %[msv]")
    return L


def render() -> str:
    out = ["// Generated by gen_gemm_steps.py -- do not edit by hand.",
           "// Step variants: source operand (B = W4 decoded, L = LoRA bf16) x next step",
           "// (B: next K-step of the same base tile, BN: first K-step of a new base tile, L: a LoRA",
           "// K-step, N: none) x copies carried (Cn: n plain copies, M: then one on lanes 0..15).",
           ""]
    names = {'bb': 'BB', 'bB': 'BBN', 'bl': 'BL', 'bn': 'BN', 'll': 'LL', 'ln': 'LN'}

    def cname(copies):
        if not copies:
            return ""
        plain = copies.count('c')
        return f"_C{plain}" + ("M" if copies.endswith('m') else "")
    for kind, copies in [('bb', 'ccc'), ('bb', 'cm'), ('bB', 'ccc'), ('bl', 'ccc'), ('bn', ''),
                         ('ll', 'cccccccm'), ('ll', 'ccc'), ('ln', '')]:
        out.append(f"#define H3Q_STEP_{names[kind]}{cname(copies)}_ASM \\")
        body = step(kind, copies)
        for n, l in enumerate(body):
            out.append(f'  "{l}\\n\\t"' + (" \\" if n + 1 < len(body) else ""))
        out.append("")
    return "\n".join(out)


INC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gemm_w4_steps.inc")

if __name__ == "__main__":
    with open(INC, "w") as f:
        f.write(render())
