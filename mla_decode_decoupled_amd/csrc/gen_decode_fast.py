"""Writes decode_fast.hip from decode_fast.in.hip by expanding the inline-asm bodies of the
MFMA latent-attention kernel (score phase, P.V phase with and without the interleaved softmax,
and the tile DMA). Run after editing the template: python gen_decode_fast.py"""
import os

HERE = os.path.dirname(os.path.abspath(__file__))
ROW_BYTES = 1152
P_STRIDE = 80

RING = list(range(88, 112, 4))   # six 4-register operand slots, v[88:111], shared by both phases


class Ring:
    """LDS operand loads through a ring of register slots, issued in program order. A load into a
    slot is issued only after the MFMA that last read the slot has issued; before an MFMA the
    lgkmcnt wait is the number of loads issued after the newest one it needs."""

    def __init__(self, out):
        self.out = out
        self.issued = []        # load ids in issue order
        self.waited = -1        # index of the newest load already waited for
        self.slot_of = {}
        self.free_after = {}    # slot -> index of the MFMA that must issue first (-1 = free)

    def issue(self, lid, slot, instrs):
        self.out.extend(instrs)
        self.issued.append(lid)
        self.slot_of[lid] = slot

    def wait(self, lids):
        idx = max(self.issued.index(l) for l in lids)
        if idx > self.waited:
            n_after = len(self.issued) - 1 - idx
            self.out.append(f"s_waitcnt lgkmcnt({n_after})")
            self.waited = idx


def qk():
    """Scores of one tile: 36 chained MFMAs (32 latent steps with the query in v[128:255], 4
    position steps with the query's position part in v[64:79]), the K chunks streamed through the
    six-slot ring, plus the nine DMA instructions of a later tile."""
    L = []
    ring = Ring(L)
    # operand loads in consumption order: (id, slot-use MFMA, instruction)
    loads = []
    for s in range(36):
        loads.append((("A", s), s, f"ds_read_b128 {{r}}, %[k{s % 4}] offset:{(s // 4) * 128}"))
    nslot = len(RING)
    slot_user = [-1] * nslot          # MFMA that reads the slot's current content
    next_load = 0

    def fill(after_mfma):
        nonlocal next_load
        while next_load < len(loads):
            slot = next_load % nslot
            if slot_user[slot] > after_mfma:   # still to be read by an MFMA not yet issued
                return
            lid, user, ins = loads[next_load]
            reg = f"v[{RING[slot]}:{RING[slot] + 3}]"
            ring.issue(lid, slot, [ins.format(r=reg)])
            slot_user[slot] = user
            next_load += 1
    fill(-1)
    for s in range(36):
        ring.wait([("A", s)])
        a_reg = RING[ring.slot_of[("A", s)]]
        a = f"v[{a_reg}:{a_reg + 3}]"
        if s < 32:
            b = f"v[{128 + 4 * s}:{131 + 4 * s}]"
        else:   # the position part of the query, held in v[64:79]
            b = f"v[{64 + 4 * (s - 32)}:{67 + 4 * (s - 32)}]"
        c = "0" if s == 0 else "v[112:127]"
        L.append(f"v_mfma_f32_32x32x16_bf16 v[112:127], {a}, {b}, {c}")
        fill(s)
        if s % 4 == 1:  # one of the 9 DMA instructions of a later tile, every 4 MFMAs
            L += dma_instr(s // 4)
    assert next_load == len(loads)
    L += ["s_nop 7", "s_nop 7", "s_nop 3"]
    return L


def pv():
    """P.V of one tile for the wave's own 32 heads: 32 MFMAs (2 key steps x 16 latent column
    blocks), B = P from v[80:87], A = V^T fragments from the tile by transpose reads through the
    six-slot ring. The softmax of the next tile (scores in v[112:127]) is interleaved; its P goes
    to v[80:83] once the first key step no longer reads them and to v[84:87] after the last MFMA."""
    sm = []
    for r in range(16):  # x = s * scale - m_ref
        sm.append(f"v_fma_f32 v{112+r}, v{112+r}, %[sc], %[nm]")
    for r in range(16):
        sm.append(f"v_exp_f32 v{112+r}, v{112+r}")
    for r in range(16):
        sm.append(f"v_add_f32 %[l], %[l], v{112+r}")
    cvt0 = [f"v_cvt_pk_bf16_f32 v{80+j}, v{112+2*j}, v{113+2*j}" for j in range(4)]
    cvt1 = [f"v_cvt_pk_bf16_f32 v{84+j}, v{120+2*j}, v{121+2*j}" for j in range(4)]
    L = []
    ring = Ring(L)
    order = [(s, cb) for s in range(2) for cb in range(16)]
    loads = []
    for i, (s, cb) in enumerate(order):
        base = s * 16 * ROW_BYTES + (cb >> 1) * 128
        loads.append(((s, cb), i, [f"ds_read_b64_tr_b16 {{r0}}, %[v{cb & 1}0] offset:{base}",
                                   f"ds_read_b64_tr_b16 {{r1}}, %[v{cb & 1}1] offset:{base}"]))
    nslot = len(RING)
    slot_user = [-1] * nslot
    next_load = 0

    def fill(after_mfma):
        nonlocal next_load
        while next_load < len(loads):
            slot = next_load % nslot
            if slot_user[slot] > after_mfma:
                return
            lid, user, ins = loads[next_load]
            r = RING[slot]
            instrs = [ins[0].format(r0=f"v[{r}:{r + 1}]"), ins[1].format(r1=f"v[{r + 2}:{r + 3}]")]
            # two instructions per fragment: record both so the waits count them
            ring.issue(("x", lid), slot, instrs[:1])
            ring.issue(lid, slot, instrs[1:])
            slot_user[slot] = user
            next_load += 1
    n_mfma = len(order)
    spread = 28
    per = [0] * n_mfma
    for i in range(len(sm)):
        per[i * spread // len(sm)] += 1
    q = list(sm)
    fill(-1)
    for i, (s, cb) in enumerate(order):
        ring.wait([(s, cb)])
        a_reg = RING[ring.slot_of[(s, cb)]]
        b = "v[80:83]" if s == 0 else "v[84:87]"
        L.append(f"v_mfma_f32_32x32x16_bf16 %[o{cb}], v[{a_reg}:{a_reg + 3}], {b}, %[o{cb}]")
        for _ in range(per[i]):
            L.append(q.pop(0))
        if i >= spread:                   # the first key step is done with v[80:83]
            L.append(cvt0[i - spread])
        fill(i)
    assert not q and next_load == len(loads)
    L += ["s_nop 7"] + cvt1           # v[84:87] was read by the last MFMA
    return L


def qload():
    """The 32 latent query fragments from the staged rows into v[128:255]."""
    L = [f"ds_read_b128 v[{128+4*s}:{131+4*s}], %[a] offset:{32*s}" for s in range(32)]
    return L + ["s_waitcnt lgkmcnt(0)"]


def dma_instr(it):
    """DMA instruction `it` (0..8) of a wave's share of a tile: 1 KB at LDS byte M0 + 1024 it. The
    instruction's offset field moves both the global and the LDS address, so M0 is set once per
    four instructions (the per-lane global offsets are biased by -1024 (it % 4) to match)."""
    L = []
    if it % 4 == 0:
        L += ["s_mov_b32 m0, %[m]" if it == 0 else "s_add_u32 m0, m0, 0x1000", "s_nop 0"]
    L.append(f"global_load_lds_dwordx4 %[o{it}], %[b] offset:{(it % 4) * 1024}")
    return L


def dma():
    L = []
    for it in range(9):
        L += dma_instr(it)
    return L

def emit(lines):
    return "\n".join(f'        "{l}\\n\\t"' for l in lines)


def generate(template_path: str) -> str:
    """The expanded kernel source for the template at template_path."""
    src = open(template_path).read()
    src = src.replace('@GENERATED_NOTE@',
                      '// GENERATED by gen_decode_fast.py from decode_fast.in.hip: edit the template, then rerun it.')
    return (src.replace('@QK_ASM@', emit(qk())).replace('@PVSM_ASM@', emit(pv())).replace('@DMA_ASM@', emit(dma()))
            .replace('@QLOAD_ASM@', emit(qload())))


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="expand decode_fast.in.hip into decode_fast.hip")
    ap.add_argument("--template", default=os.path.join(HERE, 'decode_fast.in.hip'))
    ap.add_argument("-o", "--output", default=os.path.join(HERE, 'decode_fast.hip'))
    a = ap.parse_args()
    with open(a.output, 'w') as fh:
        fh.write(generate(a.template))
    print(len(qk()), len(pv()), len(dma()))
