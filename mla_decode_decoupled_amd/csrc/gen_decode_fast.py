"""Writes decode_fast.hip from decode_fast.in.hip by expanding the inline-asm bodies of the
MFMA latent-attention kernel (score phase, P.V phase with and without the interleaved softmax,
and the tile DMA). Run after editing the template: python gen_decode_fast.py"""
import os

HERE = os.path.dirname(os.path.abspath(__file__))
ROW_BYTES = 1152
P_STRIDE = 80

RING = list(range(88, 112, 4))   # six 4-register operand slots of the score phase, v[88:111]


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
    """P.V of one tile for the wave's 128 latent columns (column blocks 4w .. 4w+3) and all 128
    heads: 32 MFMAs (2 key steps x 4 column blocks x 4 head blocks). A = V^T fragments from the tile
    by transpose reads, each feeding the 4 MFMAs of its column block; B = the P fragments of all four
    waves from the LDS P buffer (%[pb]), each feeding 4 MFMAs. Operands stream through eight
    4-register slots, v[80:111]. The softmax of the next tile (scores in v[112:127]) is interleaved;
    its P is packed in place into v[112:119] and stored to this wave's part of the other P buffer
    (%[pw]) after the last MFMA."""
    sm = []
    for r in range(16):  # x = s * scale - m_ref
        sm.append(f"v_fma_f32 v{112+r}, v{112+r}, %[sc], %[nm]")
    for r in range(16):
        sm.append(f"v_exp_f32 v{112+r}, v{112+r}")
    for r in range(16):
        sm.append(f"v_add_f32 %[l], %[l], v{112+r}")
    # in place: v[112+j] <- (v[112+2j], v[113+2j]); for j >= 1 the destination was a source of an
    # earlier pack, so the order j = 0..7 never overwrites an unread value
    sm += [f"v_cvt_pk_bf16_f32 v{112+j}, v{112+2*j}, v{113+2*j}" for j in range(8)]
    order = [(s, db, hb) for s in range(2) for db in range(4) for hb in range(4)]
    ops = []                       # operands in order of first use
    last_use = {}
    for i, (s, db, hb) in enumerate(order):
        for op in (("A", s, db), ("B", s, hb)):
            if op not in last_use:
                ops.append(op)
            last_use[op] = i

    def instrs(op, r):
        if op[0] == "A":
            _, s, db = op
            base = s * 16 * ROW_BYTES + (db >> 1) * 128
            return [f"ds_read_b64_tr_b16 v[{r}:{r + 1}], %[v{db & 1}0] offset:{base}",
                    f"ds_read_b64_tr_b16 v[{r + 2}:{r + 3}], %[v{db & 1}1] offset:{base}"]
        _, s, hb = op
        return [f"ds_read_b128 v[{r}:{r + 3}], %[pb] offset:{(2 * hb + s) * 1024}"]

    L = []
    slots = list(range(80, 112, 4))
    holder = {r: None for r in slots}      # slot -> operand it holds
    where = {}                             # operand -> slot
    issued = []                            # LDS instructions in issue order (operand of each)
    waited = [-1]
    nxt = [0]

    def fill(done):                        # MFMAs 0 .. done have issued
        while nxt[0] < len(ops):
            free = [r for r in slots if holder[r] is None or last_use[holder[r]] <= done]
            if not free:
                return
            r = free[0]
            op = ops[nxt[0]]
            holder[r] = op
            where[op] = r
            for ins in instrs(op, r):
                L.append(ins)
                issued.append(op)
            nxt[0] += 1

    def wait(ops_needed):
        idx = max(len(issued) - 1 - issued[::-1].index(op) for op in ops_needed)
        if idx > waited[0]:
            L.append(f"s_waitcnt lgkmcnt({len(issued) - 1 - idx})")
            waited[0] = idx

    n = len(order)
    spread = 28
    per = [0] * n
    for i in range(len(sm)):
        per[i * spread // len(sm)] += 1
    q = list(sm)
    fill(-1)
    for i, (s, db, hb) in enumerate(order):
        a, b = ("A", s, db), ("B", s, hb)
        wait([a, b])
        ra, rb = where[a], where[b]
        acc = db * 4 + hb
        L.append(f"v_mfma_f32_32x32x16_bf16 %[o{acc}], v[{ra}:{ra + 3}], v[{rb}:{rb + 3}], %[o{acc}]")
        for _ in range(per[i]):
            L.append(q.pop(0))
        fill(i)
    assert not q and nxt[0] == len(ops)
    # P of the next tile to this wave's part of the other buffer: 16 bytes per lane per key step
    L += ["ds_write_b128 %[pw], v[112:115] offset:0", "ds_write_b128 %[pw], v[116:119] offset:1024", "s_nop 1"]
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
