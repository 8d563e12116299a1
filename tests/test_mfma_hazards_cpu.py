"""Wait states around the matrix instructions of the built library (CPU only: reads the gfx950 code
objects of libattn.so through llvm-objdump).

Some matrix instructions of the one-wave-per-SIMD kernels are inline assembly, whose hazards the
compiler does not see; their waits are written out in csrc/attn_device.h.  This test checks what
was built, for every v_mfma in every kernel (asm or not), in straight-line code:
  * no vector-ALU write of one of its source registers within the 2 wait states before it;
  * no instruction reading or writing its result registers within the 12 wait states after it,
    except the next instruction of the same chain (same accumulator registers in full as source
    and result).
2 and 12 are what the compiler itself puts around v_mfma_f32_32x32x16_bf16 on gfx950 (an 8-pass
instruction): a vector write of a source, then the instruction; the instruction, then a vector
read or write of its result.  A window that reaches a branch or a branch target stops there
(the compiler's own recognizer covers the instructions it emits across blocks, and the kernels'
assembly chains and their waits sit in straight-line code); those stops are counted, not failed.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "tiled_online_softmax_02_amd", "libattn.so")
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
BEFORE, AFTER = 2, 12

_FUNC = re.compile(r"^([0-9a-f]+) <(\S+)>:$")
_INST = re.compile(r"^\s+(\S+)(.*?)\s*//\s*([0-9A-Fa-f]+):[^<]*(?:<(\S+)\+0x([0-9a-f]+)>)?\s*$")
_REG = re.compile(r"^([va])(?:\[(\d+):(\d+)\]|(\d+))$")


def regs(tok):
    m = _REG.match(tok.strip())
    if not m:
        return set()
    f = m.group(1)
    if m.group(4) is not None:
        return {(f, int(m.group(4)))}
    return {(f, i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}


def disassemble(tmp):
    shutil.copy(LIB, os.path.join(tmp, "libattn.so"))
    subprocess.run([OBJDUMP, "--offloading", "libattn.so"], cwd=tmp, check=True, capture_output=True, timeout=120)
    text = []
    for name in sorted(os.listdir(tmp)):
        if name.endswith("gfx950"):
            out = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", name], cwd=tmp, check=True,
                                 capture_output=True, text=True, timeout=300)
            text.append(out.stdout)
    return text


def parse(text):
    """Functions as lists of (address, op, operands); the set of branch-target addresses."""
    funcs, targets, base = [], set(), {}
    cur = None
    for line in text.splitlines():
        m = _FUNC.match(line)
        if m:
            cur = []
            funcs.append(cur)
            base[m.group(2)] = int(m.group(1), 16)
            continue
        m = _INST.match(line)
        if m and cur is not None:
            op, rest, addr = m.group(1), m.group(2), int(m.group(3), 16)
            ops = [o.strip() for o in rest.split(",")] if rest.strip() else []
            cur.append((addr, op, ops))
            if m.group(4) and ("branch" in op):
                targets.add((m.group(4), int(m.group(5), 16)))
    abs_targets = {base[f] + off for f, off in targets if f in base}
    return funcs, abs_targets


def wait_states(op, ops):
    return int(ops[0], 0) + 1 if op == "s_nop" else 1


def is_control(op):
    return op.startswith("s_cbranch") or op.startswith("s_branch") or op in ("s_endpgm", "s_setpc_b64")


def check(funcs, targets):
    n = stops = 0
    bad = []
    for ins in funcs:
        for i, (addr, op, ops) in enumerate(ins):
            if not op.startswith("v_mfma") or len(ops) < 4:
                continue
            n += 1
            dst, srcs, srcc = regs(ops[0]), set().union(*(regs(o) for o in ops[1:])), regs(ops[3])
            # before: vector-ALU writes of a source
            k, ws = i - 1, 0
            if addr in targets:
                stops += 1
            while k >= 0 and ws < BEFORE and addr not in targets:
                a2, op2, ops2 = ins[k]
                if is_control(op2):
                    stops += 1
                    break
                if op2.startswith("v_") and not op2.startswith("v_mfma") and ops2 and regs(ops2[0]) & srcs:
                    bad.append(("source written %d wait states before" % ws, hex(addr), op, ops[:4], op2, ops2[:2]))
                    break
                ws += wait_states(op2, ops2)
                if a2 in targets:
                    stops += 1
                    break
                k -= 1
            # after: any use of the result
            k, ws = i + 1, 0
            while k < len(ins) and ws < AFTER:
                a2, op2, ops2 = ins[k]
                if a2 in targets or is_control(op2):
                    stops += 1
                    break
                touched = set().union(*(regs(o) for o in ops2)) if ops2 else set()
                if touched & dst:
                    if op2.startswith("v_mfma") and len(ops2) >= 4 and regs(ops2[0]) == dst and regs(ops2[3]) == dst and srcc == dst:
                        break  # the chain goes on in the same registers
                    if op2.startswith("v_mfma") and len(ops2) >= 4 and regs(ops2[0]) == dst and regs(ops2[3]) == dst:
                        break  # first of a chain (zero start) followed by its next instruction
                    bad.append(("result touched %d wait states after" % ws, hex(addr), op, ops[:4], op2, ops2[:2]))
                    break
                ws += wait_states(op2, ops2)
                k += 1
    return n, stops, bad


@pytest.mark.skipif(not os.path.exists(LIB), reason="libattn.so not built")
@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="llvm-objdump not available")
def test_matrix_instruction_wait_states():
    with tempfile.TemporaryDirectory() as tmp:
        texts = disassemble(tmp)
    assert texts, "no gfx950 code object in libattn.so"
    n = stops = 0
    bad = []
    for t in texts:
        funcs, targets = parse(t)
        a, b, c = check(funcs, targets)
        n, stops, bad = n + a, stops + b, bad + c
    print("matrix instructions checked: %d; windows stopped at control flow: %d" % (n, stops))
    assert n > 5000, n
    assert not bad, bad[:10]


def test_checker_finds_planted_hazards():
    """The checker itself, on hand-written instruction lists: a source written one instruction
    before, a result read within the window, and a clean chain."""
    ins = [
        (0, "v_mov_b32_e32", ["v2", "v9"]),
        (4, "v_mfma_f32_32x32x16_bf16", ["v[16:31]", "v[0:3]", "v[4:7]", "v[16:31]"]),
        (12, "v_mfma_f32_32x32x16_bf16", ["v[16:31]", "v[8:11]", "v[4:7]", "v[16:31]"]),
        (20, "s_nop", ["7"]),
        (24, "v_add_f32_e32", ["v20", "v20", "v21"]),
    ]
    n, stops, bad = check([ins], set())
    assert n == 2
    kinds = sorted(b[0].split()[0] for b in bad)
    assert kinds == ["result", "source"], bad
    clean = [
        (4, "v_mfma_f32_32x32x16_bf16", ["v[16:31]", "v[0:3]", "v[4:7]", "0"]),
        (12, "v_mfma_f32_32x32x16_bf16", ["v[16:31]", "v[8:11]", "v[4:7]", "v[16:31]"]),
        (20, "s_nop", ["7"]),
        (24, "s_nop", ["7"]),
        (28, "s_nop", ["3"]),
        (32, "v_add_f32_e32", ["v20", "v20", "v21"]),
    ]
    n, stops, bad = check([clean], set())
    assert n == 2 and not bad, bad
