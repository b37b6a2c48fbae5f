"""Scan of the library's own gfx950 code for one register-reuse pattern.

A DS write (ds_write*, ds_store*) reads its data registers some time after
it issues.  gfx950 code that rewrote such a register with the very next
instruction stored the new value now and then (bf16 dequantize output with
zeros in the first dword of 16-byte chunks, different ones from run to run).
The kernels therefore keep every stored value in its register until an
``s_waitcnt lgkmcnt(...)`` has drained the wave's LDS writes.  This module
finds violations: a DS write whose data register is written by a later
instruction before the next lgkmcnt wait.  It reads the disassembly of the
objects built in this tree (``clang-offload-bundler`` + ``llvm-objdump``).
"""

import os
import re
import subprocess
import tempfile

LLVM = "/opt/rocm/llvm/bin"
BUILD = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "rotated_codebook_bit_amd", "_build")
KERNEL_OBJECTS = ("quantize", "dequantize", "matvec", "matvec_rot", "gemm", "groups", "repack", "upload")


def _vregs(op: str) -> set:
    op = op.strip()
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", op)
    return {int(m.group(1))} if m else set()


def _operands(ins: str) -> list:
    parts = ins.split(None, 1)
    if len(parts) < 2:
        return []
    return [o.strip() for o in parts[1].split(",")]


def violations(lines: list, window: int = 64) -> list:
    """(index, write, overwrite) for every DS write in `lines` (instruction
    text, one per entry) whose data registers are written again before an
    lgkmcnt wait.  The first operand of a DS write is the address; the rest
    up to the first modifier are data.  An instruction writes its first
    operand (VALU, loads)."""
    out = []
    for i, ins in enumerate(lines):
        if not ins.startswith(("ds_write", "ds_store")):
            continue
        data = set()
        for o in _operands(ins)[1:]:
            data |= _vregs(o.split()[0] if o else o)
        if not data:
            continue
        for ins2 in lines[i + 1:i + 1 + window]:
            if ins2.startswith("s_waitcnt") and "lgkmcnt" in ins2:
                break
            if ins2.startswith(("v_", "ds_read", "ds_load", "buffer_load", "global_load", "flat_load")):
                ops = _operands(ins2)
                if ops and (_vregs(ops[0]) & data):
                    out.append((i, ins, ins2))
                    break
    return out


def store_reuse(lines: list, window: int = 64) -> list:
    """(index, store, overwrite) for every buffer or global store whose data
    registers are written again before the next vmcnt wait: the same
    register-lifetime question as for DS writes, asked of VMEM stores.  The
    data operand is the first operand of a buffer store and the second of a
    global store.  (A report: the compiler emits this pattern at most VMEM
    stores, and every stored byte of the codec kernels is checked against
    the oracle at full size, so it is not a gate the way the DS-write scan
    is.)"""
    out = []
    for i, ins in enumerate(lines):
        if not ins.startswith(("buffer_store", "global_store")):
            continue
        ops = _operands(ins)
        pos = 0 if ins.startswith("buffer_store") else 1
        data = _vregs(ops[pos].split()[0]) if len(ops) > pos and ops[pos] else set()
        if not data:
            continue
        for ins2 in lines[i + 1:i + 1 + window]:
            if ins2.startswith("s_waitcnt") and "vmcnt" in ins2:
                break
            if ins2.startswith(("v_", "ds_read", "ds_load", "buffer_load", "global_load", "flat_load")):
                o2 = _operands(ins2)
                if o2 and (_vregs(o2[0]) & data):
                    out.append((i, ins, ins2))
                    break
    return out


def disassemble(obj: str) -> dict:
    """Kernel name -> list of instruction texts, from the gfx950 code object
    embedded in the host object `obj`."""
    with tempfile.TemporaryDirectory() as d:
        fb, co, tmp = os.path.join(d, "fb.bin"), os.path.join(d, "dev.co"), os.path.join(d, "t.o")
        subprocess.run([f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={fb}", obj, tmp], check=True,
                       capture_output=True)
        subprocess.run([f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={fb}", f"--output={co}"],
                       check=True, capture_output=True)
        text = subprocess.run([f"{LLVM}/llvm-objdump", "-d", "--mcpu=gfx950", co], check=True,
                              capture_output=True, text=True).stdout
    funcs, cur = {}, None
    for line in text.splitlines():
        m = re.match(r"^[0-9a-f]+ <(.+)>:$", line)
        if m:
            cur = funcs.setdefault(m.group(1), [])
            continue
        if cur is not None:
            ins = line.split("//")[0].strip()
            if ins:
                cur.append(ins)
    return funcs
