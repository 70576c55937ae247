"""Wait states in front of the tile copies that the kernels issue as inline asm.

The compiler checks no hazards into an asm block, so the block brings its
own: a VMEM instruction that reads an SGPR written by a VALU instruction
(v_readfirstlane of a page base, v_readlane of a spilled SGPR) needs 5 wait
states after that write (CDNA3 ISA, "Manually Inserted Wait States"), and
an LDS DMA needs 1 after an SALU write of M0.  Without them the copy can
take a descriptor SGPR's previous contents as its base address.  Kernels
whose descriptors may come from VALU instructions (paged K / V, the 8-wave
kernel's spilled descriptors) open each copy with s_nop 4, the others with
s_nop 0.

Every prefill source is compiled to gfx950 assembly and every direct-to-LDS
buffer load is checked on the straight line of code before it.
"""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from gqa_attention_ragged_amd import build

# one source per element type (f16 and bf16 instantiate the same code)
SOURCES = ["prefill_bf16.hip", "prefill_fp8.hip", "prefill_kv8_bf16.hip", "prefill_pp.hip",
           "prefill_persist.hip"]
VALU_SGPR_WAITS = 5
M0_WAITS = 1


def _asm(src: str, out_dir: str) -> str:
    flags = [f for f in build.HIPCC_FLAGS if not f.startswith("-Rpass")]
    out = os.path.join(out_dir, src + ".s")
    cmd = ["hipcc", "-x", "hip", *flags, "--cuda-device-only", "-S",
           os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


@pytest.fixture(scope="module")
def listings():
    if shutil.which("hipcc") is None:
        pytest.skip("hipcc not found")
    with tempfile.TemporaryDirectory() as d, ThreadPoolExecutor(len(SOURCES)) as ex:
        return dict(zip(SOURCES, ex.map(lambda s: _asm(s, d), SOURCES)))


def _sgprs(tok: str) -> set:
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"s(\d+)", tok)
    return {int(m.group(1))} if m else set()


def _instructions(text: str):
    """(mnemonic, operands, raw line, is_label) per line of code."""
    for line in text.split("\n"):
        t = line.split(";")[0].strip()
        if not t:
            continue
        if t.endswith(":") or t.startswith("."):
            yield None, [], t, True
            continue
        parts = t.split(None, 1)
        ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        yield parts[0], ops, t, False


def _scan(text: str):
    """For each direct-to-LDS buffer load: (wait states back to the nearest
    VALU write of one of its SGPRs, wait states back to the nearest SALU
    write of M0, the instruction right before it).  The walk stops at a
    label or after twice the wait states needed (None: nothing found), so
    that it also sees what lies behind an asm block's own wait states."""
    ins = list(_instructions(text))
    out = []
    for i, (op, ops, raw, lab) in enumerate(ins):
        if lab or not op.startswith("buffer_load") or not raw.endswith(" lds"):
            continue
        regs = set().union(*[_sgprs(o.split()[0]) for o in ops[1:]])
        prev = ins[i - 1][2] if i else ""
        valu_ws = m0_ws = None
        ws = 0
        for op2, ops2, raw2, lab2 in reversed(ins[:i]):
            if lab2 or ws >= 2 * VALU_SGPR_WAITS:
                break
            dst = _sgprs(ops2[0]) if ops2 else set()
            if valu_ws is None and op2.startswith("v_") and dst & regs:
                valu_ws = ws
            if m0_ws is None and op2.startswith("s_") and ops2 and ops2[0] == "m0":
                m0_ws = ws
            ws += int(ops2[0], 0) + 1 if op2 == "s_nop" else 1
        out.append((valu_ws, m0_ws, prev))
    return out


def test_every_inline_copy_opens_with_a_wait_state(listings):
    for src, text in listings.items():
        asm_copies = [c for c in _scan(text) if c[2].startswith("s_nop")]
        assert asm_copies, f"{src}: no inline-asm copies found"


def test_no_copy_reads_a_fresh_sgpr(listings):
    for src, text in listings.items():
        for valu_ws, m0_ws, prev in _scan(text):
            assert valu_ws is None or valu_ws >= VALU_SGPR_WAITS, (src, valu_ws, prev)
            assert m0_ws is None or m0_ws >= M0_WAITS, (src, m0_ws, prev)


def test_the_scan_sees_descriptors_written_by_valu(listings):
    # without the asm block's own wait states some copies would read SGPRs
    # fewer than 5 wait states after a VALU wrote them (the paged kernels,
    # the 8-wave kernel): the checks above are not vacuous
    for src in ("prefill_bf16.hip", "prefill_kv8_bf16.hip", "prefill_pp.hip"):
        near = [v for v, _, prev in _scan(listings[src])
                if v is not None and prev.startswith("s_nop")
                and v - (int(prev.split()[1], 0) + 1) < VALU_SGPR_WAITS]
        assert near, src
