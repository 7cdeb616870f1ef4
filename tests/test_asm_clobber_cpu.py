"""Inline-assembly blocks of the kernels that issue more than one load must
mark every output early-clobber ("=&v").

Without it the compiler may give an output the register of an input that a
later instruction of the same block still reads: the first load's data can
then land in the address register of the next load before that load issues,
which reads LDS at a data-dependent address.  (Seen in the small-M forward's
slot read: the 128-bit destination of the first ds_read covered the address
registers of the two following reads; results were wrong only on some runs
and builds.)"""

import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "nf4_bit_weight_amd", "csrc")
LOADS = ("ds_read", "buffer_load", "global_load", "flat_load", "scratch_load")


def _asm_blocks(text):
    """(template, outputs) of every `asm volatile(...)` statement."""
    out = []
    for m in re.finditer(r"asm\s+volatile\s*\(", text):
        i, depth = m.end(), 1
        while depth and i < len(text):
            depth += {"(": 1, ")": -1}.get(text[i], 0)
            i += 1
        parts = _split_outside_strings(text[m.end():i - 1])
        template = "".join(re.findall(r'"((?:[^"\\]|\\.)*)"', parts[0]))
        outputs = re.findall(r'"(=[^"]*)"', parts[1]) if len(parts) > 1 else []
        out.append((template, outputs))
    return out


def _split_outside_strings(body):
    """Split an asm statement's operands at the ':' that are not inside a string literal."""
    parts, cur, in_str, i = [], [], False, 0
    while i < len(body):
        c = body[i]
        if in_str and c == "\\":
            cur.append(body[i:i + 2])
            i += 2
            continue
        if c == '"':
            in_str = not in_str
        if c == ":" and not in_str:
            parts.append("".join(cur))
            cur = []
        else:
            cur.append(c)
        i += 1
    parts.append("".join(cur))
    return parts


def _sources():
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp")):
            with open(os.path.join(CSRC, name)) as f:
                # join macro continuation lines so a #define'd block reads as one statement
                yield name, f.read().replace("\\\n", "\n")


def test_multi_load_asm_outputs_are_early_clobber():
    checked = 0
    for name, text in _sources():
        for template, outputs in _asm_blocks(text):
            loads = sum(template.count(op) for op in LOADS)
            if loads >= 2 and outputs:
                checked += 1
                bad = [c for c in outputs if not c.startswith("=&")]
                assert not bad, f"{name}: block {template[:60]!r} has outputs {bad} without '&'"
    assert checked >= 4, "the slot and unit reads of the kernels were not found"


def test_asm_loads_wait_in_their_own_block():
    """An asm load whose result lands in a register must be waited for inside
    the same block: the compiler takes the output as written when the block
    ends, and could otherwise reuse or read that register while the load is
    still in flight."""
    checked = 0
    for name, text in _sources():
        for template, outputs in _asm_blocks(text):
            if outputs and any(op in template for op in LOADS):
                checked += 1
                last_load = max(template.rfind(op) for op in LOADS)
                assert "s_waitcnt" in template[last_load:], f"{name}: {template[:60]!r} returns before its loads land"
    assert checked >= 5


def test_checker_flags_a_plain_output():
    text = 'asm volatile("ds_read_b128 %0, %2\\n\\tds_read_b32 %1, %3" : "=v"(a), "=&v"(b) : "v"(p), "v"(q));'
    (template, outputs), = _asm_blocks(text)
    assert sum(template.count(op) for op in LOADS) == 2
    assert [c for c in outputs if not c.startswith("=&")] == ["=v"]
