"""CPU checks on the inline-assembly memory instructions in the HIP sources.

The compiler sees an asm block as opaque: it neither waits for the memory operations inside it nor inserts
the hardware's wait states after it.  The blocks in this library therefore follow three rules, checked here
on the source text:
  - a vector store of more than 8 bytes ends with `s_nop 1` or more: on gfx940 and later a VALU write to the
    store's data registers must wait 2 states, and the next instruction the compiler emits may be one;
  - an LDS-DMA load (global_load_lds_*) has no output operands: its data goes to LDS, and an asm output would
    be taken by the compiler as written at once while the load is still in flight;
  - M0 is written, then one wait state, before the LDS-DMA instruction that reads it.
"""
import os
import re

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "speculative_decoding_tree_parent_amd", "csrc")

# asm volatile("..." ... : clobbers);  -- the template string, then the operand sections
ASM_RE = re.compile(r'asm\s+volatile\s*\(\s*((?:"(?:[^"\\]|\\.)*"\s*)+)(.*?)\);', re.S)
WIDE_STORE_RE = re.compile(r"\b(global|buffer|flat)_store_dword(x3|x4)\b")
DMA_RE = re.compile(r"\bglobal_load_lds_dword")


def _asm_blocks():
    blocks = []
    for name in sorted(os.listdir(CSRC)):
        if not name.endswith((".hip", ".h")):
            continue
        with open(os.path.join(CSRC, name)) as f:
            text = f.read()
        for m in ASM_RE.finditer(text):
            template = "".join(re.findall(r'"((?:[^"\\]|\\.)*)"', m.group(1)))
            lines = [ln.strip() for ln in template.replace("\\n", "\n").replace("\\t", "").split("\n") if ln.strip()]
            blocks.append((name, lines, m.group(2)))
    return blocks


BLOCKS = _asm_blocks()


def test_sources_have_asm_memory_blocks():
    assert any(DMA_RE.search(" ".join(lines)) for _, lines, _ in BLOCKS)
    assert any(WIDE_STORE_RE.search(" ".join(lines)) for _, lines, _ in BLOCKS)


@pytest.mark.parametrize("name,lines,ops", [b for b in BLOCKS if WIDE_STORE_RE.search(" ".join(b[1]))])
def test_wide_store_blocks_end_with_two_wait_states(name, lines, ops):
    last = lines[-1]
    m = re.fullmatch(r"s_nop\s+(\d+)", last)
    assert m and int(m.group(1)) >= 1, f"{name}: store block must end with s_nop 1 or more: {lines}"


@pytest.mark.parametrize("name,lines,ops", [b for b in BLOCKS if DMA_RE.search(" ".join(b[1]))])
def test_lds_dma_blocks_have_no_outputs_and_set_m0_first(name, lines, ops):
    assert ops.lstrip().startswith("::"), f"{name}: LDS-DMA asm must have no output operands: {ops[:60]}"
    i = next(k for k, ln in enumerate(lines) if DMA_RE.search(ln))
    assert i >= 2 and lines[0].startswith("s_mov_b32 m0") and re.fullmatch(r"s_nop\s+\d+", lines[i - 1]), \
        f"{name}: M0 write and one wait state must precede the DMA: {lines}"
    assert '"m0"' in ops, f"{name}: M0 must be listed as clobbered"


# ------------------------------------------------------------------ counted wait in the split-KV prologue
# The prologue of a split-KV segment issues, per wave, one LDS-DMA load of the first tile's page-table slice and
# then its share of the query tile's DMA instructions (instruction ins = wave + 4k while ins * 64 lanes < the
# tile's 16-byte chunks), and waits with `s_waitcnt vmcnt(QINS / 4)` before reading the slice.  Loads complete in
# issue order, so the slice has landed once at most QINS / 4 loads are outstanding -- provided every wave issued
# at least QINS / 4 query instructions after it.  Checked for both compiled shapes (the source's constants are
# read from the text so that a change there shows up here).
def _segment_prologue_text():
    with open(os.path.join(CSRC, "verify.hip")) as f:
        text = f.read()
    start = text.index("void splitkv_segment(")
    return text[start:text.index("seg_body<R, DR>(", start)]


def test_prologue_counted_wait_is_where_the_argument_needs_it():
    t = _segment_prologue_text()
    pt = t.index("dma4_lane_addr(page_table")           # the page-table slice load ...
    q = t.index("dma16_lane_addr(q_cat")                 # ... then the query-tile loads ...
    w = t.index("wait_vmem_below<QINS / 4>();")          # ... then the counted wait ...
    r = t.index("const int slot0 = pt_s[lane];")         # ... then the read of the slice
    assert pt < q < w < r
    assert "constexpr int QINS = (M_TILE * (DQ / 8) + 63) / 64;" in t
    assert "const int ins = wave + 4 * k, pos = ins * 64 + lane;" in t
    assert "if (ins * 64 < M_TILE * QC) {" in t


@pytest.mark.parametrize("R,DR", [(512, 64), (64, 16)])
def test_prologue_counted_wait_covers_the_page_table_slice(R, DR):
    M_TILE, waves = 64, 4
    QC = (R + DR) // 8                       # 16-byte chunks of a query row
    QINS = (M_TILE * QC + 63) // 64          # query-tile DMA instructions of the workgroup
    QN = (M_TILE * QC + 255) // 256          # loop trips per wave
    issued = [sum(1 for k in range(QN) if (w + 4 * k) * 64 < M_TILE * QC) for w in range(waves)]
    assert sum(issued) == QINS
    assert min(issued) >= QINS // 4, (issued, QINS // 4)
