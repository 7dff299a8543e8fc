"""The built kernels leave two wait states between a vector write of an SGPR
pair and a vector read of it as a mask or carry (gfx950), including reads in
inline asm, which the compiler does not pad.  Runs on the CPU: it compiles
the sources to gfx950 assembly and scans it."""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import pytest

import isa_check

SNIPPET = """_Zkernel:
\tv_cmp_le_f32_e64 s[0:1], v1, v2
\tv_addc_co_u32_e64 v3, s[0:1], v3, v3, s[0:1]
\tv_cmp_le_f32_e64 s[2:3], v1, v2
\ts_nop 1
\tv_addc_co_u32_e64 v3, s[2:3], v3, v3, s[2:3]
\tv_cmp_gt_f32_e64 s[4:5], v1, v2
\ts_or_b64 s[4:5], s[4:5], s[6:7]
\tv_cndmask_b32_e64 v5, v6, v7, s[4:5]
\tv_cmp_gt_f32_e32 vcc, v1, v2
\tv_mov_b32_e32 v8, v9
\tv_cndmask_b32_e32 v5, v6, v7, vcc
"""


def test_scanner_finds_planted_reads():
    found = isa_check.close_mask_reads(SNIPPET)
    # the immediate read (distance 0) and the vcc read one instruction later; the padded
    # read and the one behind a scalar write are fine
    assert [(d, t.split()[0]) for _, t, d in found] == [(0, "v_addc_co_u32_e64"), (1, "v_cndmask_b32_e32")]


SOURCES = ["quest_grids.hip", "quest_fwd_nodq.hip", "quest_fwd_op.hip"]


@pytest.fixture(scope="module")
def assembly():
    with ThreadPoolExecutor(len(SOURCES)) as pool:
        return dict(zip(SOURCES, pool.map(isa_check.compile_asm, SOURCES)))


@pytest.mark.parametrize("source", SOURCES)
def test_no_close_mask_reads(assembly, source):
    found = isa_check.close_mask_reads(assembly[source])
    assert not found, f"{len(found)} reads too close to their write, first: {found[0]}"
