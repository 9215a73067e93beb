"""The build's check of the decode kernels' gfx950 assembly: the O-block-15 accumulator of
the VGPR-form MFMA is named by no other instruction while the MFMA may be in flight.
Hand-written assembly snippets with planted breaches pin the checker; then the checker runs
on the assembly of the current decode source (CPU only: the compiler's output is read,
nothing is run)."""

from __future__ import annotations

import os
import subprocess
import tempfile

import pytest

from sparse_mla_decode_03_amd import asm_checks as A

MFMA = "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], v[0:15]"
DRAIN = "\ts_nop 7\n\ts_nop 7\n\ts_nop 7"


def _kernel(body: str) -> str:
    return f"_Z6kernelv:\n{body}\n\ts_endpgm\n.Lfunc_end0:\n"


GOOD = _kernel(f"""\tv_mov_b32 v0, 0
.LBB0_1:
\tds_read_b128 v[20:23], v30
\tv_add_u32 v31, 1, v31
{MFMA}
\ts_cbranch_scc1 .LBB0_1
{DRAIN}
\tv_mul_f32 v40, v41, v0""")


def test_clean_kernel_passes():
    assert A.vgpr_mfma_violations(GOOD) == []
    assert A.count_vgpr_mfma_kernels(GOOD) == 1


def test_read_before_the_drain_is_caught():
    bad = GOOD.replace(f"{DRAIN}\n\tv_mul_f32 v40, v41, v0", f"\tv_mul_f32 v40, v41, v0\n{DRAIN}")
    assert any("v_mul_f32 v40, v41, v0" in m for m in A.vgpr_mfma_violations(bad))


def test_loop_carried_move_is_caught():
    # the copy sits before the MFMA in instruction order but runs after it on the back edge
    bad = GOOD.replace("\tds_read_b128 v[20:23], v30", "\tds_read_b128 v[20:23], v30\n\tv_mov_b32 v50, v7")
    assert any("v_mov_b32 v50, v7" in m for m in A.vgpr_mfma_violations(bad))


def test_out_of_order_layout_is_followed():
    # the epilogue block is laid out before the loop; the loop exits to it without a drain
    bad = _kernel(f"""\ts_branch .LBB0_2
.LBB0_1:
\tv_mul_f32 v40, v41, v3
\ts_endpgm
.LBB0_2:
{MFMA}
\ts_cbranch_scc1 .LBB0_2
\ts_branch .LBB0_1""")
    assert any("v_mul_f32 v40, v41, v3" in m for m in A.vgpr_mfma_violations(bad))
    fixed = bad.replace("\ts_branch .LBB0_1", f"{DRAIN}\n\ts_branch .LBB0_1")
    assert A.vgpr_mfma_violations(fixed) == []


def test_range_overlap_and_in_place_rules():
    assert A.vgpr_mfma_violations(GOOD.replace("v_add_u32 v31, 1, v31", "v_add_u32 v31, 1, v[14:15]"))
    assert not A.vgpr_mfma_violations(GOOD.replace("v_add_u32 v31, 1, v31", "v_add_u32 v31, 1, v[16:17]"))
    not_in_place = GOOD.replace(MFMA, "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], v[32:47]")
    assert any("in place" in m for m in A.vgpr_mfma_violations(not_in_place))
    two = GOOD.replace(DRAIN, MFMA.replace("v[0:15]", "v[32:47]") + "\n" + DRAIN)
    assert any("ranges" in m for m in A.vgpr_mfma_violations(two))


def test_current_decode_assembly_is_clean():
    from sparse_mla_decode_03_amd import build as b
    try:
        b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as td:
        path = os.path.join(td, "smla_decode.s")
        res = subprocess.run(b.decode_asm_command(path), capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        text = open(path).read()
    # kernels with three and four waves, for each of the three cache formats: both epilogues
    # of the positional splits (output or documented partials; the merge's own split format)
    # and the balanced rows' kernel (either epilogue, by each row's split count)
    assert A.count_vgpr_mfma_kernels(text) == 18
    assert A.vgpr_mfma_violations(text) == []
