"""The build-time hazard check on the kernels' generated assembly: each rule catches a planted violation,
accepts the correctly padded form, and the kernels built in this tree (if any) are clean."""
import glob
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "exact_attention_head_amd"))
import check_mfma_hazards as H  # noqa: E402


def _check(tmp_path, body):
    p = tmp_path / "k.s"
    p.write_text("kern:\n" + "\n".join("\t" + l if not l.endswith(":") else l for l in body) + "\n\ts_endpgm\n")
    return H.check(str(p))


MFMA = "v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]"


def test_mfma_result_read_too_early(tmp_path):
    assert _check(tmp_path, [MFMA, "s_nop 7", "v_accvgpr_read_b32 v10, a3"])  # 8 wait states < 12
    assert not _check(tmp_path, [MFMA, "s_nop 7", "s_nop 3", "v_accvgpr_read_b32 v10, a3"])  # 12


def test_fp8_product_needs_twenty_wait_states(tmp_path):
    f8 = "v_mfma_f32_32x32x64_f8f6f4 v[0:15], v[16:23], v[24:31], v[0:15]"
    assert _check(tmp_path, [f8, "s_nop 7", "s_nop 3", "v_mov_b32 v40, v3"])  # 12 < 20
    assert not _check(tmp_path, [f8, "s_nop 7", "s_nop 7", "s_nop 3", "v_mov_b32 v40, v3"])  # 20


def test_same_destination_accumulation_is_allowed(tmp_path):
    assert not _check(tmp_path, [MFMA, MFMA])
    # a different accumulator overlapping the first destination is not
    assert _check(tmp_path, [MFMA, "v_mfma_f32_32x32x16_bf16 a[8:23], v[0:3], v[4:7], a[8:23]"])


def test_mfma_result_overwritten_too_early(tmp_path):
    assert _check(tmp_path, [MFMA, "s_nop 4", "v_accvgpr_write_b32 a15, v1"])


def test_valu_write_then_mfma_operand(tmp_path):
    assert _check(tmp_path, ["v_mov_b32 v5, 0", MFMA])
    assert not _check(tmp_path, ["v_mov_b32 v5, 0", "s_nop 1", MFMA])


def test_transposed_read_needs_covering_wait(tmp_path):
    tr = "ds_read_b64_tr_b16 v[20:21], v30 offset:64"
    assert _check(tmp_path, [tr, "v_mov_b32 v40, v20"])
    assert _check(tmp_path, [tr, "ds_read_b128 v[50:53], v31", "s_waitcnt lgkmcnt(2)", "v_mov_b32 v40, v20"])
    assert not _check(tmp_path, [tr, "ds_read_b128 v[50:53], v31", "s_waitcnt lgkmcnt(1)", "v_mov_b32 v40, v20"])
    assert not _check(tmp_path, [tr, "s_waitcnt lgkmcnt(0)", "v_mov_b32 v40, v20"])


def test_any_lds_read_needs_covering_wait(tmp_path):
    # operand fragments read by inline assembly: a later read may not reuse the registers of one
    # that is still in flight, nor may a product consume them early
    rd = "ds_read_b128 v[164:167], v178 offset:0x8000"
    assert _check(tmp_path, [rd, "ds_read_b128 v[164:167], v177 offset:0x9000"])
    assert _check(tmp_path, [rd, "ds_read_b128 v[160:163], v182", "s_waitcnt lgkmcnt(2)",
                             "v_mfma_f32_32x32x16_bf16 v[0:15], v[164:167], v[36:39], v[0:15]"])
    assert not _check(tmp_path, [rd, "ds_read_b128 v[160:163], v182", "s_waitcnt lgkmcnt(1)",
                                 "v_mfma_f32_32x32x16_bf16 v[0:15], v[164:167], v[36:39], v[0:15]",
                                 "ds_read_b128 v[164:167], v177 offset:0x9000"])


def test_state_survives_branches_and_loop_back_edges(tmp_path):
    # the hazard sits on the taken path only
    assert _check(tmp_path, [MFMA, "s_cbranch_scc1 .LBB0_2", "s_nop 7", "s_nop 7", ".LBB0_2:",
                             "v_accvgpr_read_b32 v10, a0"])
    # an MFMA at the loop's end reaches the read at its head through the back edge
    assert _check(tmp_path, [".LBB0_1:", "v_accvgpr_read_b32 v10, a0", "s_nop 7", "s_nop 7", MFMA,
                             "s_cbranch_scc1 .LBB0_1"])


def test_built_kernels_are_clean():
    files = sorted(glob.glob(os.path.join(ROOT, "exact_attention_head_amd", "_build", "**", "*.s"), recursive=True))
    if not files:
        pytest.skip("no kernel assembly in the tree (build first)")
    bad = []
    for f in files:
        bad += H.check(f)
    assert not bad, bad[:5]
