"""The build's resource gate: every kernel's registers, spills and scratch are read from the code-object
metadata of the saved gfx950 assembly, and a spill or any scratch memory fails the build.  Checked on
a planted metadata block, and on the kernels built in this tree (if any)."""
import glob
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "exact_attention_head_amd"))
import build as B  # noqa: E402

META = """\t.text
kern_a:
\ts_endpgm
\t.amdgpu_metadata
---
amdhsa.kernels:
  - .agpr_count:     256
    .group_segment_fixed_size: 65536
    .name:           kern_a
    .private_segment_fixed_size: {scratch_a}
    .sgpr_count:     100
    .sgpr_spill_count: 12
    .vgpr_count:     512
    .vgpr_spill_count: {spill_a}
  - .agpr_count:     0
    .group_segment_fixed_size: 0
    .name:           kern_b
    .private_segment_fixed_size: 0
    .sgpr_count:     20
    .sgpr_spill_count: 0
    .vgpr_count:     32
    .vgpr_spill_count: 0
amdhsa.target:   amdgcn-amd-amdhsa--gfx950
amdhsa.version:
  - 1
  - 2
...
\t.end_amdgpu_metadata
"""


def _res(tmp_path, spill_a, scratch_a):
    p = tmp_path / "k.s"
    p.write_text(META.format(spill_a=spill_a, scratch_a=scratch_a))
    return B.kernel_resources(str(p))


def test_metadata_is_read_per_kernel(tmp_path):
    r = _res(tmp_path, 0, 0)
    assert set(r) == {"kern_a", "kern_b"}
    assert r["kern_a"] == dict(vgpr=512, agpr=256, sgpr=100, vgpr_spill=0, sgpr_spill=12, scratch=0, lds=65536)
    assert r["kern_b"]["vgpr"] == 32 and r["kern_b"]["lds"] == 0


def test_sgpr_spills_alone_pass(tmp_path):
    assert B.spills(_res(tmp_path, 0, 0)) == []


def test_vgpr_spill_or_scratch_fails(tmp_path):
    assert len(B.spills(_res(tmp_path, 14, 60))) == 1
    assert len(B.spills(_res(tmp_path, 0, 16))) == 1  # scratch without a counted spill (e.g. a stack array)
    assert "kern_a" in B.spills(_res(tmp_path, 3, 0))[0]


def test_built_kernels_do_not_spill():
    res = {}
    for s in glob.glob(os.path.join(ROOT, "exact_attention_head_amd", "_build", "*.s")):
        res.update(B.kernel_resources(s))
    assert B.spills(res) == []
