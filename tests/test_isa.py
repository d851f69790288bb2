"""Properties of the compiled gfx950 kernels that their speed rests on, read from the assembly and
code-object metadata hipcc emits for the sources with the build's own flags (no GPU needed):

* FlashAssign (small-D and split-D): at most 168 VGPRs, so three waves share a SIMD; no spills and
  no scratch; at most a third of a CU's 160 KiB of LDS, so three workgroups share a CU; and no loop
  over lane values around a buffer access (a buffer descriptor that the compiler cannot keep in
  scalar registers turns every access through it into such a loop, whose signature is a 64-bit
  compare of descriptor words: v_cmp_eq_u64).
* The segmented reduction at the headline instance (2-byte rows of 128 elements, 16-byte loads,
  raw buffer gathers): at most 80 VGPRs, six waves per SIMD, no spills.
"""
import os
import re
import subprocess

import pytest

from exact_lloyd_means_02_amd import build as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not available")

LDS_THIRD = 160 * 1024 // 3


def _asm(src, tmp_path):
    out = tmp_path / (os.path.splitext(src)[0] + ".s")
    cmd = [B.HIPCC, *[f for f in B.FLAGS if f != "-fPIC"], *B.EXTRA.get(src, []), "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _kernels(asm, pattern):
    """{mangled name: (metadata dict, body)} for the kernels whose name matches `pattern`."""
    meta = {}
    for blk in asm.split("\n  - ")[1:]:
        m = re.search(r"\.name:\s+(\S+)", blk)
        if not m or not re.search(pattern, m.group(1)):
            continue
        meta[m.group(1)] = {k: int(v) for k, v in re.findall(
            r"\.(vgpr_count|agpr_count|vgpr_spill_count|sgpr_spill_count|private_segment_fixed_size|"
            r"group_segment_fixed_size):\s+(\d+)", blk)}
    out = {}
    for name, md in meta.items():
        start = asm.index(name + ":")
        out[name] = (md, asm[start:asm.index("s_endpgm", start)])
    return out


@pytest.fixture(scope="module")
def assign_asm(tmp_path_factory):
    d = tmp_path_factory.mktemp("isa")
    return _asm("k_assign.hip", d) + _asm("k_assign_d64.hip", d) + _asm("k_assign_d128.hip", d)


@pytest.fixture(scope="module")
def update_asm(tmp_path_factory):
    return _asm("k_update.hip", tmp_path_factory.mktemp("isa"))


def test_assign_kernels_three_waves_per_simd(assign_asm):
    ks = _kernels(assign_asm, r"assign_(small|split)_d_kernel")
    # every small-D instance (fp32 at padded D 8..128, 2-byte at 16..256, the D = 64 unit) and split-D
    assert len(ks) >= 16, sorted(ks)
    for name, (md, body) in ks.items():
        assert md["vgpr_count"] + md.get("agpr_count", 0) <= 168, (name, md)
        assert md["vgpr_spill_count"] == 0 and md["sgpr_spill_count"] == 0, (name, md)
        assert md["private_segment_fixed_size"] == 0, (name, md)
        assert md["group_segment_fixed_size"] <= LDS_THIRD, (name, md)
        assert "scratch_" not in body, name


def test_assign_buffer_descriptors_stay_scalar(assign_asm):
    for name, (_, body) in _kernels(assign_asm, r"assign_(small|split)_d_kernel").items():
        assert "v_cmp_eq_u64" not in body, name


def test_segsum_headline_instance_six_waves_per_simd(update_asm):
    ks = _kernels(update_asm, r"upd_segsum_kernelILi2ELi8ELi1ELb0ELb1E")
    assert len(ks) == 1, sorted(ks)
    (md, body), = ks.values()
    assert md["vgpr_count"] + md.get("agpr_count", 0) <= 80, md
    assert md["vgpr_spill_count"] == 0 and md["private_segment_fixed_size"] == 0, md
    assert "v_cmp_eq_u64" not in body
