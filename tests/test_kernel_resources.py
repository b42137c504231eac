"""Register use of the built kernels, read on the CPU from the gfx950 code
object inside libattnres.so: no kernel spills registers to scratch memory,
and the row kernel fits the 128 VGPRs that let two 448-lane workgroups share
a compute unit.  A spill costs a stream of scratch traffic per lane beside
the row traffic the kernels are built around."""
import os
import re
import shutil
import subprocess

import pytest

from kimi_k3_attention_amd import build as kbuild

LLVM = "/opt/rocm/llvm/bin"


def _kernels(tmp_path):
    objdump, readelf = os.path.join(LLVM, "llvm-objdump"), os.path.join(LLVM, "llvm-readelf")
    if not (os.path.exists(objdump) and os.path.exists(readelf)):
        pytest.skip("ROCm LLVM tools not installed")
    if not os.path.exists(kbuild.LIB):
        kbuild.build()
    lib = tmp_path / "libattnres.so"
    shutil.copy(kbuild.LIB, lib)
    # Writes each offloaded code object next to the copy.
    subprocess.run([objdump, "--offloading", str(lib)], check=True, capture_output=True)
    objs = [p for p in tmp_path.iterdir() if "gfx950" in p.name]
    assert len(objs) == 1, [p.name for p in tmp_path.iterdir()]
    notes = subprocess.run([readelf, "--notes", str(objs[0])], check=True, capture_output=True,
                           text=True).stdout
    kernels = {}
    for block in re.split(r"\n\s+- \.agpr_count", notes)[1:]:
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        if name.endswith(".kd"):
            continue

        def field(key):
            m = re.search(rf"\.{key}:\s+(\d+)", block)
            return int(m.group(1)) if m else None
        kernels[name] = dict(vgprs=field("vgpr_count"), spills=field("vgpr_spill_count"),
                             scratch=field("private_segment_fixed_size"))
    assert kernels, "no kernel metadata found"
    return kernels


def test_no_kernel_spills_to_scratch(tmp_path):
    ks = _kernels(tmp_path)
    bad = {n: k for n, k in ks.items() if k["scratch"] or k["spills"]}
    assert not bad, bad


def test_row_kernel_fits_two_workgroups_per_cu(tmp_path):
    ks = _kernels(tmp_path)
    row = {n: k for n, k in ks.items() if "attnres_row_kernel" in n}
    # nb 0..8 x (delta, norm); cached variants at nb >= 1; ranged ones at nb >= 2
    assert len(row) == 9 * 4 + 8 * 4 + 7 * 4
    assert all(k["vgprs"] <= 128 for k in row.values()), row


def test_any_h_staged_variants_fit_one_more_workgroup_per_cu(tmp_path):
    """The any-H kernel with three bank rows staged in LDS exists to fit one
    more workgroup per compute unit: at two segments per lane four 5-wave
    workgroups need at most 96 VGPRs (five waves per SIMD) and four 6-wave
    ones at most 80 (six); at four segments two 5- or 6-wave ones at most
    168 (three)."""
    ks = _kernels(tmp_path)
    stg = {n: k for n, k in ks.items()
           if "attnres_anyh_kernel" in n and "Li3ELb" in n[-30:]}
    five = {n: k for n, k in stg.items()
            if "anyh_kernelILi2E" in n and n.endswith("Li3ELb0EEEvNS0_7KParamsE")}
    six = {n: k for n, k in stg.items()
           if "anyh_kernelILi2E" in n and n.endswith("Li3ELb1EEEvNS0_7KParamsE")}
    four = {n: k for n, k in stg.items() if "anyh_kernelILi4E" in n}
    # each: masked or not x nb 4..8 x (delta, norm, cached)
    assert len(five) == len(six) == len(four) == 2 * 5 * 8 and len(stg) == 3 * 80, len(stg)
    assert all(k["vgprs"] <= 96 for k in five.values()), five
    assert all(k["vgprs"] <= 80 for k in six.values()), six
    assert all(k["vgprs"] <= 168 for k in four.values()), four
