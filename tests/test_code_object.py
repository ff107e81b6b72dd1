"""Properties of the built gfx950 code object (CPU only: reads the kernel
descriptors' metadata from libsfmla.so, runs nothing).

The 8-wave forward kernels run at the 256-VGPR limit of two waves per SIMD.  At
that limit the compiler may move a private array into scratch memory, which
makes every access a memory round trip (an output copy demoted this way once
cost the separate-V forward 15 us of 75).  These checks fail the build
instead of the timing.
"""

import os
import re
import shutil
import struct
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "sparse_shared_kv_amd", "libsfmla.so")
READELF = "/opt/rocm/llvm/bin/llvm-readelf"
LDS_BYTES = 160 * 1024


def _gfx950_object(blob):
    """The gfx950 entry of the clang offload bundle embedded in the library."""
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    base = blob.find(magic)
    assert base >= 0, "no offload bundle in libsfmla.so"
    p = base + len(magic)
    (n,) = struct.unpack_from("<Q", blob, p)
    p += 8
    for _ in range(n):
        off, size, tlen = struct.unpack_from("<QQQ", blob, p)
        p += 24
        triple = blob[p:p + tlen].decode()
        p += tlen
        if triple.endswith("gfx950"):
            return blob[base + off:base + off + size]
    raise AssertionError("no gfx950 code object in the bundle")


@pytest.fixture(scope="module")
def kernels():
    if not os.path.exists(LIB):
        pytest.skip("libsfmla.so not built")
    if not os.path.exists(READELF) and not shutil.which("llvm-readelf"):
        pytest.skip("llvm-readelf not available")
    with open(LIB, "rb") as f:
        co = _gfx950_object(f.read())
    with tempfile.NamedTemporaryFile(suffix=".co", delete=False) as t:
        t.write(co)
    try:
        exe = READELF if os.path.exists(READELF) else shutil.which("llvm-readelf")
        notes = subprocess.run([exe, "--notes", t.name], capture_output=True, text=True,
                               check=True).stdout
    finally:
        os.unlink(t.name)
    out = {}
    # one metadata block per kernel, each starting at its argument list
    for blk in notes.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", blk).group(1)
        fields = {k: int(v) for k, v in re.findall(
            r"\.(private_segment_fixed_size|vgpr_spill_count|vgpr_count|"
            r"group_segment_fixed_size|max_flat_workgroup_size):\s+(\d+)", blk)}
        out[name] = fields
    assert out, "no kernel metadata found"
    return out


def _fwd(kernels):
    """fwd_kernel instantiations as (waves, d_qk, separate V, format) -> fields."""
    res = {}
    for name, f in kernels.items():
        m = re.fullmatch(r"_ZN5sfmla10fwd_kernelILi(\d+)ELi1ELi(\d+)ELi(\d)ELi(\d)EEEvNS_7FwdArgsE",
                         name)
        if m:
            res[tuple(int(x) for x in m.groups())] = f
    return res


def test_every_forward_variant_is_built(kernels):
    fwd = _fwd(kernels)
    # bf16 / float16 rows: d_qk 512 or 576, V shared or separate
    for fmt in (0, 3):
        for dqk in (512, 576):
            for vmode in (0, 1):
                assert (8, dqk, vmode, fmt) in fwd
    # packed INT8 / FP8 rows, with and without rope
    for fmt in (1, 2):
        for dqk in (512, 576):
            assert (4, dqk, 0, fmt) in fwd
    assert any("plan_kernel" in k for k in kernels)
    assert any("combine_kernel" in k for k in kernels)


def test_forward_kernels_fit_their_waves_per_simd_and_the_lds(kernels):
    # one workgroup per CU: 8 waves are two per SIMD (256 VGPRs each), the
    # 4-wave packed kernel is one per SIMD (up to 512)
    for key, f in _fwd(kernels).items():
        waves = key[0]
        assert f["max_flat_workgroup_size"] == 64 * waves, key
        assert f["vgpr_count"] <= 2048 // waves, (key, f)
        assert f["group_segment_fixed_size"] <= LDS_BYTES, key


def test_forward_kernels_use_no_scratch(kernels):
    for key, f in _fwd(kernels).items():
        waves, dqk, vmode, fmt = key
        if waves == 8 and dqk == 576 and vmode == 0:
            # rope rows with V = K nope: a few values live across the main loop
            # are saved once before it and restored after it
            assert f["vgpr_spill_count"] <= 8 and f["private_segment_fixed_size"] <= 64, (key, f)
            continue
        assert f["private_segment_fixed_size"] == 0, (key, f)
        assert f["vgpr_spill_count"] == 0, (key, f)
