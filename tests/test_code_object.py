"""Properties of the built gfx950 code object (CPU only: reads the kernel
descriptors' metadata from libsfmla.so, runs nothing).

The 8-wave forward kernels run at the 256-VGPR limit of two waves per SIMD.  At
that limit the compiler may move a private array into scratch memory, which
makes every access a memory round trip (an output copy demoted this way once
cost the separate-V forward 15 us of 75).  These checks fail the build
instead of the timing.  The disassembly checks read the AMD assembly of this
repository's own build.
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


OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"


@pytest.fixture(scope="module")
def disasm():
    """Instruction lines of every kernel in this repository's own gfx950
    build (the AMD assembly of code built here), keyed by symbol."""
    if not os.path.exists(LIB):
        pytest.skip("libsfmla.so not built")
    if not os.path.exists(OBJDUMP):
        pytest.skip("llvm-objdump not available")
    with open(LIB, "rb") as f:
        co = _gfx950_object(f.read())
    with tempfile.NamedTemporaryFile(suffix=".co", delete=False) as t:
        t.write(co)
    try:
        out = subprocess.run([OBJDUMP, "-d", "--no-show-raw-insn", t.name], capture_output=True,
                             text=True, check=True).stdout
    finally:
        os.unlink(t.name)
    res, cur = {}, None
    for ln in out.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:$", ln)
        if m:
            cur = res.setdefault(m.group(1), [])
        elif cur is not None and ln.strip():
            cur.append(ln.strip())
    assert res, "no kernels disassembled"
    return res


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


FWD_NAME = (r"_ZN5sfmla10fwd_kernelILi(\d+)ELi(\d)ELi(\d+)ELi(\d)ELi(\d)ELb(\d)ELb(\d)EEEv"
            r"NS_7FwdArgsE")


def _key(m):
    """(waves, d_qk, separate V, format, query tiles, wave pairs); every
    wave holds one 16-head block"""
    waves, hb, dqk, vmode, fmt, tiled, pair = (int(x) for x in m.groups())
    assert hb == 1, m.group(0)
    return (waves, dqk, vmode, fmt, tiled, pair)


def _fwd(kernels):
    """fwd_kernel instantiations as (waves, d_qk, separate V, format, query
    tiles, wave pairs) -> fields."""
    res = {}
    for name, f in kernels.items():
        m = re.fullmatch(FWD_NAME, name)
        if m:
            res[_key(m)] = f
    return res


def _eight_wave_packed(key):
    """The eight-wave packed kernel runs two waves per SIMD at the 256-register
    limit; with FP8 codes and rope a couple of values may spill outside the
    tile loop (bounded here: at most 40 registers, 128 bytes per lane)."""
    return key[0] == 8 and key[3] in (1, 2)


def test_every_forward_variant_is_built(kernels):
    fwd = _fwd(kernels)
    # bf16 / float16 rows: d_qk 512 or 576, V shared or separate, one query
    # row per workgroup or query tiles
    for fmt in (0, 3):
        for dqk in (512, 576):
            for vmode in (0, 1):
                for tiled in (0, 1):
                    assert (8, dqk, vmode, fmt, tiled, 0) in fwd
                # eight waves in four pairs (never tiled)
                assert (8, dqk, vmode, fmt, 0, 1) in fwd
                assert (8, dqk, vmode, fmt, 1, 1) not in fwd
        # four waves, two workgroups per CU: d_qk 512 with V = K nope only
        assert (4, 512, 0, fmt, 0, 0) in fwd
        assert (4, 576, 0, fmt, 0, 0) not in fwd and (4, 512, 1, fmt, 0, 0) not in fwd
    # packed INT8 / FP8 rows, with and without rope, V the key codes or a
    # value tensor of codes, on eight waves, with and without wave pairs
    # (never tiled)
    for fmt in (1, 2):
        for dqk in (512, 576):
            for vmode in (0, 1):
                assert (8, dqk, vmode, fmt, 0, 0) in fwd
                assert (8, dqk, vmode, fmt, 0, 1) in fwd
                assert (4, dqk, vmode, fmt, 0, 0) not in fwd
                assert (8, dqk, vmode, fmt, 1, 0) not in fwd
    assert any("plan_kernel" in k for k in kernels)
    assert any("combine_kernel" in k for k in kernels)


def test_forward_kernels_fit_their_waves_per_simd_and_the_lds(kernels):
    # one workgroup per CU: 8 waves are two per SIMD (256 VGPRs each)
    for key, f in _fwd(kernels).items():
        waves = key[0]
        assert f["max_flat_workgroup_size"] == 64 * waves, key
        assert f["vgpr_count"] <= 2048 // waves, (key, f)
        assert f["group_segment_fixed_size"] <= LDS_BYTES, key
        if waves == 4 and key[3] in (0, 3):
            # the 16-bit four-wave kernel runs two workgroups per CU
            assert f["vgpr_count"] <= 256 and 2 * f["group_segment_fixed_size"] <= LDS_BYTES, (key, f)


def test_forward_kernels_use_no_scratch_in_the_main_loop(kernels, disasm):
    """The tile loop (every MFMA of a forward kernel) touches no scratch
    memory; spills outside it (prologue, merge) stay few, and the headline's
    instantiation (bf16, rope, separate V) has none at all."""
    fwd = _fwd(kernels)
    for key, f in fwd.items():
        if key == (8, 576, 1, 0, 0, 0):
            assert f["vgpr_spill_count"] == 0 and f["private_segment_fixed_size"] == 0, (key, f)
        if _eight_wave_packed(key):
            assert f["vgpr_spill_count"] <= 40 and f["private_segment_fixed_size"] <= 128, (key, f)
        else:
            assert f["vgpr_spill_count"] <= 16 and f["private_segment_fixed_size"] <= 64, (key, f)
    found = 0
    for name, body in disasm.items():
        m = re.fullmatch(FWD_NAME, name)
        if not m:
            continue
        found += 1
        mf = [i for i, ln in enumerate(body) if "v_mfma" in ln]
        assert mf, name
        loop = body[mf[0]:mf[-1] + 1]
        bad = [ln for ln in loop if "scratch_" in ln or "buffer_load_dword" in ln and "off, s[0:3]" in ln]
        assert not bad, (name, bad[:3])
    assert found == len(fwd)


def test_lds_dma_reads_m0_only_as_an_input(disasm):
    """Every LDS DMA in the kernels follows the wait state its inline asm
    carries, and M0 is only ever written by plain moves or adds (the
    compiler's, for the DMA's operand), never inside the DMA sequences."""
    n = 0
    for name, body in disasm.items():
        for i, ln in enumerate(body):
            if "global_load_lds_dwordx4" in ln:
                n += 1
                assert "s_nop" in body[i - 1], (name, body[i - 2:i + 1])
            if re.search(r"\bs_\w+\s+m0\b", ln):
                assert re.search(r"\bs_(mov|add|sub|lshl|or|mul)\w*\s+m0\b", ln), (name, ln)
    assert n > 0


def test_no_inline_asm_load_writes_a_register():
    """Inline-asm loads are allowed only where they write LDS (the DMA
    gathers).  A load the compiler does not track that writes a VGPR lands
    asynchronously in a register the compiler believes it already holds; the
    compiler may spill or reuse that register before the data arrives (an
    address register overwritten this way made a build of the forward kernel
    access memory out of bounds).  Every register load is an ordinary one."""
    src = open(os.path.join(ROOT, "sparse_shared_kv_amd", "csrc", "sfmla_kernels.hip")).read()
    for m in re.finditer(r'asm\s+volatile\s*\(\s*"([^"]*)"\s*:\s*([^:;]*)', src):
        text, outs = m.group(1), m.group(2)
        if re.search(r"\b(global|buffer|flat|scratch)_load", text):
            assert "global_load_lds" in text and "=v" not in outs, text
