"""Properties of the built device code that the tests on the card cannot see
(CPU; reads the gfx950 code objects of the in-tree libsattn.so with the ROCm
disassembler):

* no packed fp32 arithmetic (v_pk_add_f32, v_pk_mul_f32, v_pk_fma_f32): the
  library is built with that target feature off, and no source writes them;
* no stores, atomics, write-backs or discards through the scalar data cache;
  every global or LDS write is a vector instruction;
* no kernel spills to scratch (private segment size 0), and every kernel's
  LDS fits the 160 KiB of a CU;
* the split-key kernel's direct-to-LDS loads set M0 themselves, one wait
  state before each load.
"""
import glob
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "causal_attention_forward_amd", "libsattn.so")
LLVM = "/opt/rocm/llvm/bin"


@pytest.fixture(scope="module")
def code_objects():
    if not os.path.exists(LIB):
        pytest.skip("libsattn.so not built")
    if not os.path.exists(os.path.join(LLVM, "llvm-objdump")):
        pytest.skip("ROCm llvm-objdump not available")
    d = tempfile.mkdtemp()
    try:
        shutil.copy(LIB, os.path.join(d, "lib.so"))
        subprocess.run([os.path.join(LLVM, "llvm-objdump"), "--offloading", "lib.so"], cwd=d,
                       check=True, capture_output=True)
        objs = sorted(glob.glob(os.path.join(d, "lib.so.*gfx950*")))
        assert objs, "no gfx950 code object in libsattn.so"
        asm = "".join(subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--no-show-raw-insn", o],
                                     check=True, capture_output=True, text=True).stdout for o in objs)
        notes = "".join(subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", o],
                                       check=True, capture_output=True, text=True).stdout for o in objs)
        yield asm, notes
    finally:
        shutil.rmtree(d)


def mnemonics(asm):
    out = []
    for line in asm.splitlines():
        m = re.match(r"\s+([a-z_0-9]+)\b", line)
        if m:
            out.append(m.group(1))
    return out


def test_no_packed_fp32(code_objects):
    asm, _ = code_objects
    bad = {m for m in mnemonics(asm) if m in ("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32")}
    assert not bad, bad


def test_no_scalar_cache_writes(code_objects):
    asm, _ = code_objects
    pat = re.compile(r"^s_(store|buffer_store|scratch_store|atomic|buffer_atomic|dcache_wb|dcache_discard)")
    bad = {m for m in mnemonics(asm) if pat.match(m)}
    assert not bad, bad


def test_no_spills_and_lds_fits(code_objects):
    _, notes = code_objects
    names = re.findall(r"\.name:\s+(\S+)", notes)
    kernels = [n for n in names if "sattn" in n]
    assert len(kernels) >= 20, kernels
    priv = [int(v) for v in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", notes)]
    lds = [int(v) for v in re.findall(r"\.group_segment_fixed_size:\s+(\d+)", notes)]
    assert priv and max(priv) == 0, priv
    assert lds and max(lds) <= 160 * 1024, lds


def test_lds_loads_set_m0_first(code_objects):
    asm, _ = code_objects
    lines = [l.strip() for l in asm.splitlines()]
    hits = 0
    for i, l in enumerate(lines):
        if re.match(r"buffer_load_dword\w* .* lds\b", l):
            hits += 1
            assert lines[i - 1].startswith("s_nop"), lines[i - 2:i + 1]
            assert lines[i - 2].startswith("s_mov_b32 m0,"), lines[i - 2:i + 1]
    assert hits > 0
