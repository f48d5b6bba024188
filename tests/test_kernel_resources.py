"""Resources of the built decode kernels, read from the gfx950 code objects in
libkvq.so (no GPU needed): the matrix-core and FP8 decode kernels use no
private (scratch) memory and spill nothing, and the kernels of the measured
workloads stay within the register budget of their planned occupancy.

Scratch in these kernels is never intended: the compiler puts a local array
on the stack when it is indexed with a per-lane value, and a stack load in the
page or residual-step loop waits on memory (the 2-bit decode at batch 16 x
4096 tokens ran 22.8 us with 32 bytes of scratch against 20.5 us without)."""

import os
import re
import shutil
import subprocess

import pytest

import kv_cache_quantisation_amd as kvq

LLVM = "/opt/rocm/llvm/bin"
BUNDLE = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def _tools():
    need = [shutil.which("objcopy"), os.path.join(LLVM, "clang-offload-bundler"),
            os.path.join(LLVM, "llvm-readelf")]
    if not need[0] or not all(os.path.exists(t) for t in need[1:]):
        pytest.skip("binutils / ROCm LLVM tools not available")
    return need


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    """{mangled kernel name: {metadata key: value}} over every code object."""
    objcopy, bundler, readelf = _tools()
    tmp = tmp_path_factory.mktemp("co")
    fat = tmp / "fatbin"
    # objcopy rewrites its input when given no output file: work on a copy, so
    # that the library a test process has mapped is never touched
    lib = tmp / "libkvq.so"
    shutil.copyfile(kvq.kvq.LIB_PATH, lib)
    subprocess.run([objcopy, "--dump-section", f".hip_fatbin={fat}", str(lib), str(tmp / "out.so")],
                   check=True)
    data = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(BUNDLE), data)]
    assert starts, "no offload bundles in libkvq.so"
    out = {}
    for i, s in enumerate(starts):
        one = tmp / f"b{i}"
        one.write_bytes(data[s:starts[i + 1] if i + 1 < len(starts) else len(data)])
        co = tmp / f"b{i}.co"
        r = subprocess.run([bundler, "--type=o", f"--targets={TARGET}", f"--input={one}",
                            f"--output={co}", "--unbundle"], capture_output=True)
        if r.returncode or not co.exists() or co.stat().st_size == 0:
            continue
        notes = subprocess.run([readelf, "--notes", str(co)], capture_output=True, text=True).stdout
        cur = {}
        for line in notes.splitlines():
            m = re.match(r"\s*\.(\w+):\s+(\S+)\s*$", line)
            if not m:
                continue
            key, val = m.groups()
            cur[key] = val
            if key == "vgpr_spill_count":   # last key of a kernel's entry
                out[cur["name"]] = dict(cur)
                cur = {}
    assert out, "no kernel metadata read"
    return out


def _family(kernels, stem):
    return {n: v for n, v in kernels.items() if stem in n}


@pytest.mark.parametrize("stem", ["kivi_mfma_kernel", "kivi_deq_kernel", "kivi_chunk_kernel", "rope4_kernel",
                                  "paged_mfma_kernel"])
def test_matrix_core_decodes_use_no_scratch(kernels, stem):
    fam = _family(kernels, stem)
    assert fam, stem
    bad = {n: (v["private_segment_fixed_size"], v["vgpr_spill_count"]) for n, v in fam.items()
           if int(v["private_segment_fixed_size"]) or int(v["vgpr_spill_count"])}
    assert not bad, bad


# kernels of the measured workloads: (mangled-name fragment, VGPR budget).
# Budgets: 512 registers per lane of a SIMD shared by its waves, allocated in
# granules of 8: two eight-wave blocks per CU (4 waves per SIMD) -> 128;
# three four-wave blocks (3 per SIMD) -> 168; one eight-wave block -> 256.
BUDGETS = [
    ("kivi_mfma_kernelILi2ELi2ELi128ELi4ELb0ELi1E", 128),   # KIVI 2-bit, GQA 4, d 128
    ("kivi_mfma_kernelILi4ELi2ELi128ELi4ELb0ELi1E", 256),   # 4-bit keys, 2-bit values (88 KB LDS)
    ("kivi_mfma_kernelILi4ELi4ELi128ELi4ELb0ELi1E", 168),   # KIVI 4-bit
    ("kivi_mfma_kernelILi2ELi2ELi128ELi4ELb0ELi2E", 256),   # 2-bit, two queries per block (one per CU)
    ("kivi_deq_kernelILi2ELi2ELi128E", 256),                # 2-bit, four queries per block, dequantised keys
    ("rope4_kernelILi128ELi4E", 168),                       # rotary keys, GQA 4
]


@pytest.mark.parametrize("frag,budget", BUDGETS)
def test_hot_decode_register_budget(kernels, frag, budget):
    fam = _family(kernels, frag)
    assert len(fam) == 1, list(fam)
    (name, meta), = fam.items()
    assert int(meta["vgpr_count"]) <= budget, (name, meta["vgpr_count"])
