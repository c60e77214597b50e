"""Guard of the prefill tile kernel's hand-counted memory waits (CPU only).

gemm_tile_kernel copies both operands into LDS with the buffer unit's LDS-DMA
and waits for a group's copies with an explicit `s_waitcnt vmcnt(N)` before a
bare `s_barrier`. Each N is a compile-time count of the loads and stores the
wave issued after the ones it waits for: every group issues NCOPY = 2 + TPW
copies (two activation fragments, TPW code tiles), every item TPW scale loads,
one row-index load, one gather-index load and NST epilogue stores. The counts
hold only while the compiler emits exactly those memory instructions. This
test reads the gfx950 code object of the built library (our own build) and
checks, for every tile-kernel instance:
  * no scratch (spill) instruction, whose loads and stores would enter the
    same counter;
  * no vector-memory instruction outside the designed set (LDS-DMA 16-byte
    copies, the scale / index loads, 16-byte stores, the expert-offset loads
    of the table built at the start);
  * every LDS-DMA copy is one 16-byte instruction with no instruction offset
    (an offset would move the LDS destination too);
  * the vmcnt of every wait that precedes a barrier is one of the design's
    counts for that instance, and each of them occurs.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "w4a16_grouped_gemm_amd", "libmoe_w4a16.so")
LLVM = "/opt/rocm/llvm/bin"
BUNDLER = os.path.join(LLVM, "clang-offload-bundler")
OBJDUMP = os.path.join(LLVM, "llvm-objdump")

# (KIND, waves, subtiles) of the instantiated tile kernels
INSTANCES = [(0, 8, 4), (1, 8, 4), (0, 4, 2), (1, 4, 2)]
TPW = 4                                   # tiles per wave


def symbol(kind, waves, ns):
    return f"_ZN3moe12_GLOBAL__N_116gemm_tile_kernelILi{kind}ELi{waves}ELi{ns}EEEvNS0_8GemmArgsE"


def design_waits(kind, ns):
    """The wait counts the kernel source is written for."""
    ncopy = 2 + TPW
    cs = 16 * ns                          # rows per item
    swiglu = kind == 0
    cols = 8 if swiglu else 16            # output columns per tile
    halves = 1 if swiglu else 2
    ocols = (TPW // halves) * cols
    rpp = 64 // (ocols * 2 // 16)         # rows per store pass
    nst = halves * (cs // rpp)            # stores per wave and item
    return {2 * ncopy + TPW + 2 + nst,    # before group 0
            ncopy + TPW + 2 + nst,        # before group 1
            ncopy,                        # groups 2 .. G-2
            2 * ncopy,                    # the last group
            nst}                          # after the epilogue


def code_objects(tmp_path):
    """The gfx950 code objects of every source file of the library."""
    fat = tmp_path / "fat.bin"
    r = subprocess.run(["objcopy", "--dump-section", f".hip_fatbin={fat}", LIB, str(tmp_path / "lib.copy")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    data = fat.read_bytes()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    starts = [m.start() for m in re.finditer(re.escape(magic), data)]
    assert starts, "no offload bundle in the library"
    out = []
    for n, (a, b) in enumerate(zip(starts, starts[1:] + [len(data)])):
        part = tmp_path / f"b{n}.bin"
        part.write_bytes(data[a:b])
        co = tmp_path / f"b{n}.co"
        r = subprocess.run([BUNDLER, "--type=o", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={part}",
                            f"--output={co}", "--unbundle"], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        out.append(co)
    return out


def disassemble(cos, sym):
    for co in cos:
        d = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", f"--disassemble-symbols={sym}", str(co)],
                           capture_output=True, text=True).stdout
        if f"<{sym}>:" in d:
            return d
    raise AssertionError(f"{sym} not found in the library")


def instructions(dis):
    out = []
    for line in dis.split("\n"):
        m = re.match(r"^\s+([a-z][a-z0-9_]*)\b(.*?)(//.*)?$", line)
        if m:
            out.append((m.group(1), m.group(2)))
    return out


@pytest.mark.skipif(not (os.path.exists(LIB) and os.path.exists(BUNDLER) and os.path.exists(OBJDUMP)
                         and shutil.which("objcopy")), reason="needs the built library and the ROCm LLVM tools")
@pytest.mark.parametrize("kind,waves,ns", INSTANCES)
def test_tile_kernel_memory_waits_match_design(kind, waves, ns, tmp_path):
    ins = instructions(disassemble(code_objects(tmp_path), symbol(kind, waves, ns)))
    assert len(ins) > 500
    allowed = {"buffer_load_dwordx4", "buffer_load_dword", "buffer_load_dwordx2", "buffer_store_dwordx4",
               "global_load_dword"}
    copies = 0
    for op, rest in ins:
        assert not op.startswith("scratch_"), f"spill: {op}{rest}"
        if re.match(r"(buffer|global|flat)_", op):
            assert op in allowed, f"unexpected memory instruction {op}{rest}"
            if " lds" in rest:
                assert op == "buffer_load_dwordx4" and "offset:" not in rest, f"{op}{rest}"
                copies += 1
    assert copies > 0
    waits = set()
    for i, (op, rest) in enumerate(ins):
        if op == "s_waitcnt" and "vmcnt" in rest:
            nxt = next((o for o, _ in ins[i + 1:] if o != "s_nop"), "")
            if nxt == "s_barrier":
                waits.add(int(re.search(r"vmcnt\((\d+)\)", rest).group(1)))
    assert waits == design_waits(kind, ns), (sorted(waits), sorted(design_waits(kind, ns)))
