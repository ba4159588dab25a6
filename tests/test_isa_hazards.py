"""Machine-code check of the attention kernels (CPU only; needs hipcc).

The compiler inserts the wait states a matrix-core (MFMA) result needs
before a vector instruction reads it only in front of instructions it
emits itself, not in front of inline assembly.  The hardware does not
interlock such a read, so inline assembly that reads a product's result
before any compiled instruction has read it may see a partly written
register; for the row maximum this made repeated forward calls differ in
the last bit.  This test compiles the kernels for gfx950 and checks, per
basic block, that no inline-assembly instruction reads (or overwrites) a
register that an MFMA wrote (or reads as its accumulator) before a
compiled vector instruction has read that MFMA's result.  The scan is per
basic block (state is dropped at every label), so it would miss a product
issued at the end of one block and read by inline assembly at the start of
the block that follows it."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_masked_build_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def _regs(tok):
    out = set()
    for r in re.findall(r"v\[(\d+):(\d+)\]|v(\d+)", tok):
        out.update([int(r[2])] if r[2] else range(int(r[0]), int(r[1]) + 1))
    return out


def _scan(body):
    """Inline-assembly lines that touch an MFMA result (or accumulator)
    before a compiled vector instruction has read that MFMA's result.  The scan is per
basic block (state is dropped at every label), so it would miss a product
issued at the end of one block and read by inline assembly at the start of
the block that follows it."""
    pending, groups, srcc, gid, in_asm, bad = {}, {}, {}, 0, False, []
    for raw in body.split("\n"):
        if ";;#ASMSTART" in raw:
            in_asm = True
            continue
        if ";;#ASMEND" in raw:
            in_asm = False
            continue
        line = raw.split(";")[0].strip()
        if line.endswith(":"):  # a block label: the scan is per basic block
            pending, srcc = {}, {}
            continue
        if not line or line.startswith("."):
            continue
        op = line.split()[0]
        args = line[len(op):].split(",")
        dst = _regs(args[0]) if op.startswith("v_") else set()
        srcs = set().union(*[_regs(x) for x in args[1:]]) if len(args) > 1 else set()
        if in_asm:
            if any(r in pending for r in srcs) or any(r in pending or r in srcc for r in dst):
                bad.append(line)
        elif op.startswith("v_") and not op.startswith("v_mfma"):
            for g in {pending[r] for r in srcs if r in pending}:
                for r in groups[g]:
                    pending.pop(r, None)
            srcc = {}
        if op.startswith("v_mfma"):
            gid += 1
            groups[gid] = _regs(args[0])
            for r in groups[gid]:
                pending[r] = gid
            for r in (_regs(args[3]) if len(args) > 3 else set()):
                srcc[r] = gid
        elif op.startswith("v_"):
            for r in dst:
                pending.pop(r, None)
    return bad


_ASM = {}


def _objects():
    from block_sparse_masked_build_amd import build
    return build


BUILD = _objects()
# the objects the build compiles: (source, object name, flags)
ATTN_OBJECTS = [e[1] for e in BUILD.SOURCES if e[0] in ("attn_fwd.hip", "attn_bwd.hip")]
ALL_OBJECTS = [e[1] for e in BUILD.SOURCES if e[0].endswith(".hip")]


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    """Device assembly of each object the build compiles, with its own
    flags: the build's saved copy when its stamp matches the current
    sources, else compiled here (all missing ones concurrently)."""
    if not _ASM:
        tmp = tmp_path_factory.mktemp("isa")
        procs = {}
        for src, obj, extra in BUILD.SOURCES:
            if not src.endswith(".hip"):
                continue
            d = BUILD.object_dir(obj)
            saved = os.path.join(d, os.path.splitext(src)[0] + "-hip-amdgcn-amd-amdhsa-gfx950.s")
            stamp = os.path.join(d, "stamp.txt")
            if os.path.exists(saved) and os.path.exists(stamp) and open(stamp).read() == BUILD.source_stamp(extra):
                _ASM[obj] = open(saved).read()
                continue
            out = tmp / (obj + ".s")
            cmd = [HIPCC, *BUILD.compile_flags(), *extra, "-x", "hip", "--cuda-device-only", "-S",
                   os.path.join(CSRC, src), "-o", str(out)]
            procs[obj] = (subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE), out)
        for obj, (proc, out) in procs.items():
            _, err = proc.communicate()
            assert proc.returncode == 0, (obj, err.decode()[-2000:])
            _ASM[obj] = out.read_text()
    return lambda key: _ASM[key]


@pytest.mark.parametrize("src", ATTN_OBJECTS)
def test_no_inline_assembly_reads_of_pending_matrix_results(src, asm):
    text = asm(src)
    kernels = re.findall(r"^(_Z\S*kernel\S*):", text, re.M)
    assert kernels
    problems = {}
    for k in kernels:
        a = text.index(k + ":")
        body = text[a:text.index(".Lfunc_end", a)]
        bad = _scan(body)
        if bad:
            problems[k] = bad[:3]
    assert not problems, problems



@pytest.mark.parametrize("src", ALL_OBJECTS)
def test_m0_is_only_written_by_the_lds_copies(src, asm):
    """The asynchronous LDS copies set M0 (the LDS destination) in inline
    assembly and list it as clobbered, but M0 is a register the compiler
    reserves, and it does not promise to preserve a value of its own in M0
    across such a block.  So the compiled code must not use M0 at all: no
    instruction outside inline assembly may read or write it, and there is
    no dynamic VGPR indexing (which keeps its index in M0) and no call."""
    text = asm(src)
    bad, in_asm = [], False
    for raw in text.split("\n"):
        if ";;#ASMSTART" in raw:
            in_asm = True
            continue
        if ";;#ASMEND" in raw:
            in_asm = False
            continue
        line = raw.split(";")[0].strip()
        if not line or line.startswith(".") or line.endswith(":"):
            continue
        op = line.split()[0]
        if in_asm:
            continue
        if re.search(r"\bm0\b", line) or "gpr_idx" in op or "movrel" in op or op == "s_swappc_b64":
            bad.append(line)
    assert not bad, bad[:5]
