"""The compiled step schedule of every kernel instance, and spill-free key
loops in every attention kernel (CPU only).

Each 32-key step of attn_fwd_kernel is meant to
interleave its 16 MFMAs with the softmax VALU work and the LDS operand reads
(sched_group_barrier in the source).  Small, equivalent source changes have
made the compiler fall back to source order instead: the whole softmax
first, then each MFMA behind its own LDS read, about 11% slower on MI355X.
This test compiles the kernel to gfx950 assembly with the same flags as the
build and checks, for every instance (head dim, mask, one pass or key
ranges) and every loop whose body holds a full step, that the first MFMA is
issued within a handful of instructions of the loop head.
"""

import os
import re
import subprocess

import pytest

from exact_io_aware_27_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL = os.path.join(ROOT, "exact_io_aware_27_amd", "csrc", "attn_fwd_kernel.hip")
INSTANCES = ["_ZN11attn_gfx95015attn_fwd_kernelILi%dELb%dELb%dELi%dEEEvNS_5KArgsE" % (d, c, s, w)
             for d in (128, 64) for c in (1, 0) for s in (0, 1) for w in ((8, 4) if d == 128 and s else
                                                                            (8,) if d == 128 else (4,))]
SKIP = re.compile(r"^\s*(;|$)")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    hipcc = build.HIPCC
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "kernel.s")
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC") and not f.startswith("-Wl,")]
    subprocess.check_call([hipcc] + flags + ["--cuda-device-only", "-S", "-o", out, KERNEL])
    with open(out) as f:
        return f.read().splitlines()


def _instance(lines, name):
    start = next(i for i, l in enumerate(lines) if l.startswith(name + ":"))
    end = next(i for i in range(start, len(lines)) if "s_endpgm" in lines[i])
    return lines[start:end + 1]


@pytest.mark.parametrize("instance", INSTANCES)
def test_steps_interleave_mfma_with_softmax(asm, instance):
    body = _instance(asm, instance)
    heads = [i for i, l in enumerate(body) if "Loop Header: Depth=" in l]
    checked = 0
    for h in heads:
        instrs = []
        for l in body[h:h + 600]:
            if "s_barrier" in l:
                break
            if SKIP.match(l) or l.lstrip().startswith(".") or "ASMSTART" in l or "ASMEND" in l:
                continue
            instrs.append(l.split()[0])
        if sum(1 for x in instrs if x.startswith("v_mfma")) < 8:
            continue  # not a compute step (the copy-only loop of idle waves)
        # scalar work and the compares of a wave-uniform branch between step
        # variants do not count: the failure looked for is softmax VALU work
        # (tens of instructions) issued ahead of the step's first MFMA
        work = [x for x in instrs if not (x.startswith("s_") or x.startswith("v_cmp"))]
        first = next(i for i, x in enumerate(work) if x.startswith("v_mfma"))
        assert first <= 12, "step at loop head %d issues %d instructions before its first MFMA: %s" % (
            h, first, " ".join(work[:first + 1]))
        checked += 1
    assert checked >= 2, "expected the unmasked and the masked step loops"


def key_loop_spills(body):
    """(key loops, scratch accesses inside them) of one kernel's assembly.
    Every basic block's label carries the compiler's loop annotation (the
    loop header it belongs to); the key loops are the innermost loops that
    issue MFMAs."""
    loop_of = []  # per line: header label of the innermost loop holding the line, or None
    parent = {}   # loop header -> enclosing loop header
    cur = None
    for i, l in enumerate(body):
        m = re.match(r"^(?:\.L(BB\w+)|; %bb\.(\d+)):", l)  # a labelled or a fall-through block
        if m:
            note = l + (body[i + 1] if i + 1 < len(body) else "")
            if "Loop Header" in note and m.group(1):
                cur = m.group(1)
                up = re.findall(r"Parent Loop (BB\w+)", note)
                parent.setdefault(cur, up[-1] if up else None)
            else:
                inner = re.search(r"in Loop: Header=(BB\w+)", l)
                cur = inner.group(1) if inner else None
        loop_of.append(cur)
    has_child = {p for p in parent.values() if p}
    mfma = {}
    for l, lp in zip(body, loop_of):
        if lp and "v_mfma" in l:
            mfma[lp] = mfma.get(lp, 0) + 1
    key_loops = {lp for lp, n in mfma.items() if n >= 4 and lp not in has_child}
    spills = [(lp, l.strip()) for l, lp in zip(body, loop_of) if lp in key_loops and "scratch_" in l]
    return key_loops, spills


@pytest.mark.parametrize("instance", INSTANCES)
def test_no_scratch_in_key_loops(asm, instance):
    """No spill or reload runs inside a key loop of the forward kernel."""
    key_loops, spills = key_loop_spills(_instance(asm, instance))
    assert len(key_loops) >= 2, "expected the unmasked and the masked key loops, found %s" % sorted(key_loops)
    assert not spills, "scratch access inside a key loop: %s" % spills[:3]


OTHER_SOURCES = {"bwd": "attn_bwd_kernel.hip", "fp8": "attn_fp8_kernel.hip"}


@pytest.fixture(scope="module")
def other_asm(tmp_path_factory):
    hipcc = build.HIPCC
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC") and not f.startswith("-Wl,")]
    out = {}
    for key, name in OTHER_SOURCES.items():
        path = str(tmp_path_factory.mktemp("asm_" + key) / "kernel.s")
        subprocess.check_call([hipcc] + flags + ["--cuda-device-only", "-S", "-o", path,
                                                 os.path.join(ROOT, "exact_io_aware_27_amd", "csrc", name)])
        with open(path) as f:
            out[key] = f.read().splitlines()
    return out


@pytest.mark.parametrize("key", sorted(OTHER_SOURCES))
def test_no_scratch_in_backward_and_fp8_key_loops(other_asm, key):
    """The backward kernels and the FP8 attention kernel: every instance has
    a key loop and none of its key loops touches scratch."""
    lines = other_asm[key]
    names = [l.split(":")[0] for l in lines if re.match(r"^_ZN\w+:", l)]
    names = [n for n in names if "quantize" not in n]  # no key loop
    assert len(names) == (8 if key == "bwd" else 2), names
    for name in names:
        key_loops, spills = key_loop_spills(_instance(lines, name))
        assert key_loops, "%s: no key loop found" % name
        assert not spills, "%s: scratch access inside a key loop: %s" % (name, spills[:3])


def mfma_inside_output_branch(body):
    """MFMAs between the last lane-masking s_and_saveexec before the first
    store of the output and that store: the body of the branch that only
    the lanes of valid queries run."""
    store = next(i for i, l in enumerate(body) if l.strip().startswith(("global_store", "buffer_store")))
    masks = [i for i in range(store) if body[i].strip().startswith(("s_and_saveexec", "s_and_b64 exec, exec"))]
    if not masks:
        return []
    return [body[i].strip() for i in range(masks[-1], store) if body[i].strip().startswith("v_mfma")]


@pytest.mark.parametrize("instance", INSTANCES)
def test_output_mfmas_run_with_every_lane(asm, instance):
    """The last P V MFMAs feed only the stores of valid query rows; the
    compiler may sink them into that lane-masked branch, where an MFMA does
    not compute the rows of the live lanes (seen as wrong rows in a tile
    whose last wave holds a few valid queries).  The kernel pins O after
    them; this checks the compiled result."""
    bad = mfma_inside_output_branch(_instance(asm, instance))
    assert not bad, "MFMA inside the output branch: %s" % bad[:2]


def test_fp8_output_mfmas_run_with_every_lane(other_asm):
    lines = other_asm["fp8"]
    names = [l.split(":")[0] for l in lines if re.match(r"^_ZN\w+:", l) and "quantize" not in l]
    assert len(names) == 2, names
    for name in names:
        bad = mfma_inside_output_branch(_instance(lines, name))
        assert not bad, "%s: MFMA inside the output branch: %s" % (name, bad[:2])
