"""Structure of the generated gfx950 code: no workgroup barrier inside a divergent loop.

A loop whose exit the compiler takes as lane-dependent is run with an exec mask: lanes that leave
it wait, masked off, until every lane of the wave has left. A barrier inside such a loop is then
passed by a wave whose waiting lanes have not done their part of the iteration; when that part is
the work of one lane (claiming the next item, setting a flag), the rest of the workgroup runs on
with stale state and the launch never ends. The persistent LCB kernel hung this way once, with its
claim loop's exit read from LDS into a vector register. The test compiles every kernel source to
assembly and checks, from the compiler's own loop annotations, that no s_barrier sits in a loop
(or inside a loop nested in one) whose latch updates exec."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "request_candidate_broadcast_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")

LABEL = re.compile(r"^(\.LBB\d+_\d+):|^; %bb\.\d+:")
HEADER = re.compile(r"=>\s*This (?:Inner )?Loop Header: Depth=(\d+)")
IN_LOOP = re.compile(r"in Loop: Header=BB(\d+_\d+) Depth=(\d+)")
PARENT = re.compile(r"Parent Loop BB(\d+_\d+) Depth=(\d+)")


def kernels(asm: str):
    lines = asm.splitlines()
    i = 0
    while i < len(lines):
        m = re.match(r"^(_Z\S+):", lines[i])
        if m:
            j = i
            while j < len(lines) and not lines[j].startswith(".Lfunc_end"):
                j += 1
            yield m.group(1), lines[i:j]
            i = j
        i += 1


def barriers_in_divergent_loops(lines):
    """Lines of s_barrier whose enclosing loops include one with an exec-updating latch."""
    loop_of = [None] * len(lines)      # innermost loop header of each line's block
    parent = {}                        # loop header -> parent loop header
    cur = None
    for i, l in enumerate(lines):
        lab = LABEL.match(l)
        if lab:
            cur = None
            m = IN_LOOP.search(l)
            if m:
                cur = "BB" + m.group(1)
            if lab.group(1) and HEADER.search(l):
                cur = "BB" + lab.group(1)[4:]
        elif l.lstrip().startswith(";"):
            # comment lines right after a label carry the header / parent annotations
            m = HEADER.search(l)
            if m:
                j = i
                while j >= 0 and not LABEL.match(lines[j]):
                    j -= 1
                lab = LABEL.match(lines[j]).group(1)
                if lab:
                    cur = "BB" + lab[4:]
                    for k in range(j, i + 1):
                        loop_of[k] = cur
            m = PARENT.search(l)
            if m:
                j = i
                while j >= 0 and not LABEL.match(lines[j]):
                    j -= 1
                lab = LABEL.match(lines[j]).group(1)
                if lab:
                    hdr = "BB" + lab[4:]
                    d = int(m.group(2))
                    # the deepest parent listed is the direct one
                    if hdr not in parent or d > parent[hdr][1]:
                        parent[hdr] = ("BB" + m.group(1), d)
        loop_of[i] = cur
    divergent = {loop_of[i] for i, l in enumerate(lines) if loop_of[i] and re.search(r"s_andn2_b64 exec, exec,", l)}

    def chain(h):
        while h:
            yield h
            h = parent.get(h, (None, 0))[0]

    return [(i + 1, loop_of[i]) for i, l in enumerate(lines)
            if "s_barrier" in l and loop_of[i] and any(h in divergent for h in chain(loop_of[i]))]


def test_checker_flags_a_barrier_in_a_divergent_loop():
    """The checker itself, on a hand-made fragment with the shape of the hang."""
    frag = """_Zk:
.LBB0_1:                                ; =>This Loop Header: Depth=1
	s_waitcnt lgkmcnt(0)
	s_barrier
	ds_read_b64 v[2:3], v1
; %bb.2:                                ;   in Loop: Header=BB0_1 Depth=1
	s_andn2_b64 exec, exec, s[30:31]
	s_cbranch_execnz .LBB0_1
.LBB0_3:
	s_endpgm
.Lfunc_end0:"""
    (_, lines), = list(kernels(frag))
    assert [b[1] for b in barriers_in_divergent_loops(lines)] == ["BB0_1"]
    ok = frag.replace("s_andn2_b64 exec, exec, s[30:31]\n\ts_cbranch_execnz", "s_cmp_lg_u32 s3, 0\n\ts_cbranch_scc1")
    (_, lines), = list(kernels(ok))
    assert barriers_in_divergent_loops(lines) == []


def test_no_barrier_in_a_divergent_loop():
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    tmp = tempfile.mkdtemp(prefix="ikbo_asm_")
    try:
        procs = []
        for f in srcs:
            out = os.path.join(tmp, f + ".s")
            cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-I" + os.path.join(ROOT, "include"),
                   "-I" + CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "--cuda-device-only",
                   "-S", os.path.join(CSRC, f), "-o", out]
            procs.append((f, out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        bad, seen = [], 0
        for f, out, p in procs:
            log = p.communicate(timeout=600)[0].decode(errors="replace")
            assert p.returncode == 0, "hipcc -S failed for %s:\n%s" % (f, log[-2000:])
            for name, lines in kernels(open(out).read()):
                seen += 1
                hits = barriers_in_divergent_loops(lines)
                if hits:
                    bad.append("%s %s: %s" % (f, name, hits[:4]))
        assert seen >= 10, "expected every kernel in the assembly, found %d" % seen
        assert not bad, "s_barrier inside a divergent loop:\n" + "\n".join(bad)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
