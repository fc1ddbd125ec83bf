"""Static check of the built kernels (CPU only): no workgroup barrier can be reached while an LDS
write of the same wave may still be outstanding.

A barrier hands LDS data from the waves that wrote it to the waves that read it after the
barrier; the write must have completed (s_waitcnt lgkmcnt(0)) before the writer arrives.  The
compiler emits that wait on straight-line paths but not always on a loop's back edge, so every
kernel's gfx950 assembly is compiled here and each path to each s_barrier is followed.
"""
import os
import re
import subprocess

import pytest

from mla_latent_cache_absorb_amd import build

CSRC = build.CSRC


def kernels_assembly(src: str, tmp_path) -> str:
    out = os.path.join(str(tmp_path), os.path.basename(src) + ".s")
    cmd = [build.hipcc(), "-O3", "-std=c++17", f"--offload-arch={build.ARCH}", *build.DEVICE_FLAGS,
           "-I", os.path.join(build.ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S", src, "-o", out]
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    return open(out).read()


def unwaited_barriers(asm: str):
    """(kernel, line) of every s_barrier some path reaches with an LDS write not yet waited for."""
    lines = asm.split("\n")
    found = []
    # functions only (a file may also define device variables, whose labels look alike)
    funcs = set(re.findall(r"\.type\s+(\S+),\s*@function", asm))
    starts = [i for i, l in enumerate(lines)
              if re.match(r"^_Z\S+:\s*(;.*)?$", l) and l.split(":")[0] in funcs]
    for st in starts:
        name = lines[st].split(":")[0]
        en = next(i for i in range(st, len(lines)) if lines[i].strip().startswith(".Lfunc_end"))
        body = [l.strip() for l in lines[st:en]]
        labels = {l.split(":")[0]: i for i, l in enumerate(body) if re.match(r"^\.LBB\S+:", l)}
        seen, work = set(), [(1, False)]
        while work:
            i, pending = work.pop()
            while i < len(body):
                if (i, pending) in seen:
                    break
                seen.add((i, pending))
                t = body[i]
                if t.startswith("s_barrier") and pending:
                    found.append((name, i))
                if re.match(r"ds_(write|add|sub|min|max|and|or|xor|inc|dec)", t):
                    pending = True
                if t.startswith("s_waitcnt") and "lgkmcnt(0)" in t:
                    pending = False
                m = re.match(r"s_(cbranch_\w+|branch)\s+(\.LBB\S+)", t)
                if m:
                    work.append((labels[m.group(2)], pending))
                    if m.group(1) == "branch":
                        break
                if t.startswith("s_endpgm"):
                    break
                i += 1
    return found


def test_checker_flags_a_missing_wait():
    # a loop whose back edge carries an LDS write to the barrier, and the same with the wait
    bad = "\n".join(["\t.type _Zk,@function", "_Zk:", "  s_nop 0", ".LBB0_1:", "  s_barrier", "  ds_write_b32 v0, v1",
                     "  s_cbranch_scc1 .LBB0_1", "  s_endpgm", ".Lfunc_end0:"])
    good = bad.replace("  s_cbranch_scc1", "  s_waitcnt lgkmcnt(0)\n  s_cbranch_scc1")
    assert unwaited_barriers(bad) == [("_Zk", 3)]
    # a device variable's label is not a kernel
    assert unwaited_barriers(bad + "\n_ZN12_GLOBAL__N_17scratchE:\n\t.zero 256") == [("_Zk", 3)]
    assert unwaited_barriers(good) == []


@pytest.mark.parametrize("src", sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")))
def test_no_barrier_with_an_lds_write_in_flight(src, tmp_path):
    asm = kernels_assembly(os.path.join(CSRC, src), tmp_path)
    assert unwaited_barriers(asm) == []
