"""The expert GEMMs' load pipelines count their own loads: each k-step waits
with `s_waitcnt vmcnt(N)` until at most N vector-memory operations of the
wave are outstanding, N being the loads of the stages that may stay in flight
(stages x loads per stage, all issued in program order and retired in order).
If the compiler issues fewer loads per stage than the source counts (it drops
a load whose result no path reads), N lets the stage that is about to be read
still be in flight, and the k-step reads LDS the direct loads have not filled.

This compiles the weight-streaming GEMM for gfx950 with the library's flags
(the source whose loops know at compile time that a row group is empty) and
checks the unrolled k-steps in the assembly: a wait N that heads three or more
k-steps issuing L > 0 loads each must be a whole number of stages, N = m * L,
with the same m (the stages left in flight) for every loop of the kernel.
(Stages that the compiler had cut from 7 loads to 6 under a wait of 7 x 7 =
49, and from 9 to 7 under 7 x 9 = 63 — 9 stages "in flight" of 8 — are what
this guards against.)  Kernels whose unrolled loop
repeats no k-step shape three times (the two-stage bf16 and fp32 rings, whose
row-group test is a runtime branch) are outside this check.  The tiled GEMM
has no optional loads and its compile takes minutes: not checked here."""
import collections
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_align_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")) is None,
                                reason="hipcc not available")


def _device_asm(src, out):
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "moe_build", os.path.join(ROOT, "mixture_experts_layer_align_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    flags = [f for f in b.FLAGS if f != "-fPIC"]
    cmd = [b.HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


def step_waits(asm, kernel_re):
    """{kernel: Counter((N, loads in the region up to the next such wait))}
    for the explicit nonzero vmcnt waits of each matching kernel."""
    res = {}
    for m in re.finditer(r"^(" + kernel_re + r"):", asm, re.M):
        name = m.group(1)
        body = asm[m.end():asm.find(".Lfunc_end", m.end())].split("\n")
        heads = [i for i, l in enumerate(body) if re.search(r"s_waitcnt vmcnt\((\d+)\)", l)]
        c = collections.Counter()
        for a, b in zip(heads, heads[1:] + [len(body)]):
            n = int(re.search(r"vmcnt\((\d+)\)", body[a]).group(1))
            loads = sum(1 for l in body[a:b] if re.search(r"\b(global_load|buffer_load)", l))
            c[(n, loads)] += 1
        res[name] = c
    return res


def violations(waits):
    bad = []
    for name, c in waits.items():
        steps = [(n, loads, k) for (n, loads), k in c.items() if n > 2 and loads > 0 and k >= 3]
        ratios = {n // loads for n, loads, _ in steps if n % loads == 0}
        for n, loads, k in steps:
            if n % loads != 0 or len(ratios) > 1:
                bad.append((name, n, loads, k))
    return sorted(bad)


def test_checker_flags_a_dropped_load():
    # a k-loop unrolled over 8 stages whose source counts 7 loads a stage but
    # whose compiled stages issue 6: the wait of 49 does not cover the stage
    step = ["s_waitcnt vmcnt(49)"] + ["global_load_lds_dwordx4 v[0:1], off"] * 4 + \
           ["global_load_dwordx4 v[2:5], v[0:1], off"] * 2 + ["v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]"]
    asm = "_Zkernel:\n" + "\n".join(step * 8) + "\n.Lfunc_end0:\n"
    assert violations(step_waits(asm, r"_Zkernel")) == [("_Zkernel", 49, 6, 8)]
    # ... and two loops of one kernel, 7 x 9 = 63 over 9 loads (7 stages in
    # flight) and over 7 loads (9 "in flight")
    nine = [l.replace("vmcnt(49)", "vmcnt(63)") for l in step[:1]] + \
           ["global_load_lds_dwordx4 v[0:1], off"] * 5 + ["global_load_dwordx4 v[2:5], v[0:1], off"] * 4
    seven = nine[:1] + nine[1:6] + nine[6:8]
    asm = "_Zkernel:\n" + "\n".join(nine * 8 + seven * 8) + "\n.Lfunc_end0:\n"
    assert violations(step_waits(asm, r"_Zkernel")) == [("_Zkernel", 63, 7, 8), ("_Zkernel", 63, 9, 8)]
    good = [l.replace("vmcnt(49)", "vmcnt(42)") for l in step]
    asm = "_Zkernel:\n" + "\n".join(good * 8) + "\n.Lfunc_end0:\n"
    assert violations(step_waits(asm, r"_Zkernel")) == []


def test_every_k_step_wait_is_whole_stages(tmp_path):
    waits = step_waits(_device_asm("expert_gemm_stream.hip", str(tmp_path / "stream.s")),
                       r"_Z\S*k_expert_stream\S*")
    # the 8-bit and 4-bit weight kernels (their rings run four or eight stages)
    # all show their steady-state k-steps
    deep = [n for n in waits if re.search(r"ILi1ELi[234]E", n)]
    assert len(deep) >= 10, sorted(waits)
    assert all(any(n > 2 and l > 0 and k >= 3 for (n, l), k in waits[d].items()) for d in deep)
    assert violations(waits) == []
