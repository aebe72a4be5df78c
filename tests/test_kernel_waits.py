"""The hand-counted memory waits of the fused kernels, checked on the gfx950 assembly of this
repository's own sources (CPU only: hipcc cross-compiles without a GPU).

The forward and dX kernels copy the next step's X (dY) tile into LDS by DMA and then load the
codes of the step after it into registers; the step ends with a hand-written
`s_waitcnt vmcnt(N); s_barrier` that must retire the DMA group and nothing younger, so N must
equal the number of vector-memory operations issued after the step's last DMA (the code loads).
The M <= 16 stream kernel issues its copies as inline assembly; its stage loop must contain no
vector-memory operation but those copies and no wait the compiler inserted, and its hand waits
are the two counts the source derives from its copy constants. In every main loop, a wait the
compiler inserted must not retire an operation issued in the same step (that would stall on the
copies the pipeline keeps in flight).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "nf4_dequant_gemm_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
VMEM = re.compile(r"^(buffer|global|flat)_(load|store|atomic)")

pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not available")


def device_asm(src, tmp_path):
    out = os.path.join(tmp_path, os.path.basename(src) + ".s")
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--offload-device-only", "-S",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-x", "hip", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read().split("\n")


def kernels(lines):
    """{kernel symbol: its instruction lines}."""
    out, name, body = {}, None, []
    for ln in lines:
        m = re.match(r"^(_ZN\S+):", ln)
        if m:
            name, body = m.group(1), []
            continue
        if name and re.match(r"^\.Lfunc_end\d+:", ln):
            out[name] = body
            name = None
            continue
        if name:
            body.append(ln)
    return out


def loops(body):
    """Innermost loop bodies laid out from their header down to their backward branch, as lists
    of (kind, text, in_asm). (A loop whose latch block sits above its header, such as a short
    search loop, is left out: its body is not one straight run of lines.)"""
    res = []
    for i, ln in enumerate(body):
        if ln.startswith(".LBB") and "Inner Loop Header" in ln:
            lab = ln.split(":")[0]
            seq, inasm, closed = [], False, False
            for t in body[i + 1:]:
                t = t.strip()
                if "Loop Header" in t or t.startswith("s_endpgm"):
                    break
                if t == ";;#ASMSTART":
                    inasm = True
                    continue
                if t == ";;#ASMEND":
                    inasm = False
                    continue
                if (t.startswith("s_cbranch") or t.startswith("s_branch")) and t.endswith(lab):
                    closed = True
                    break
                if VMEM.match(t):
                    seq.append(("mem", t, inasm))
                elif re.match(r"s_waitcnt.*vmcnt\(\d+\)", t):
                    seq.append(("wait", t, inasm))
            if closed:
                res.append(seq)
    return res


def main_loops(body):
    """The loops holding a hand-written wait (the pipelined main loops)."""
    return [s for s in loops(body) if any(k == "wait" and a for k, _, a in s)]


def vmcnt(t):
    return int(re.search(r"vmcnt\((\d+)\)", t).group(1))


def check_step_pipeline(name, seq):
    """Per step (hand wait to hand wait): N of the hand wait == memory ops after the last DMA;
    no compiler wait retires an op of the same step."""
    steps, cur = [], []
    for item in seq:
        cur.append(item)
        if item[0] == "wait" and item[2]:
            steps.append(cur)
            cur = []
    assert steps, f"{name}: no hand wait in the main loop"
    for st in steps:
        issued = 0
        after_dma = None
        for kind, t, inasm in st:
            if kind == "mem":
                issued += 1
                if t.endswith(" lds"):
                    after_dma = 0
                elif after_dma is not None:
                    after_dma += 1
            elif not inasm:
                assert vmcnt(t) >= issued, f"{name}: compiler '{t}' retires ops of its own step"
            else:
                assert after_dma is not None, f"{name}: a step without its DMA group"
                assert vmcnt(t) == after_dma, (f"{name}: hand wait '{t}' but {after_dma} loads follow "
                                               f"the step's DMA group")


@pytest.mark.parametrize("src,prefix", [("fwd.hip", "fwd_"), ("dx.hip", "dx_")])
def test_gemm_step_waits(tmp_path, src, prefix):
    ks = {k: b for k, b in kernels(device_asm(src, str(tmp_path))).items() if prefix in k}
    assert len(ks) >= 6
    for name, body in ks.items():
        mls = main_loops(body)
        assert len(mls) == 1, f"{name}: {len(mls)} pipelined loops"
        check_step_pipeline(name, mls[0])


def test_stream_kernel_stage_waits(tmp_path):
    src = open(os.path.join(CSRC, "decode16.hip")).read()
    const = {k: int(v) for k, v in re.findall(r"constexpr int (kStageCopies|kWindowCopies) = (\d+);", src)}
    pending = 2 * const["kStageCopies"]
    allowed = {pending, pending + const["kWindowCopies"], 0}
    ks = kernels(device_asm("decode16.hip", str(tmp_path)))
    (name, body), = [(k, b) for k, b in ks.items() if "decode16" in k]
    mls = main_loops(body)
    assert len(mls) == 1
    seq = mls[0]
    waits = [t for k, t, a in seq if k == "wait"]
    assert waits and all(a for k, t, a in seq if k == "wait"), "compiler waits in the stage loop"
    assert {vmcnt(t) for t in waits} <= allowed, waits
    mem = [t for k, t, a in seq if k == "mem"]
    assert mem and all(t.endswith(" lds") and a for (k, t, a) in seq if k == "mem"), \
        "the stage loop must hold only the hand-issued copies"
