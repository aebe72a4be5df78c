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
    """Innermost loops, each as the list of (kind, text, in_asm) of one iteration in execution
    order. Blocks carry the compiler's loop annotation ('Inner Loop Header' on the header, 'in
    Loop: Header=...' on the other blocks of the innermost loop holding them); an iteration runs
    from the header down through the loop's blocks below it, then through those laid out above it
    (a latch block placed above the header falls through into it)."""
    blocks = []                       # (first line, innermost loop header name or None, is header)
    for i, ln in enumerate(body):
        m = re.match(r"^(\.LBB\d+_\d+:|; %bb\.\d+:)", ln)
        if not m:
            continue
        if "Inner Loop Header" in ln:
            blocks.append((i, ln.split(":")[0][len(".L"):], True))
        else:
            h = re.search(r"in Loop: Header=(\S+)", ln)
            blocks.append((i, h.group(1) if h else None, False))
    ends = [b[0] for b in blocks[1:]] + [len(body)]
    res = []
    for hb, (start, name, is_hdr) in enumerate(blocks):
        if not is_hdr:
            continue
        members = [k for k, b in enumerate(blocks) if b[1] == name]
        order = [k for k in members if k >= hb] + [k for k in members if k < hb]
        seq, inasm = [], False
        for k in order:
            for t in body[blocks[k][0]:ends[k]]:
                t = t.strip()
                if t == ";;#ASMSTART":
                    inasm = True
                elif t == ";;#ASMEND":
                    inasm = False
                elif VMEM.match(t):
                    seq.append(("mem", t, inasm))
                elif re.match(r"s_waitcnt.*vmcnt\(\d+\)", t):
                    seq.append(("wait", t, inasm))
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


@pytest.mark.parametrize("src,pattern", [("fwd.hip", r"fwd_(fused|grouped|pair)_kernel"),
                                         ("dx.hip", r"dx_(fused|grouped)_kernel")])
def test_gemm_step_waits(tmp_path, src, pattern):
    """The pipelined GEMM kernels (not the small tail kernel beside the grouped dX)."""
    ks = {k: b for k, b in kernels(device_asm(src, str(tmp_path))).items() if re.search(pattern, k)}
    assert len(ks) >= 6
    for name, body in ks.items():
        mls = main_loops(body)
        assert len(mls) == 1, f"{name}: {len(mls)} pipelined loops"
        check_step_pipeline(name, mls[0])


def test_stream_kernel_stage_waits(tmp_path):
    """The M <= 16 stream kernel (NF4 and E2M1 with T given; T formed in the kernel, NF4 from 1, 2
    or 4 rank tiles, E2M1 from 1): the copying waves' stage loop holds the hand-issued copies and
    the hand waits only (E2M1 forming T: two more copies per stage, A's slice); the other waves'
    stage loop issues no copy, and with NF4 forming T it holds A's loads, which the compiler
    tracks and waits for itself."""
    src = open(os.path.join(CSRC, "decode16.hip")).read()
    const = {k: int(v) for k, v in re.findall(r"constexpr int (kStageCopies|kWindowCopies|kACopies) = (\d+);", src)}
    ks = {k: b for k, b in kernels(device_asm("decode16.hip", str(tmp_path))).items() if "decode16" in k}
    # NF4 (Lb0) and E2M1 (Lb1) with T given (Li0); NF4 with 1, 2 or 4 rank tiles of T formed,
    # E2M1 with 1
    assert sorted(re.search(r"ILb([01])ELi(\d)E", k).groups() for k in ks) == \
        [("0", "0"), ("0", "1"), ("0", "2"), ("0", "4"), ("1", "0"), ("1", "1")], sorted(ks)
    for name, body in ks.items():
        fp4 = "ILb1E" in name
        kq = int(re.search(r"ILb[01]ELi(\d)E", name).group(1))
        pending = 2 * (const["kStageCopies"] + (const["kACopies"] if fp4 and kq else 0))
        # the E2M1 form copies no windows of block codes: only the stage count
        allowed = {pending, 0} if fp4 else {pending, pending + const["kWindowCopies"], 0}
        ls = loops(body)
        copying = [seq for seq in ls if any(k == "mem" and t.endswith(" lds") for k, t, a in seq)]
        assert len(copying) == 1, (name, len(copying))
        seq = copying[0]
        waits = [t for k, t, a in seq if k == "wait"]
        assert waits and all(a for k, t, a in seq if k == "wait"), f"{name}: compiler waits in the copying loop"
        assert {vmcnt(t) for t in waits} <= allowed, (name, waits)
        assert all(t.endswith(" lds") and a for (k, t, a) in seq if k == "mem"), \
            f"{name}: the copying loop must hold only the hand-issued copies"
        others = [q for q in ls if q is not seq]
        assert not any(a for q in others for k, t, a in q if k == "mem"), f"{name}: hand-issued loads elsewhere"
        if kq and not fp4:
            tl = [q for q in others if any(k == "mem" and t.startswith("buffer_load_dwordx4") for k, t, a in q)]
            assert tl, f"{name}: no stage loop loading A"
