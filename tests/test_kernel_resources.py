"""Every gfx950 kernel of the library compiles without register spills and
without private (scratch) memory.  A register array the compiler cannot index
statically, or a spill, silently moves data to scratch and costs a large
share of a kernel's time; this keeps such a regression from passing unseen.
Runs on the CPU (hipcc cross-compiles to assembly)."""
import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from sparse_attention_fp4_fp4idx_amd import build


def _assemble(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    cmd = [build.HIPCC, *build.FLAGS, "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(f"hipcc failed for {src}:\n{r.stderr[-2000:]}")
    return open(out).read()


def _kernels(asm: str):
    for m in re.finditer(r"^\s+- \.agpr_count:.*?(?=^\s+- \.agpr_count:|\Z)", asm, re.S | re.M):
        block = m.group(0)
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name:
            continue
        field = lambda key: int(re.search(r"\." + key + r":\s+(\d+)", block).group(1))  # noqa: E731
        yield (name.group(1), field("private_segment_fixed_size"), field("vgpr_spill_count"),
               field("sgpr_spill_count"))


def test_no_kernel_spills_or_uses_scratch():
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    srcs = build.sources()
    with tempfile.TemporaryDirectory() as d, ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        asms = list(ex.map(lambda s: _assemble(s, d), srcs))
    seen, bad = 0, []
    for src, asm in zip(srcs, asms):
        for name, scratch, vspill, sspill in _kernels(asm):
            seen += 1
            if scratch or vspill or sspill:
                bad.append(f"{os.path.basename(src)}: {name} scratch={scratch} vgpr_spill={vspill} "
                           f"sgpr_spill={sspill}")
    assert seen >= 40, f"only {seen} kernels found in the assembly"
    assert not bad, "\n".join(bad)


def _vgprs(asm: str):
    for m in re.finditer(r"^\s+- \.agpr_count:.*?(?=^\s+- \.agpr_count:|\Z)", asm, re.S | re.M):
        block = m.group(0)
        name = re.search(r"\.name:\s+(\S+)", block)
        if name:
            agpr = int(re.search(r"\.agpr_count:\s+(\d+)", block).group(1))
            vgpr = int(re.search(r"\.vgpr_count:\s+(\d+)", block).group(1))
            yield name.group(1), vgpr + agpr


def test_register_budgets_the_launch_shapes_rely_on():
    """Launch shapes chosen for occupancy: a 512-thread top-k row (eight
    waves) shares a CU with a second row only at <= 128 registers per lane
    (four waves per SIMD), and the shared-page logits kernel's 4 x 2 shape was
    picked for four waves per SIMD as well (and its scheduled form, which
    runs the same body on the plan's items), as was the FP8 shared-page
    kernel's 4 x 1 shape."""
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    srcs = [s for s in build.sources() if os.path.basename(s) in ("topk.hip", "logits.hip")]
    with tempfile.TemporaryDirectory() as d:
        regs = dict(kv for s in srcs for kv in _vgprs(_assemble(s, d)))
    want = {n: r for n, r in regs.items()
            if "topk_reg_kernelILi512E" in n or "mqa_logits_shared_kernelINS_9Fp4StagedELi4ELi2ELi4E" in n
            or "mqa_logits_planned_kernelILi4ELi2ELi4E" in n or "mqa_logits_shared_kernelINS_9Fp8StagedELi4ELi1ELi4E" in n}
    assert len(want) >= 8, sorted(regs)
    over = {n: r for n, r in want.items() if r > 128}
    assert not over, over
