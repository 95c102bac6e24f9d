"""Build check (no GPU): every kernel compiled for gfx950 keeps its registers
in registers. A kernel that spills or indexes a private array dynamically gets
a private segment, which on this path costs far more than the work it holds.
The one allowance: a spill of at most 16 bytes whose scratch accesses all lie
outside every loop (executed once per wavefront, as in a set-up), which costs
nothing measurable."""

import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "long_context_attention_commvq_amd", "csrc")
SOURCES = ["decode_fast.hip", "decode.hip", "decode_merge.hip", "decode_bitv.hip", "encode.hip", "naive.hip", "em.hip"]


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES)
def test_kernels_have_no_private_segment(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
           "-o", str(out), os.path.join(CSRC, src)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    text = out.read_text()
    names = re.findall(r"^\s+\.name:\s+(\S+)", text, re.M)
    sizes = [int(v) for v in re.findall(r"^\s+\.private_segment_fixed_size:\s+(\d+)", text, re.M)]
    assert names and len(names) == len(sizes)
    bodies = _kernel_bodies(text)
    bad = [(n, v) for n, v in zip(names, sizes) if v and (v > 16 or _scratch_in_loop(bodies.get(n, [])))]
    assert not bad, bad


def _kernel_bodies(text):
    """Kernel name -> its instruction lines (from its label to its end marker)."""
    out, cur, lines = {}, None, []
    for line in text.splitlines():
        m = re.match(r"^(\S+):\s*(;.*)?$", line)
        if m and not m.group(1).startswith("."):
            cur, lines = m.group(1), []
            continue
        if cur is not None:
            if ".end_amdhsa_kernel" in line or line.strip().startswith(".Lfunc_end"):
                out[cur], cur = lines, None
            else:
                lines.append(line)
    return out


def _scratch_in_loop(lines):
    """True if a scratch access lies between a label and a later branch back to it."""
    labels = {}
    for i, line in enumerate(lines):
        m = re.match(r"^(\.\w+):", line)
        if m:
            labels[m.group(1)] = i
    spans = []
    for i, line in enumerate(lines):
        m = re.match(r"^\s+s_(?:cbranch_\w+|branch)\s+(\.\w+)", line)
        if m and m.group(1) in labels and labels[m.group(1)] <= i:
            spans.append((labels[m.group(1)], i))
    hits = [i for i, line in enumerate(lines) if re.match(r"^\s+(scratch_|buffer_\w+ .*off(?:en)?,.*s\[0:3\])", line)]
    return any(a <= i <= b for i in hits for a, b in spans)


def test_scratch_loop_detector_on_synthetic_listings():
    inside = [".LBB0_1:", "\tv_add_u32 v1, v1, v2", "\tscratch_load_dword v3, off, off", "\ts_cbranch_scc1 .LBB0_1"]
    outside = ["\tscratch_store_dword off, v3, off", ".LBB0_1:", "\tv_add_u32 v1, v1, v2", "\ts_cbranch_scc1 .LBB0_1",
               "\tscratch_load_dword v3, off, off"]
    forward = ["\ts_cbranch_execz .LBB0_2", "\tscratch_load_dword v3, off, off", ".LBB0_2:"]
    assert _scratch_in_loop(inside)
    assert not _scratch_in_loop(outside)
    assert not _scratch_in_loop(forward)
