"""Build check (no GPU): every kernel compiled for gfx950 keeps its registers
in registers. A kernel that spills or indexes a private array dynamically gets
a private segment, which on this path costs far more than the work it holds."""

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
    bad = [(n, v) for n, v in zip(names, sizes) if v]
    assert not bad, bad
