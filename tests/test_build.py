"""Build properties of the gfx950 kernels, checked on the CPU: no kernel keeps
registers in scratch memory (a spill turns register arrays into memory
traffic and cost 10-20% wherever it appeared)."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_attention_06_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["compress.hip", "indexer.hip", "topk.hip", "attn.hip"]
# Deliberate spills, each with the most scratch it may use and why it is kept.
ALLOWED = {
    # four workgroups per CU need at most 128 registers; about 15 dwords of
    # the select's tail go to scratch, and the prefill top-k still runs 7%
    # faster than the spill-free form at three workgroups per CU
    "_ZN3csa15topk_row_kernelILi64EEEvNS_8TopkArgsE": 96,
}


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES)
def test_no_scratch(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"), "--cuda-device-only", "-S", "-o", str(out),
           os.path.join(CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    kernels = re.findall(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", asm, flags=re.S)
    assert kernels, "no kernel found"
    spilled = [k for k, body in kernels
               if int(re.search(r"private_segment_fixed_size (\d+)", body).group(1)) > ALLOWED.get(k, 0)]
    assert not spilled, f"kernels using scratch: {spilled}"
