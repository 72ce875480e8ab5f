"""Code-generation checks of the gfx950 kernels (CPU only: hipcc
cross-compiles).  Private arrays that land in scratch memory (dynamically
indexed accumulators, staging registers) made the GEMM phases several times
slower before; this keeps them out."""

import os
import re
import shutil
import subprocess
import tempfile

import pytest

from matrix_aware_optimizer_muon_amd import build as B

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
@pytest.mark.parametrize("src", [s for s in B.SOURCES if s.endswith(".hip")])
def test_no_scratch_memory_in_kernels(src):
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "k.s")
        cmd = [HIPCC, f"--offload-arch={B.ARCH}", "-O3", "-std=c++17", "-x", "hip",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "--cuda-device-only", "-S", f"-I{B.INCLUDE}", os.path.join(B.CSRC, src), "-o", out]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        assert r.returncode == 0, r.stdout
        asm = open(out).read()
    kernels = re.split(r"\n(?=_Z\S+:)", asm)
    offenders = []
    for k in kernels:
        name = k.split(":", 1)[0]
        if re.search(r"\bscratch_(load|store)", k):
            offenders.append(name)
    assert not offenders, f"kernels using scratch memory: {offenders}"
    # the private segment size the code objects declare is zero as well
    sizes = [int(x) for x in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", asm)]
    assert all(s == 0 for s in sizes), sizes
