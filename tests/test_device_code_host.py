"""Host-side checks of the generated gfx950 code (no GPU needed).

The prefill kernels issue their loads straight into LDS from inline
assembly that writes M0 without restoring it (M0 is a reserved register
the compiler does not preserve around an asm statement).  That is sound
only while no code the compiler generates for those kernels uses M0 on its
own; this compiles the source to assembly with the library's flags and
checks it, so that a compiler or source change that starts using M0 is
caught on the host.
"""
import os
import re
import shutil
import subprocess

import pytest

from paged_kv_cache_467_amd import build as B

SOURCE = os.path.join(B.CSRC, "paged_attention_prefill.hip")
ASM_BEGIN, ASM_END = ";;#ASMSTART", ";;#ASMEND"


def device_assembly(tmp_path, source):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not shutil.which(hipcc):
        pytest.skip("hipcc not available")
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    out = tmp_path / "device.s"
    cmd = [hipcc, *flags, "--cuda-device-only", "-S", "-x", "hip", source, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def kernel_bodies(asm, name_part):
    """(symbol, lines) of every function whose symbol contains name_part."""
    bodies, cur, lines = [], None, []
    for line in asm.split("\n"):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            cur, lines = m.group(1), []
            continue
        if cur is not None:
            if line.startswith(".Lfunc_end"):
                if name_part in cur:
                    bodies.append((cur, lines))
                cur = None
            else:
                lines.append(line)
    return bodies


def test_prefill_m0_only_in_the_lds_load_asm(tmp_path):
    asm = device_assembly(tmp_path, SOURCE)
    bodies = kernel_bodies(asm, "prefill_kernel")
    assert len(bodies) >= 12  # f16/bf16 x head_dim 64/128/256 x block table kinds, x shared
    asm_loads = 0
    for name, lines in bodies:
        inside = False
        for line in lines:
            text = line.strip()
            if not text.startswith(";;#ASM"):
                text = text.split(";")[0].strip()  # drop the comment
            if text.startswith(ASM_BEGIN):
                inside = True
                continue
            if text.startswith(ASM_END):
                inside = False
                continue
            if inside:
                if text.startswith("global_load_lds"):
                    asm_loads += 1
                continue
            assert not re.search(r"\bm0\b", text), f"{name}: compiler code uses M0: {text}"
            # every load into LDS goes through the written-out form
            assert not text.startswith("global_load_lds"), f"{name}: {text}"
    assert asm_loads > 0
