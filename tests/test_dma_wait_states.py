"""The LDS-DMA loads (global_load_lds_*, inline asm) need 5 wait states after
a VALU write of their base SGPRs; the compiler does not check hazards inside
inline asm and may restore a spilled base with v_readlane right before one.
This compiles both kernel files to gfx950 assembly with the build's flags and
checks every such load site. CPU only (hipcc cross-compiles)."""
import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from sampled_block_sparse_amd import build as absa_build

FILES = ["plan_kernels.hip", "attn_kernels.hip"]


def _assembly(src, out):
    flags = [f for f in absa_build.source_flags(src)
             if f not in ("-fPIC", "-Wall", "-Wno-unused-function")]
    cmd = [absa_build.hipcc(), *flags, "--cuda-device-only", "-S",
           os.path.join(absa_build.CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read()


def _short_waits(asm):
    """(site, wait states) for every DMA load with < 5 wait states between a
    VALU write of one of its base SGPRs and the load, scanning back within
    straight-line code."""
    bad = []
    sites = 0
    lines = [l.strip() for l in asm.split("\n")]
    for n, l in enumerate(lines):
        if not l.startswith("global_load_lds"):
            continue
        sites += 1
        m = re.search(r"s\[(\d+):(\d+)\]", l)
        assert m, l
        regs = (f"s{m.group(1)}", f"s{m.group(2)}")
        ws, k = 0, n - 1
        while k >= 0 and ws < 5:
            t = lines[k]
            k -= 1
            if not t or t.startswith((";", ".")):
                if t.startswith(".LBB") or t.startswith("; %bb"):
                    bad.append((n, ws, "block boundary"))   # predecessors unknown
                    break
                continue
            nop = re.match(r"s_nop (\d+)", t)
            if nop:
                ws += int(nop.group(1)) + 1
                continue
            if t.startswith("v_") and any(re.match(r"v_\w+\s+" + r + r"\b", t) for r in regs):
                bad.append((n, ws, t))
                break
            ws += 1
    return sites, bad


def test_dma_loads_wait_after_base_writes():
    try:
        absa_build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=len(FILES)) as ex:
            asms = list(ex.map(lambda f: _assembly(f, os.path.join(tmp, f + ".s")), FILES))
    total = 0
    for f, asm in zip(FILES, asms):
        sites, bad = _short_waits(asm)
        total += sites
        assert not bad, f"{f}: DMA loads without 5 wait states: {bad[:5]}"
    assert total > 0
