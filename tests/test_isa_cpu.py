"""CPU check of the prefill kernels' machine code (gfx950 assembly from
hipcc, no GPU needed): the LDS-DMA loads set M0 in their own asm statement
without declaring it clobbered, which is sound only while nothing the
compiler emits in these kernels reads or writes M0.  Every M0 reference in
the assembly must be such a load's own set, followed by its load."""
import os
import re
import subprocess

import pytest

from chunked_prefill_causal_rope_amd import build as lib_build


def test_m0_only_feeds_the_lds_dma_loads(tmp_path):
    try:
        cc = lib_build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    src = os.path.join(lib_build.CSRC, "prefill_bf16.hip")
    out = tmp_path / "prefill_bf16.s"
    r = subprocess.run([cc, *lib_build.COMMON_FLAGS, "--cuda-device-only", "-S", "-o", str(out), src],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln.split(";")[0].strip() for ln in out.read_text().splitlines()]
    uses = [i for i, ln in enumerate(lines) if re.search(r"\bm0\b", ln)]
    assert uses, "no LDS-DMA load in the prefill kernels"
    for i in uses:
        assert re.match(r"s_mov_b32 m0, s\d+$", lines[i]), f"M0 used by the compiler: {lines[i]!r}"
        nxt = next(ln for ln in lines[i + 1:] if ln)
        assert nxt.startswith("buffer_load_dwordx4") and nxt.endswith(" lds"), f"M0 set for {nxt!r}"
