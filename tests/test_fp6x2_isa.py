"""The gfx950 scaled fp6 conversions write their first result dwords before
they read their last operand registers, so a result register range that
overlaps an operand's turns the last elements wrong. The kernels issue them
with results apart from their operands; this check compiles fp6x2.hip for
gfx950 and verifies it in every instance (CPU only: hipcc cross-compiles)."""

import re
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
SRC = ROOT / "mxfp4_expert_top_amd" / "csrc" / "fp6x2.hip"
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not Path(HIPCC).exists(), reason="hipcc not installed")
def test_scaled_fp6_conversions_do_not_overlap_their_operands(tmp_path):
    out = tmp_path / "fp6x2.s"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang",
                    "-target-feature", "-Xclang", "-packed-fp32-ops",
                    f"-I{ROOT / 'include'}", f"-I{SRC.parent}", "--cuda-device-only", "-S",
                    "-o", str(out), str(SRC)], check=True, capture_output=True)
    n = 0
    for line in out.read_text().splitlines():
        m = re.search(r"v_cvt_scalef32_(?:2xpk16_fp6_f32|pk32_f32_fp6)\s+v\[(\d+):(\d+)\],(.*)",
                      line)
        if not m:
            continue
        n += 1
        d0, d1 = int(m.group(1)), int(m.group(2))
        for a, b in re.findall(r"v\[(\d+):(\d+)\]", m.group(3)):
            assert int(b) < d0 or int(a) > d1, line
        for a in re.findall(r"(?<![\[:\d])v(\d+)\b", m.group(3)):
            assert not d0 <= int(a) <= d1, line
    assert n >= 8
