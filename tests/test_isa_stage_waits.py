"""The GEMM stage loops wait only as designed (CPU: cross-compiled gfx950
assembly, no GPU). The ring's correctness and speed rest on constant
`s_waitcnt vmcnt(N)` waits; the compiler adds a full drain, `vmcnt(0)`,
wherever it cannot prove an in-flight DMA or load is done, and such a drain
inside a stage loop stalls every step. The innermost loop holding the MFMAs
must carry exactly one vector-memory wait: (STAGES-3)*DPS for the read-ahead
loop, (STAGES-2)*DPS for the 3-stage loops. Two things once put extra drains
there and are kept out: reading the expert order from the kernel arguments
with a lane-varying index (a vector load; the order now comes from an LDS
copy), and weight-gradient kernels holding every output mode's epilogue (the
accumulating epilogues' loads into registers; each mode is now its own
kernel). Any further wait is a regression."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "moe_grouped_block_mx_amd", "csrc", "gemm_mx.hip")

# kernel name fragment (TileCfg parameters) -> the waits its stage loop must carry
EXPECTED = {
    # a4w4 forward / input gradient: 8 waves, 128-deep stages, 4-stage
    # read-ahead ring, DPS 5 (Lb1: every stage full, scalar-base DMA issue;
    # Lb0: the general issue)
    "grouped_fwd_kernelINS_7TileCfgILi256ELi256ELi2ELi4ELi128ELi4ELi0ELi1ELi7ELi1EEELb1E": [5],
    "grouped_dgrad_kernelINS_7TileCfgILi256ELi256ELi2ELi4ELi128ELi4ELi0ELi1ELi7ELi1EEELb1E": [5],
    "grouped_fwd_kernelINS_7TileCfgILi256ELi256ELi2ELi4ELi128ELi4ELi0ELi1ELi7ELi1EEELb0E": [5],
    "grouped_dgrad_kernelINS_7TileCfgILi256ELi256ELi2ELi4ELi128ELi4ELi0ELi1ELi7ELi1EEELb0E": [5],
    # the same with both operands' codes in 64-byte K blocks
    "grouped_fwd_kernelINS_8KBlockedINS_7TileCfgILi256ELi256ELi2ELi4ELi128ELi4ELi0ELi1ELi7ELi1EEEEELb1E": [5],
    "grouped_dgrad_kernelINS_8KBlockedINS_7TileCfgILi256ELi256ELi2ELi4ELi128ELi4ELi0ELi1ELi7ELi1EEEEELb1E": [5],
    "grouped_fwd_kernelINS_8KBlockedINS_5MfmaBINS_7TileCfgILi256ELi256ELi2ELi4ELi128ELi4ELi0ELi1ELi7ELi1EEEEEEELb1E": [5],
    "grouped_dgrad_kernelINS_8KBlockedINS_5MfmaBINS_7TileCfgILi256ELi256ELi2ELi4ELi128ELi4ELi0ELi1ELi7ELi1EEEEEEELb1E": [5],
    # the same with the weights' scales in the MFMA layout
    "grouped_fwd_kernelINS_5MfmaBINS_7TileCfgILi256ELi256ELi2ELi4ELi128ELi4ELi0ELi1ELi7ELi1EEEEELb1E": [5],
    "grouped_dgrad_kernelINS_5MfmaBINS_7TileCfgILi256ELi256ELi2ELi4ELi128ELi4ELi0ELi1ELi7ELi1EEEEELb1E": [5],
    "grouped_fwd_kernelINS_5MfmaBINS_7TileCfgILi256ELi256ELi2ELi4ELi128ELi4ELi0ELi1ELi7ELi1EEEEELb0E": [5],
    "grouped_dgrad_kernelINS_5MfmaBINS_7TileCfgILi256ELi256ELi2ELi4ELi128ELi4ELi0ELi1ELi7ELi1EEEEELb0E": [5],
    # a4w4 weight gradient: 4 waves, same ring, DPS 10 (every output mode)
    "grouped_wgrad_kernelINS_7TileCfgILi256ELi256ELi2ELi2ELi128ELi4ELi0ELi1ELi7ELi1EEELb0E": [10],
    # power-of-two blockwise forward / input gradient (operands in 64-byte K
    # blocks): 64-deep stages, 3-stage ring, DPS 6
    "grouped_fwd_kernelINS_8KBlockedINS_7TileCfgILi256ELi256ELi2ELi4ELi64ELi3ELi3ELi1ELi5ELi128EEEEELb1E": [6],
    "grouped_dgrad_kernelINS_8KBlockedINS_7TileCfgILi256ELi256ELi2ELi4ELi64ELi3ELi3ELi1ELi5ELi128EEEEELb1E": [6],
    "grouped_fwd_kernelINS_8KBlockedINS_7TileCfgILi256ELi256ELi2ELi4ELi64ELi3ELi3ELi1ELi5ELi128EEEEELb0E": [6],
    "grouped_dgrad_kernelINS_8KBlockedINS_7TileCfgILi256ELi256ELi2ELi4ELi64ELi3ELi3ELi1ELi5ELi128EEEEELb0E": [6],
    # MXFP8 weight gradient (DPS 5, general issue) and power-of-two blockwise
    # weight gradient (DPS 6, scalar-base issue), every output mode
    "grouped_wgrad_kernelINS_7TileCfgILi256ELi256ELi2ELi4ELi64ELi3ELi4ELi1ELi5ELi1EEELb0E": [5],
    # blockwise FP8 weight gradient, power-of-two scales (operands in 64-byte
    # K blocks): 4 waves, stage read-ahead, 4-stage ring, DPS 10, two steps
    # per loop iteration (every output mode)
    "grouped_wgrad_kernelINS_8KBlockedINS_7TileCfgILi256ELi256ELi2ELi2ELi64ELi4ELi3ELi1ELi8ELi1EEEEELb1E": [10, 10],
}


def _hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return h if os.path.exists(h) else None


def stage_loop_waits(asm_lines):
    """{kernel label: [vmcnt values of the waits in the innermost loop holding
    its MFMAs]}, from the block structure the compiler prints in comments."""
    out, kern, blocks, cur = {}, None, {}, None

    def finish():
        if kern is None:
            return
        # the loop whose blocks hold the most MFMAs (a stage loop unrolled by
        # two leaves a one-stage tail in the enclosing tile loop)
        count = {}
        for hdr, lines in blocks.values():
            if hdr:
                count[hdr] = count.get(hdr, 0) + sum("v_mfma" in l for l in lines)
        loops = [hdr for hdr, n in count.items() if n > 0]
        assert loops, kern
        h = max(loops, key=lambda x: count[x])
        out[kern] = [int(m.group(1)) for hdr, lines in blocks.values() if hdr == h
                     for l in lines for m in [re.search(r"s_waitcnt vmcnt\((\d+)\)", l)] if m]

    for line in asm_lines:
        m = re.match(r"^(_ZN4mxgg\S*_kernel\S*):", line)  # kernel entry labels only
        if m:
            finish()
            kern, blocks, cur = m.group(1), {}, "entry"
            blocks[cur] = (None, [])
            continue
        if kern is None:
            continue
        if line.startswith(".LBB") or line.startswith("; %bb."):
            name = line.split(":")[0].strip().lstrip(".").replace("; %", "")
            if "This Loop Header" in line or "This Inner Loop Header" in line:
                hdr = name.replace("LBB", "BB")
            else:
                mh = re.search(r"Header=(BB\d+_\d+)", line)
                hdr = mh.group(1) if mh else None
            cur = name
            blocks[cur] = (hdr, [])
            continue
        if ("This Loop Header" in line or "This Inner Loop Header" in line) and not blocks[cur][1]:
            # a header comment wrapped onto the line after the label
            blocks[cur] = (cur.replace("LBB", "BB"), [])
            continue
        blocks[cur][1].append(line)
        if "s_endpgm" in line:
            finish()
            kern = None
    return out


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_stage_loops_carry_only_the_ring_wait(tmp_path):
    asm = tmp_path / "gemm.s"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", f"-I{os.path.join(ROOT, 'include')}", "--cuda-device-only", "-S", SRC, "-o", str(asm)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    waits = stage_loop_waits(asm.read_text().splitlines())
    for frag, want in EXPECTED.items():
        found = [k for k in waits if frag in k]
        assert found, (frag, list(waits))
        for k in found:
            assert waits[k] == want, (k, waits[k])
