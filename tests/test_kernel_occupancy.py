"""Register use of the kernels, read from the compiler's own metadata for this library's sources (gfx950),
must leave the occupancy the launch shapes were tuned for.  A 94-SGPR build of the gather kernel once
cut it from 8 to 7 waves per SIMD and ran every gather about 7% slower with no other change."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "all_gather_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
         "--cuda-device-only", "-S"]


def _kernels(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    r = subprocess.run([HIPCC, *FLAGS, "-o", str(out), src], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    txt = out.read_text()
    res = {}
    for m in re.finditer(r"\.name:\s+(\S+)\n(.*?)(?=\n  - \.|\Z)", txt, re.S):
        v = re.search(r"\.vgpr_count:\s+(\d+)", m.group(2))
        s = re.search(r"\.sgpr_count:\s+(\d+)", m.group(2))
        sp = re.search(r"\.vgpr_spill_count:\s+(\d+)", m.group(2))
        if v and s:
            res[m.group(1)] = (int(v.group(1)), int(s.group(1)), int(sp.group(1)) if sp else 0)
    return res


def _waves_per_simd(vgpr, sgpr):
    # 512 VGPRs per lane and 800 SGPRs per SIMD, allocated in granules of 8 and 16 (plus 6 reserved
    # SGPRs); at most 8 waves per SIMD
    by_v = 512 // (((vgpr + 7) // 8) * 8)
    by_s = 800 // (((sgpr + 6 + 15) // 16) * 16)
    return min(8, by_v, by_s)


@pytest.mark.slow
@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_register_use_keeps_the_tuned_occupancy(tmp_path):
    ks = _kernels(os.path.join(CSRC, "gather_kernels.hip"), tmp_path)
    ks.update(_kernels(os.path.join(CSRC, "reduce_kernels.hip"), tmp_path))
    seen = set()
    for name, (v, s, spill) in ks.items():
        assert spill == 0, f"{name} spills {spill} VGPRs"
        w = _waves_per_simd(v, s)
        wm = re.search(r"(?:Bf16|Fp16|Fp32)ELi(\d+)E", name)
        if "param_contig" in name:
            want = 8
        elif wm and int(wm.group(1)) <= 8 and "oneshot_vec" in name and name.endswith(
                tuple(["Li256ELi4ELb0EEEvNS_8RankPtrsEPcNS_11ReduceShapeEmi"])):
            want = 3  # the wide one-shot tile keeps 4 packs x W ranks in flight per lane (tuned that way)
        elif wm and int(wm.group(1)) <= 8 and "oneshot_pair" in name:
            want = 2  # two wide tiles per workgroup, the first one's results held (measured at 2 per SIMD)
        elif ("Lb1E" in name and ("oneshot_vec" in name or "twoshot_vec" in name)) or (
                "twoshot_xcd" in name and "Lb1ELb1E" in name):
            want = 2  # realigned inputs (neighbour packs moved between lanes): no spills, 2+ waves (measured)
        elif wm and int(wm.group(1)) <= 8 and "twoshot_xcd" in name:
            want = 3  # wide units plus four-unit copies: 768 resident workgroups (measured that way)
        elif wm and int(wm.group(1)) <= 8 and ("oneshot" in name or "twoshot" in name):
            want = 8  # the tuned launch shapes (W up to 8); wider W only has to avoid spills
        else:
            continue
        seen.add(name)
        assert w >= want, f"{name}: {v} VGPRs, {s} SGPRs -> {w} waves per SIMD, expected {want}"
    assert len(seen) >= 20
