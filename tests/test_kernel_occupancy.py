"""Register use of the kernels, read from the compiler's own metadata for this library's sources (gfx950:
the code objects of the library's own build when it is current, else compiled here), must leave the
occupancy the launch shapes were tuned for.  A 94-SGPR build of the gather kernel once
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


LLVM = "/opt/rocm/llvm/bin"


def _metadata_from_build(src, tmp_path):
    """The kernel metadata of the library's own build of `src` (the gfx950 code object inside the fat
    binary of _build/<name>.o), if that object is newer than the source and the shared header; else None."""
    obj = os.path.join(ROOT, "_build", os.path.splitext(os.path.basename(src))[0] + ".o")
    hdr = os.path.join(CSRC, "mr_internal.h")
    if not os.path.exists(obj) or os.path.getmtime(obj) < max(os.path.getmtime(src), os.path.getmtime(hdr)):
        return None
    fb, co = tmp_path / "fatbin.bin", tmp_path / "kernels.co"
    steps = [[f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={fb}", obj, str(tmp_path / "host.o")],
             [f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o", f"--input={fb}",
              "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"]]
    for cmd in steps:
        if subprocess.run(cmd, capture_output=True, text=True, timeout=300).returncode != 0:
            return None
    r = subprocess.run([f"{LLVM}/llvm-readelf", "--notes", str(co)], capture_output=True, text=True, timeout=300)
    return r.stdout if r.returncode == 0 and ".vgpr_count" in r.stdout else None


def _kernels(src, tmp_path):
    txt = _metadata_from_build(src, tmp_path)
    if txt is None:  # no current build: compile the device code to assembly here
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
                ("Li256ELi4ELb0ELb0EEEvNS_8RankPtrsEPcNS_11ReduceShapeEmi",
                 "Li256ELi4ELb0ELb1EEEvNS_8RankPtrsEPcNS_11ReduceShapeEmi")):
            want = 3  # the wide one-shot tile keeps 4 packs x W ranks in flight per lane (tuned that way)
        elif wm and int(wm.group(1)) <= 8 and "oneshot_pipe" in name:
            want = 3  # pipelined wide tiles: three resident workgroups per CU at W=8 (measured that way)
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
