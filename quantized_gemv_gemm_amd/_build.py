"""Build libtl.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree, and record each
kernel's register, scratch and LDS use as the compiler reports it (_build/kernel_resources.json)."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import json
import os
import re
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtl.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
    "-ffp-contract=off",
    "-Wall", "-Wno-unused-function",
]
DEVICE = [
    f"--offload-arch={ARCH}",
    # no packed-fp32 instructions anywhere (the host pass warns that it does not know the feature)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


RESOURCES = os.path.join(BUILD, "kernel_resources.json")
# device assembly of the sources whose kernels count their own memory waits (read
# by the CPU tests: every counted wait must cover the loads it claims to)
ASM_SOURCES = ("k_gemv.hip", "k_gemm.hip")
_FIELDS = {"TotalSGPRs": "sgprs", "VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch",
           "Occupancy [waves/SIMD]": "occupancy", "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill",
           "LDS Size [bytes/block]": "lds"}


def _resources(remarks: str) -> dict:
    """Per-kernel register, scratch and LDS figures from the compiler's
    kernel-resource-usage remarks (mangled kernel name -> figures)."""
    out, cur = {}, None
    for line in remarks.splitlines():
        m = re.search(r"remark: +(.+?): (\S+) \[-Rpass-analysis=kernel-resource-usage\]", line)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None and key in _FIELDS:
            cur[_FIELDS[key]] = int(val) if val.lstrip("-").isdigit() else val
    return out


def _compile(src: str, build_dir: str = BUILD, defines: tuple = ()):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    flags = [f"-D{d}" for d in defines]
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", *DEVICE, *COMMON, *flags, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, *flags, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, _resources(r.stderr)


def asm_path(src_name: str) -> str:
    return os.path.join(BUILD, src_name.replace(".hip", ".s"))


def _assemble(src: str) -> str:
    out = asm_path(os.path.basename(src))
    cmd = [HIPCC, "-x", "hip", *DEVICE, *COMMON, "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"assembly listing failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source under csrc/ and link libtl.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        listings = [ex.submit(_assemble, os.path.join(CSRC, n)) for n in ASM_SOURCES]
        done = list(ex.map(_compile, srcs))
        for f in listings:
            f.result()
    objs = [o for o, _ in done]
    resources = {}
    for src, (_, res) in zip(srcs, done):
        for name, fig in res.items():
            resources[name] = dict(fig, source=os.path.basename(src))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    with open(RESOURCES, "w") as f:
        json.dump(resources, f, indent=1, sort_keys=True)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


STAMPS_DIR = os.path.join(BUILD, "stamps")             # its objects
STAMPS_LIB = os.path.join(PKG, "libtl_stamps.so")      # beside libtl.so, so that it travels with it


def build_stamps(verbose: bool = False) -> str:
    """The same library with the decode GEMV's phase timestamps compiled in
    (TL_PHASE_STAMPS=1, adds tl_phase_stamps_set), for `bench.py --phase-stamps`
    only; never loaded by the package."""
    os.makedirs(STAMPS_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = [o for o, _ in ex.map(lambda s: _compile(s, STAMPS_DIR, ("TL_PHASE_STAMPS=1",)), srcs)]
    tmp = STAMPS_LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, STAMPS_LIB)
    if verbose:
        print(f"built {STAMPS_LIB}")
    return STAMPS_LIB


if __name__ == "__main__":
    import sys
    if "--phase-stamps" in sys.argv:
        build_stamps(verbose=True)
    else:
        build(verbose=True)
