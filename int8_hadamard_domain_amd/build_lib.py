"""Build libi8h.so in-tree with hipcc for gfx950 (run on a machine with ROCm;
no GPU needed). `python -m int8_hadamard_domain_amd.build_lib` or build().

Every kernel's resource use (registers, LDS, private memory, spills) comes
from the compiler's resource remarks and goes to _build/kernel_resources.txt;
the build fails if any kernel needs private (scratch) memory, a dynamic stack
or spills vector registers: none of the kernels is meant to touch memory
outside its arguments and LDS."""

import concurrent.futures as cf
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build", "obj")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libi8h.so")
# the measurement probes (HBM read bandwidth, FP8 matrix-core precision, MFMA/VALU overlap):
# their own library
PROBE_LIB = os.path.join(LIBDIR, "libi8h_probe.so")
PROBE_SOURCES = ["probe.hip", "probe_fp8_mfma.hip", "probe_overlap.hip"]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed FP32 instructions are kept out of every kernel (the compiler would
# otherwise form them from plain float code).
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]

RESOURCES = os.path.join(ROOT, "_build", "kernel_resources.txt")

SOURCES = ["abi.hip", "route.hip", "fwht.hip", "gateup_i8h_gemv.hip", "gateup_gemm.hip", "gateup_fp8.hip",
           "down.hip", "linear.hip", "gateup_skinny.hip", "gateup_i8g.hip"]


def _resources(src, stderr):
    """Per-kernel resource remarks of one compile: [(kernel, {field: value})]."""
    out, cur = [], None
    for line in stderr.splitlines():
        m = re.search(r"remark:\s+(.*?)\s+\[-Rpass-analysis=kernel-resource-usage\]", line)
        if not m:
            continue
        text = m.group(1)
        if text.startswith("Function Name:"):
            cur = {}
            out.append((text.split(":", 1)[1].strip(), cur))
        elif cur is not None and ":" in text:
            key, val = text.rsplit(":", 1)
            cur[key.strip()] = val.strip()
    return [(src, name, fields) for name, fields in out]


def _compile(src):
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return out, _resources(src, r.stderr)


def _check_resources(rows):
    """Write the resource table; raise if a kernel uses private memory."""
    keys = ["VGPRs", "AGPRs", "TotalSGPRs", "LDS Size [bytes/block]", "Occupancy [waves/SIMD]",
            "ScratchSize [bytes/lane]", "Dynamic Stack", "VGPRs Spill", "SGPRs Spill"]
    lines = ["# source  kernel  " + "  ".join(k.replace(" ", "_") for k in keys)]
    bad = []
    for src, name, f in rows:
        lines.append(f"{src}  {name}  " + "  ".join(f.get(k, "?") for k in keys))
        if f.get("ScratchSize [bytes/lane]", "0") != "0" or f.get("Dynamic Stack", "False") != "False" \
                or f.get("VGPRs Spill", "0") != "0":
            bad.append(f"{src}: {name}: scratch {f.get('ScratchSize [bytes/lane]')} B/lane, "
                       f"VGPR spills {f.get('VGPRs Spill')}, dynamic stack {f.get('Dynamic Stack')}")
    with open(RESOURCES, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    if bad:
        raise RuntimeError("kernels that use private memory:\n  " + "\n  ".join(bad))


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        done = dict(zip(srcs, ex.map(_compile, srcs)))
    objs = {s: o for s, (o, _) in done.items()}
    rows = [row for s in srcs for row in done[s][1]]
    if not rows:
        raise RuntimeError("hipcc printed no kernel resource remarks")
    _check_resources(rows)
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
