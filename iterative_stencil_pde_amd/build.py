"""Build the engine library (``_libpk.so``) for gfx950 with hipcc, in-tree.

Usage: ``python -m iterative_stencil_pde_amd.build`` (or ``build()``).
The library is C-ABI only (``include/pk.h``); nothing here links torch.
"""

from __future__ import annotations

import hashlib
import json
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "_libpk.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",                 # the canonical sum order, no fused multiply-add
    "-fno-gpu-flush-denormals-to-zero",  # keep fp32 subnormals (the top-edge field makes them)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wextra", "-Wno-unused-parameter",
]

# the device code: launch-per-sweep and setup kernels, and the persistent kernel's
# instances, one translation unit per layout (compiled in parallel)
DEVICE_SOURCES = ["pk_kernels.hip", "pk_kern_stream_f32.hip", "pk_kern_stream_f64.hip",
                  "pk_kern_resident.hip", "pk_kern_register_f32.hip", "pk_kern_register_f64.hip"]
SOURCES = [*DEVICE_SOURCES, "pk_host.cpp"]
# the compiler's per-kernel resource report of the last build (VGPRs, SGPRs,
# scratch bytes per lane), with a hash of the sources it was made from
RESOURCE_REPORT = os.path.join(CSRC, "_build", "resource_usage.json")


def sources_sha() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".h", ".hip", ".cpp")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def parse_resource_usage(text: str) -> dict:
    """kernel-resource-usage remarks -> {mangled kernel name: {vgpr, sgpr, vgpr_spill,
    sgpr_spill, scratch}}."""
    out, name = {}, None
    for ln in text.splitlines():
        m = re.search(r"Function Name: (\S+)", ln)
        if m:
            name = m.group(1)
            out[name] = {}
            continue
        for key, pat in (("vgpr", r" VGPRs: (\d+)"), ("sgpr", r"TotalSGPRs: (\d+)"),
                         ("vgpr_spill", r"VGPRs Spill: (\d+)"), ("sgpr_spill", r"SGPRs Spill: (\d+)"),
                         ("scratch", r"ScratchSize \[bytes/lane\]: (\d+)")):
            m = re.search(pat, ln)
            if m and name:
                out[name][key] = int(m.group(1))
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(os.path.join(CSRC, "_build"), exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, "_build", src + ".o")
        cmd = [HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if src in DEVICE_SOURCES:
            cmd += ["-Rpass-analysis=kernel-resource-usage", "-fno-caret-diagnostics"]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((src, obj, cmd, subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True)))
    kernels, failed = {}, None
    for src, obj, cmd, proc in jobs:
        _, err = proc.communicate()
        # the compiler's diagnostics, without the resource remarks
        sys.stderr.write("".join(ln + "\n" for ln in err.splitlines()
                                 if "remark:" not in ln and not ln.startswith("In file included from")))
        if proc.returncode != 0 and failed is None:
            failed = subprocess.CalledProcessError(proc.returncode, cmd)
        if src in DEVICE_SOURCES:
            kernels.update(parse_resource_usage(err))
    if failed is not None:
        raise failed
    with open(RESOURCE_REPORT, "w") as f:
        json.dump({"sources_sha": sources_sha(), "kernels": kernels}, f, indent=1)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *(obj for _, obj, _, _ in jobs), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
