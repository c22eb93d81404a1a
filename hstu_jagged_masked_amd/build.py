"""Build libhstu_attn.so (gfx950) in-tree with hipcc.

Every HIP source under csrc/ is compiled to an object in _build/ (in parallel)
and linked into hstu_jagged_masked_amd/libhstu_attn.so.  No fast-math: the
kernels rely on IEEE fp32 behaviour of adds and multiplies.  Packed fp32 vector
instructions are disabled for the device code.

The compiler's per-kernel resource report is checked: the MFMA kernels must
keep two waves per SIMD and must not fall back to scratch memory for their
register arrays (a register array the compiler cannot keep in registers costs
an order of magnitude in speed, with no other symptom).  The report is written
to _build/resource_usage.txt.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libhstu_attn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMPILE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-Rpass-analysis=kernel-resource-usage",
    "-I", INCLUDE, "-I", CSRC,
]

# kernels whose resources are checked (by mangled-name fragment; the key-owner
# kernel's instantiations <store P, atomic dQ> separately): (minimum waves per
# SIMD, maximum scratch bytes per lane).  The atomic-dQ instantiation runs one
# wave per SIMD by design.  A few bytes of scratch are spills of values used outside
# the tile loops; hundreds mean a register array was demoted to memory.
HOT_KERNELS = {"k_fwd_bf16": (2, 64), "k_bwd_kvILb0ELb0E": (2, 192), "k_bwd_kvILb1ELb0E": (2, 192),
               "k_bwd_kvILb0ELb1E": (1, 64), "k_bwd_q": (2, 64), "k_bwd_dq": (2, 64)}


def _resource_report(stderr: str):
    """[(kernel, {field: value})] from -Rpass-analysis=kernel-resource-usage remarks."""
    out, cur = [], None
    for line in stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            out.append(cur)
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\S+) \[-Rpass", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return out


def _check_resources(reports) -> list:
    problems = []
    for r in reports:
        for kern, (min_occ, max_scratch) in HOT_KERNELS.items():
            if kern not in r["name"]:
                continue
            occ = int(r.get("Occupancy", "0"))
            scratch = int(r.get("ScratchSize", "0"))
            if occ < min_occ or scratch > max_scratch:
                problems.append(f"{kern} ({r['name']}): occupancy {occ} waves/SIMD (need >= "
                                f"{min_occ}), scratch {scratch} B/lane (allowed {max_scratch})")
    return problems


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMPILE_FLAGS, "-c", src, "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{proc.stderr}")
    return obj, _resource_report(proc.stderr)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        results = list(ex.map(_compile, srcs))
    objs = [o for o, _ in results]
    reports = [r for _, rs in results for r in rs]
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        for r in reports:
            f.write(" ".join(f"{k}={v}" for k, v in r.items()) + "\n")
    problems = _check_resources(reports)
    if problems:
        raise RuntimeError("kernel resource check failed:\n  " + "\n  ".join(problems))
    tmp = LIBRARY + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed:\n{proc.stderr}")
    os.replace(tmp, LIBRARY)
    if verbose:
        print(f"built {LIBRARY} from {len(srcs)} sources")
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
