"""Summaries of rocprofv3 output for the HSTU attention kernels.

    python -m hstu_jagged_masked_amd.profiling stats DIR          # --kernel-trace --stats CSVs
    python -m hstu_jagged_masked_amd.profiling pmc DIR [DIR ...]  # --pmc counter CSVs
    python -m hstu_jagged_masked_amd.profiling traffic FETCH_DIR WRITE_DIR OUT.json
    python -m hstu_jagged_masked_amd.profiling isa                # compiled hot loops

``stats`` prints per-kernel launch count and average / total duration.
``pmc`` prints the average of each counter per dispatch, per kernel.
``traffic`` turns FETCH_SIZE and WRITE_SIZE (KiB per dispatch) into HBM bytes per
launch of each MFMA/streaming kernel.
``isa`` compiles the MFMA kernels' sources to gfx950 assembly (the library's
own flags) and prints the instruction mix of each basic block that issues
at least 16 MFMAs (the tile and step bodies): MFMAs, transcendentals, other
VALU instructions, LDS reads, and, where the block evaluates SiLU (two
transcendentals per score element), those counts per 64 score elements, i.e.
per accumulator register.  The raw counters are scaled by the
factor that maps the same counter of a plain device-to-device copy of known
size (the ``bench.py`` calibration copy, a device-to-device hipMemcpy that the
runtime performs with its copy kernel; the largest such dispatch in the run)
onto its true byte count, read and write separately.  The JSON records the
sha256 of each kernel's source so a reader can tell whether it is still current.
"""
from __future__ import annotations

import collections
import csv
import glob
import hashlib
import json
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
KERNELS = ("k_fwd_bf16", "k_bwd_kv", "k_bwd_kv_p", "k_bwd_kv_atomic", "k_bwd_q", "k_bwd_dq",
           "k_targets_fwd", "k_targets_bwd")
KERNEL_SOURCES = {"k_fwd_bf16": ["fwd.hip"], "k_bwd_kv": ["bwd.hip"], "k_bwd_kv_p": ["bwd.hip"],
                  "k_bwd_kv_atomic": ["bwd.hip", "atomic_dq.h"],
                  "k_bwd_q": ["bwd.hip"],
                  "k_bwd_dq": ["dq.hip"], "k_targets_fwd": ["targets.hip"],
                  "k_targets_bwd": ["targets.hip"]}
COMMON_SOURCES = ["common.h", "tiles.h"]
COPY_KERNEL = "__amd_rocclr_copybuffer"  # the HIP runtime's device-to-device copy kernel


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES.get(kernel, []) + COMMON_SOURCES:
        with open(os.path.join(PKG, "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def short_name(name: str) -> str:
    m = re.search(r"(k_\w+)(<[^>]*>)?", name)
    if m and "hstu" in name:
        # the key-owner kernel's instantiations <store P, atomic dQ> are named
        # as in the library's own timing
        if m.group(1) == "k_bwd_kv" and m.group(2):
            targs = [a.strip() for a in m.group(2)[1:-1].split(",")]
            if targs[0] == "true":
                return "k_bwd_kv_p"
            if len(targs) > 1 and targs[1] == "true":
                return "k_bwd_kv_atomic"
        return m.group(1)
    return name.split("(")[0][-60:]


def read_rows(path_glob):
    rows = []
    for f in sorted(glob.glob(path_glob, recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def stats(directory: str) -> str:
    """Per-kernel durations from the kernel trace, one line per (kernel, grid
    size): the production workload and the smaller ones bench.py also runs
    (the padded-interval comparison) launch the same kernels on other grids."""
    rows = read_rows(os.path.join(directory, "**", "*kernel_trace.csv"))
    groups = collections.defaultdict(list)
    for r in rows:
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        groups[(short_name(r["Kernel_Name"]), grid)].append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6)
    total = sum(sum(v) for v in groups.values())
    out = ["kernel                        grid  calls   avg_ms      total_ms   pct"]
    for (name, grid), ds in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"{name[:26]:26s} {grid:8d} {len(ds):6d} {sum(ds) / len(ds):9.4f} "
                   f"{sum(ds):11.3f} {100.0 * sum(ds) / total:6.2f}")
    return "\n".join(out)


def pmc_table(directories, largest_grid=True):
    """Counter values per kernel name; with largest_grid, only the dispatches
    on each kernel's largest grid (the production workload)."""
    rows = []
    for d in directories:
        rows.extend(read_rows(os.path.join(d, "**", "*counter_collection.csv")))
    top = collections.defaultdict(int)
    for r in rows:
        top[r["Kernel_Name"]] = max(top[r["Kernel_Name"]], int(r["Grid_Size"]))
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in rows:
        if largest_grid and int(r["Grid_Size"]) != top[r["Kernel_Name"]]:
            continue
        agg[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return agg


def pmc(directories) -> str:
    agg = pmc_table(directories)
    out = []
    for name, counters in sorted(agg.items(), key=lambda kv: short_name(kv[0])):
        short = short_name(name)
        if short not in KERNELS:
            continue
        out.append(f"== {short}")
        avg = {c: sum(vals) / len(vals) for c, vals in counters.items()}
        for c in sorted(avg):
            out.append(f"   {c:32s} {avg[c]:.6g}")
        out.extend(derived(avg))
    return "\n".join(out)


SIMDS = 1024  # 256 CUs x 4 SIMDs


def derived(avg) -> list:
    """Ratios of one kernel's counters (per-dispatch averages): VALU
    instructions per MFMA instruction, the share of wave cycles spent waiting
    for any instruction's inputs, the share of MFMA-busy cycles in which VALU
    work co-executed, and MFMA-busy cycles per SIMD (divide by the kernel's
    duration times the shader clock for the busy fraction)."""
    out = []

    def ratio(name, num, den):
        if num in avg and den in avg and avg[den]:
            out.append(f"   {name:32s} {avg[num] / avg[den]:.4g}")

    ratio("VALU per MFMA instruction", "SQ_INSTS_VALU", "SQ_INSTS_MFMA")
    ratio("wait cycles per wave cycle", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES")
    ratio("co-executed per MFMA-busy cycle", "SQ_VALU_MFMA_COEXEC_CYCLES",
          "SQ_VALU_MFMA_BUSY_CYCLES")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
        out.append(f"   {'MFMA-busy cycles per SIMD':32s} "
                   f"{avg['SQ_VALU_MFMA_BUSY_CYCLES'] / SIMDS:.4g}")
    return out


def _calibration(agg, counter):
    """(counter value, true bytes) of the largest copy kernel dispatch."""
    best = None
    for name, counters in agg.items():
        if COPY_KERNEL not in name.lower() or counter not in counters:
            continue
        v = max(counters[counter])
        if best is None or v > best:
            best = v
    return best


def traffic(fetch_dir: str, write_dir: str, out_path: str, copy_bytes: int) -> dict:
    fa, wa = pmc_table([fetch_dir]), pmc_table([write_dir])
    f_cal, w_cal = _calibration(fa, "FETCH_SIZE"), _calibration(wa, "WRITE_SIZE")
    if not f_cal or not w_cal:
        raise SystemExit("no calibration copy kernel found in the counter runs")
    f_scale = copy_bytes / (f_cal * 1024.0)
    w_scale = copy_bytes / (w_cal * 1024.0)
    result = {"_calibration": {"copy_bytes": copy_bytes, "fetch_kib": f_cal, "write_kib": w_cal,
                               "fetch_scale": f_scale, "write_scale": w_scale}}
    for name in set(fa) | set(wa):
        short = short_name(name)
        if short not in KERNELS:
            continue
        fk = fa.get(name, {}).get("FETCH_SIZE")
        wk = wa.get(name, {}).get("WRITE_SIZE")
        if not fk or not wk:
            continue
        fb = sum(fk) / len(fk) * 1024.0 * f_scale
        wb = sum(wk) / len(wk) * 1024.0 * w_scale
        result[short] = {"fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
                         "bytes_per_launch": fb + wb, "source_sha256": source_digest(short)}
    with open(out_path, "w") as f:
        json.dump(result, f, indent=1, sort_keys=True)
    return result


ISA_SOURCES = ("fwd.hip", "bwd.hip", "dq.hip")
TRANSCENDENTAL = ("v_exp_f32", "v_rcp_f32")


def isa_blocks(asm_text: str):
    """[(kernel, block, Counter of opcodes)] over the blocks of each kernel."""
    out, kernel, block, ops = [], None, None, None
    for line in asm_text.splitlines():
        t = line.strip()
        m = re.match(r"^(_Z\w+):", line)
        if m:
            kernel, block, ops = short_name_isa(m.group(1)), "entry", collections.Counter()
            out.append((kernel, block, ops))
            continue
        if kernel is None or not t or t.startswith(";"):
            continue
        if t.startswith(".Lfunc_end"):
            kernel = None
            continue
        m = re.match(r"^(\.LBB\w+):", t)
        if m:
            block, ops = m.group(1), collections.Counter()
            out.append((kernel, block, ops))
            continue
        if t.startswith("."):
            continue
        ops[t.split()[0]] += 1
    return out


def short_name_isa(symbol: str) -> str:
    m = re.search(r"(k_\w+?)(I[LbB0-9E]+)?E", symbol)
    name = m.group(1) if m else symbol[:40]
    if name == "k_bwd_kv" and "k_bwd_kvILb1E" in symbol:
        name = "k_bwd_kv_p"
    elif name == "k_bwd_kv" and "k_bwd_kvILb0ELb1E" in symbol:
        name = "k_bwd_kv_atomic"
    return name


def isa(build_dir: str = None) -> str:
    import subprocess
    from . import build as bld
    build_dir = build_dir or bld.BUILD
    os.makedirs(build_dir, exist_ok=True)
    flags = [f for f in bld.COMPILE_FLAGS if not f.startswith("-Rpass")]
    lines = ["kernel           block       mfma trans valu  lds_rd | per 64 elements: valu trans "
             "(valu = other vector ALU instructions)"]
    for src in ISA_SOURCES:
        out = os.path.join(build_dir, src + ".s")
        cmd = [bld.HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(PKG, "csrc", src),
               "-o", out]
        proc = subprocess.run(cmd, capture_output=True, text=True)
        if proc.returncode != 0:
            raise RuntimeError(f"hipcc -S failed for {src}:\n{proc.stderr}")
        with open(out) as f:
            for kernel, block, ops in isa_blocks(f.read()):
                mfma = sum(v for k, v in ops.items() if k.startswith("v_mfma"))
                if mfma < 16:
                    continue
                trans = sum(v for k, v in ops.items() if k.startswith(TRANSCENDENTAL))
                valu = sum(v for k, v in ops.items() if k.startswith("v_") and
                           not k.startswith(("v_mfma", "v_accvgpr") + TRANSCENDENTAL))
                lds = sum(v for k, v in ops.items() if k.startswith("ds_read"))
                per = (f"{valu / (trans / 2):6.2f} {2.0:5.1f}" if trans else "")
                lines.append(f"{kernel:16s} {block:11s} {mfma:4d} {trans:5d} {valu:4d} {lds:6d}"
                             f" | {per}")
    return "\n".join(lines)


def main(argv):
    if len(argv) >= 2 and argv[0] == "stats":
        print(stats(argv[1]))
    elif len(argv) >= 2 and argv[0] == "pmc":
        print(pmc(argv[1:]))
    elif len(argv) >= 1 and argv[0] == "isa":
        print(isa())
    elif len(argv) >= 4 and argv[0] == "traffic":
        copy_bytes = int(argv[4]) if len(argv) > 4 else 1 << 30
        print(json.dumps(traffic(argv[1], argv[2], argv[3], copy_bytes), indent=1))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
