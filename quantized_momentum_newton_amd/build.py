"""Build libqmuon.so in-tree for gfx950 with hipcc.

Every HIP translation unit is compiled with packed-fp32 instructions turned
off (-Xclang -target-feature -Xclang -packed-fp32-ops) and for gfx950 only.
The q8 update unit also gets -ffp-contract=off: its binary32 arithmetic must
keep one rounding per operation to stay bit-identical to the CPU definition.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqmuon.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", "-fvisibility=hidden", "-I", os.path.join(ROOT, "include"), "-I", CSRC]

# (source, extra flags)
UNITS = [
    ("q8_update.hip", ["-ffp-contract=off"]),
    ("ns.hip", []),
    ("grasp.hip", ["-ffp-contract=off"]),
    ("hbm_stream.hip", []),
    ("plan.cpp", []),
    ("timing.cpp", ["-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include"]),
]


# Per-kernel register use of the last build (the compiler's resource-usage
# remarks), one line per kernel: name, VGPRs, AGPRs, VGPR spill, SGPR spill,
# scratch bytes per lane, occupancy.  tests/test_build_cpu.py checks it.
USAGE = os.path.join(BUILD, "kernel_resources.tsv")


def _resource_lines(stderr):
    import re
    rows, cur = [], None
    for line in stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            rows.append(cur)
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|VGPRs Spill|SGPRs Spill|ScratchSize \[bytes/lane\]|"
                      r"Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1)] = int(m.group(2))
    return ["\t".join(str(r.get(k, "")) for k in ("name", "VGPRs", "AGPRs", "VGPRs Spill", "SGPRs Spill",
                                                 "ScratchSize [bytes/lane]", "Occupancy [waves/SIMD]"))
            for r in rows]


def _compile(src, extra, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = [] if src.endswith(".hip") else ["-x", "c++"]
    remarks = ["-Rpass-analysis=kernel-resource-usage"] if src.endswith(".hip") else []
    cmd = [HIPCC, *HIP_FLAGS, *extra, *remarks, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l and "kernel-resource-usage" not in l)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj, _resource_lines(r.stderr)


def build(verbose: bool = False) -> str:
    """Compile every unit and link libqmuon.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    units = [(s, f) for s, f in UNITS if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(4, len(units))) as ex:
        done = list(ex.map(lambda u: _compile(u[0], u[1], verbose), units))
    objs = [o for o, _ in done]
    with open(USAGE, "w") as f:
        f.write("kernel\tvgprs\tagprs\tvgpr_spill\tsgpr_spill\tscratch_per_lane\toccupancy\n")
        for _, rows in done:
            f.writelines(r + "\n" for r in rows)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
