"""Build libmx.so (the HIP library behind include/mx.h) in-tree for gfx950.

    python -m precision_block_amax_amd.build

Each translation unit is compiled with hipcc in parallel, then linked into a
shared library next to this file.  The packed-fp32 target feature is turned
off (hipcc would otherwise form v_pk_{add,mul,fma}_f32 from scalar code), and
fp contraction is off so the rotation's adds and multiplies round one by one.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from typing import List

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libmx.so")
SOURCES = tuple(sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")))
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS: List[str] = [
    "--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stdout))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stdout)
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


def resource_usage(out_path: str) -> None:
    """Compile every translation unit with hipcc's kernel-resource-usage remarks and write a
    table of each kernel's VGPRs, AGPRs, SGPRs, spills, LDS bytes and waves per SIMD."""
    import re
    cmd_shown = "python -m precision_block_amax_amd.build --resource-usage " + os.path.relpath(out_path, ROOT)
    def remarks(src):
        cmd = [HIPCC] + CFLAGS + ["-c", os.path.join(CSRC, src), "-o", os.devnull,
                                  "-Rpass-analysis=kernel-resource-usage"]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stdout))
        return src, r.stdout

    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 4)) as ex:
        outputs = list(ex.map(remarks, SOURCES))
    rows = []
    for src, text in outputs:
        cur = None
        for line in text.splitlines():
            m = re.search(r"remark: Function Name: (\S+)", line)
            if m:
                cur = {"kernel": m.group(1), "tu": src}
                rows.append(cur)
                continue
            m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^]]*\])?: (\d+)", line)
            if m and cur is not None:
                cur[m.group(1).strip()] = int(m.group(2))
    seen, uniq = set(), []
    for r in rows:
        if r["kernel"] not in seen and "k_" in r["kernel"]:
            seen.add(r["kernel"])
            uniq.append(r)
    demangle = subprocess.run(["c++filt"], input="\n".join(r["kernel"] for r in uniq), stdout=subprocess.PIPE,
                              text=True).stdout.splitlines()
    lines = ["# Kernel resources (hipcc -Rpass-analysis=kernel-resource-usage, gfx950)", "",
             "Command (run from the repository root):", "", "    " + cmd_shown, "",
             "Registers per lane; LDS per workgroup; occupancy in waves per SIMD as the compiler reports it. "
             "One kernel per template instantiation, first translation unit that emits it.", "",
             "| kernel | VGPRs | AGPRs | SGPRs | VGPR spills | SGPR spills | LDS (bytes) | waves/SIMD |",
             "|---|---|---|---|---|---|---|---|"]
    for r, name in zip(uniq, demangle):
        name = name.replace("mx::(anonymous namespace)::", "").replace("(mx::GemmArgs)", "")
        name = re.sub(r"\(.*\)$", "", name)
        lines.append("| `%s` | %s | %s | %s | %s | %s | %s | %s |" % (
            name, r.get("VGPRs", "?"), r.get("AGPRs", "?"), r.get("TotalSGPRs", "?"), r.get("VGPRs Spill", "?"),
            r.get("SGPRs Spill", "?"), r.get("LDS Size", "?"), r.get("Occupancy", "?")))
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "--resource-usage":
        resource_usage(os.path.abspath(sys.argv[2]))
    else:
        build(verbose=True)
    sys.exit(0)
