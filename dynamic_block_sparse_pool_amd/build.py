"""Build libdbsp.so in-tree with hipcc for gfx950.

    python -m dynamic_block_sparse_pool_amd.build [--verbose] [--save-temps DIR]

Every .hip file under csrc/ is compiled to an object in _build/ (in parallel), then linked into
dynamic_block_sparse_pool_amd/libdbsp.so next to this file. The benchmark's read-bandwidth
probe (csrc/probe/) is built into its own libdbsp_probe.so beside it.
"""
from __future__ import annotations

import argparse
import glob
import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libdbsp.so")
PROBE_PATH = os.path.join(PKG_DIR, "libdbsp_probe.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

# Packed fp32 VALU forms are switched off for all device code: hipcc would otherwise form them
# from ordinary float code.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, save_temps: str | None = None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmd = [HIPCC, *COMMON_FLAGS, "-c", src, "-o", obj]
        if save_temps:
            os.makedirs(save_temps, exist_ok=True)
            cmd.insert(1, f"-save-temps={'obj'}")
            cmd[-1] = os.path.join(save_temps, os.path.basename(src) + ".o")
            obj = cmd[-1]
        objs.append(obj)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            cwd=save_temps or BUILD_DIR)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # the host pass does not know the packed-fp32 feature name; that notice is harmless
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if p.returncode != 0:
            failed.append(src)
            print("\n".join(lines), file=sys.stderr)
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"hipcc failed for: {', '.join(os.path.basename(f) for f in failed)}")
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    build_probe(verbose)
    return LIB_PATH


def build_probe(verbose: bool = False) -> str:
    """The benchmark's read-bandwidth probe, a separate small library."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip")))
    tmp = PROBE_PATH + ".tmp"
    cmd = [HIPCC, *COMMON_FLAGS, "-shared", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if p.returncode != 0:
        print(p.stdout.decode(errors="replace"), file=sys.stderr)
        raise RuntimeError("hipcc failed for the read-bandwidth probe")
    os.replace(tmp, PROBE_PATH)
    return PROBE_PATH


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--save-temps", default=None, help="keep intermediate files (ISA) in DIR")
    args = ap.parse_args(argv)
    path = build(verbose=args.verbose, save_temps=args.save_temps)
    print(path)


if __name__ == "__main__":
    main()
