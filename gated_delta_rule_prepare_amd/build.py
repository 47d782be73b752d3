"""Build libgdn.so (the HIP kernels + C ABI) in-tree for gfx950.

Every source is compiled by hipcc to an object under ``_build/`` in parallel,
then linked into ``gated_delta_rule_prepare_amd/libgdn.so``.  Packed-FP32
instructions are disabled for all device code.  The measurement probe of the
decode's memory access pattern is linked into its own ``libgdn_probe.so``,
which only ``bench.py --rmw-probe`` loads.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgdn.so")
PROBE_SOURCES = ["probe_slot_rmw.hip"]
PROBE_LIB = os.path.join(HERE, "libgdn_probe.so")
SOURCES = ["gdn_api.cpp", "gdn_prepare.hip", "gdn_decode.hip", "gdn_prefill.hip", "gdn_epilogue.hip", "gdn_spec.hip", "gdn_kda.hip", "gdn_mamba2.hip"]
ARCH = os.environ.get("GDN_OFFLOAD_ARCH", "gfx950")
FLAGS = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES + PROBE_SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        if src in SOURCES:
            objs.append(obj)
        cmd = ["hipcc", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l and "warning: unknown target feature" not in l]
        if pr.returncode != 0:
            failed.append(src)
            sys.stderr.write(f"---- {src} ----\n" + "\n".join(lines) + "\n")
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    subprocess.run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], check=True)
    os.replace(tmp, LIB)
    pobjs = [os.path.join(BUILD, os.path.splitext(src)[0] + ".o") for src in PROBE_SOURCES]
    subprocess.run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", PROBE_LIB + ".tmp", *pobjs], check=True)
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
