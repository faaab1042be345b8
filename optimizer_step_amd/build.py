"""Build the HIP library libopt_step.so for gfx950, in-tree.

hipcc flags: -O3, no FMA contraction (-ffp-contract=off) so the binary32
recipe runs in the written order, packed-fp32 instructions disabled, and the
default correctly rounded fp32 division and square root.
"""
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libopt_step.so")
# (source, extra flags): the blockwise step compiles once per parameter storage
SOURCES = [("opt_api.cpp", []), ("opt_kernels.hip", []), ("opt_kernels_ew.hip", []), ("opt_kernels_1s.hip", []),
           ("opt_kernels_q8.hip", ["-DOPT_Q8_PD=0"]), ("opt_kernels_q8.hip", ["-DOPT_Q8_PD=1"]),
           ("opt_kernels_q8.hip", ["-DOPT_Q8_PD=2"])]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-I", CSRC, "-I", os.path.join(ROOT, "include"),
]


def hipcc():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


# The host pass of hipcc does not know the packed-fp32 target feature (it is
# a device feature) and says so once per compile; that line is dropped.
_HARMLESS = "'-packed-fp32-ops' is not a recognized feature for this target"


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    text = "\n".join(l for l in r.stdout.splitlines() if _HARMLESS not in l)
    if text.strip():
        print(text, flush=True)
    if r.returncode != 0:
        raise subprocess.CalledProcessError(r.returncode, cmd)


def build(verbose=False, out=LIB, extra_flags=()):
    tmpdir = tempfile.mkdtemp(prefix="optstep_build_")
    try:
        objs, cmds = [], []
        for i, (src, flags) in enumerate(SOURCES):
            obj = os.path.join(tmpdir, f"{i}_{src}.o")
            cmd = [hipcc(), *HIPCC_FLAGS, *flags, *extra_flags, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            cmds.append(cmd)
            objs.append(obj)
        # the translation units compile independently: in parallel
        with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as pool:
            for f in [pool.submit(_run, c) for c in cmds]:
                f.result()
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
