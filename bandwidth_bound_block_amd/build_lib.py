"""Builds libqmv.so (hand-written HIP for gfx950) in-tree with hipcc.

Usage: python -m bandwidth_bound_block_amd.build_lib  (or call build()).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqmv.so")
SOURCES = ["qmv_host.cpp", "qmv_blocks.hip", "qmv_fmt_q8_0.hip", "qmv_fmt_q4_0.hip", "qmv_fmt_q4_1.hip", "qmv_q4k.hip", "qmv_q6k.hip", "qmv_int8.hip", "qmv_chain.hip", "qmv_decode.hip", "qmv_mma.hip", "qmv_stream.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 anywhere in the device code.
# No fast-math and no denormal flushing: fp16 scales decode exactly.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-fno-gpu-rdc", "-Wall", "-Wno-unused-function",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def build(verbose=False, extra=(), jobs=None):
    """Compiles every source to an object (in parallel, one hipcc per
    source), then links libqmv.so.  Objects go to a scratch folder beside
    the sources and are removed afterwards."""
    import concurrent.futures
    import shutil
    import tempfile
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    objdir = tempfile.mkdtemp(prefix="_build_", dir=HERE)
    try:
        compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"] + list(extra)
        objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
        cmds = [[hipcc()] + compile_flags + ["-c", s, "-o", o] for s, o in zip(srcs, objs)]
        jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = LIB + ".tmp"
        _run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-fno-gpu-rdc", "-o", tmp] + objs, verbose)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
