"""Build ``libmac_attention.so`` (gfx950) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmac_attention.so")
# Diagnostic build with the step kernel's per-workgroup timeline (the marks
# compile to nothing in LIB); its objects go to a folder of their own.
TIMELINE_LIB = os.path.join(PKG, "libmac_attention_timeline.so")
TIMELINE_OBJ = os.path.join(ROOT, "_build", "timeline")
# The one-launch step kernels are split by (K/V dtype, head dim) so that
# the sources compile in parallel.
SOURCES = ["mac_step_bf16_128.hip", "mac_kernels.hip", "mac_step_bf16_64.hip",
           "mac_step_f32_128.hip", "mac_step_f32_64.hip", "mac_api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 anywhere in the device code.
# -ffp-contract=on: a multiply-add is fused only within one source
# expression, never across statements by the backend, so a device function
# rounds the same way in every kernel that inlines it (the one-launch and
# three-kernel forms of the decode step agree bit for bit).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=on",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def build(verbose: bool = False, extra: list | None = None, jobs: int = 0,
          timeline: bool = False) -> str:
    """Compile every source (``jobs`` at a time; 0 = one per source, at most
    the CPU count) and link the shared library (with ``timeline``, the
    diagnostic TIMELINE_LIB instead)."""
    objs, cmds = [], []
    lib, odir = LIB, CSRC
    if timeline:
        lib, odir = TIMELINE_LIB, TIMELINE_OBJ
        extra = [*(extra or []), "-DMAC_TIMELINE"]
        os.makedirs(odir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(odir, src.replace(".hip", ".o"))
        cmds.append([HIPCC, *FLAGS, *(extra or []), "-I", INCLUDE, "-I", CSRC, "-c",
                     os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    n = jobs or max(1, min(len(cmds), os.cpu_count() or 1))

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)

    with concurrent.futures.ThreadPoolExecutor(n) as ex:
        for f in [ex.submit(run, c) for c in cmds]:
            f.result()
    tmp = lib + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                           *objs, "-o", tmp])
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, timeline="--timeline" in sys.argv))
