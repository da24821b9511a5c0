"""Build libnk.so (all HIP kernels + the C ABI) for gfx950 with hipcc.

Run as ``python -m ragged_paged_kv_amd.build`` or through
``__graft_entry__.build()``.  The library is written next to this file.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnk.so")
SOURCES = ["api.hip", "rope_write.hip", "attn_decode.hip", "attn_prefill.hip", "attn_f32.hip", "attn_backward.hip",
           "lse_merge.hip"]
ARCH = "gfx950"
# per-file extra flags: the decode kernel keeps its MFMA accumulators in
# ordinary VGPRs (its VALU rescales them every step)
FILE_FLAGS = {"attn_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # packed fp32 VALU ops are left out of the generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result", "-Wno-unknown-warning-option"]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose=False, jobs=None, extra_flags=(), out_path=None, objdir=None):
    cc = hipcc()
    objdir = objdir or os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc, *FLAGS, *FILE_FLAGS.get(src, []), *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        errs = [l for l in text.splitlines() if "error" in l.lower() and "packed-fp32-ops" not in l]
        if p.returncode != 0:
            failed.append((src, text))
        elif verbose and errs:
            print(text)
    if failed:
        for src, text in failed:
            sys.stderr.write(f"---- {src}\n{text}\n")
        raise RuntimeError("HIP compilation failed: " + ", ".join(s for s, _ in failed))
    lib = out_path or LIB
    tmp = lib + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
