"""Build libtokenswift.so in-tree with hipcc for gfx950.

Usage: python -m long_kv_attention_amd.build [-v]
"""

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "libtokenswift.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["csrc/api.cpp", "csrc/attn.hip", "csrc/select.hip", "csrc/penalty.hip", "csrc/accept.hip", "csrc/ngram.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU instructions stay disabled (the compiler would otherwise
# form them from scalar or float2 code).
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the softmax rescale touches the accumulators with
    # VALU ops, which would otherwise force AGPR<->VGPR copies every tile.
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
    "-Wall", "-Wno-unused-result",
]


def _compile(src, obj):
    # The resource-usage remarks report every kernel's scratch use: a kernel
    # that spills to scratch fails the build (the attention kernels keep their
    # LDS ring and accumulators in registers; a spill would also cost time).
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(HERE, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    lines = (r.stderr or "").splitlines()
    spills, kernel = [], None
    for l in lines:
        if "Function Name:" in l:
            kernel = l.split("Function Name:")[-1].split("[-Rpass")[0].strip()
        elif "ScratchSize [bytes/lane]:" in l and not l.rstrip().endswith(": 0") and "remark" in l:
            size = l.split("ScratchSize [bytes/lane]:")[-1].split()[0]
            if size != "0":
                spills.append(f"{kernel}: {size} bytes/lane of scratch")
    noise = ("is not a recognized feature for this target", "remark:", "[-Rpass-analysis")
    err = "\n".join(l for l in lines if not any(n in l for n in noise))
    rc = r.returncode
    if not rc and spills:
        rc, err = 1, err + "\nkernels using scratch (register spills):\n  " + "\n  ".join(spills)
    return rc, " ".join(cmd), err


def build(verbose=False, jobs=None):
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    objs = [os.path.join(out_dir, os.path.basename(s) + ".o") for s in SOURCES]
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda so: _compile(*so), zip(SOURCES, objs)))
    for rc, cmd, err in results:
        if verbose or rc:
            print(cmd)
            if err.strip():
                print(err)
        if rc:
            raise RuntimeError(f"compilation failed: {cmd}")
    tmp = LIB_PATH + ".tmp"
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"link failed: {' '.join(link)}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
