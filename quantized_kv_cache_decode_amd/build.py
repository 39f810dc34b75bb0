"""Build libtqattn.so for gfx950 with hipcc (in-tree, next to this file).

    python -m quantized_kv_cache_decode_amd.build
Each .hip file under csrc/ is compiled to an object under _build/ in parallel,
then linked into quantized_kv_cache_decode_amd/libtqattn.so.
"""
import concurrent.futures as cf
import glob
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libtqattn.so")
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: no AGPR<->VGPR copies around the softmax rescale
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
]


RESOURCE_REPORT = os.path.join(HERE, "_build", "kernel_resources.txt")


def _compile(src, obj):
    cmd = [HIPCC, *DEVICE_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-fno-caret-diagnostics", "-c", src,
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("is not a recognized feature for this target", "kernel-resource-usage")
    err = "\n".join(l for l in r.stderr.splitlines() if not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return err, _resources(r.stderr)


def _resources(remarks):
    """(kernel, VGPRs, scratch bytes per lane) from the compiler's resource-usage remarks."""
    out, name, vgpr = [], None, None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r" VGPRs: (\d+)", line)
        if m:
            vgpr = int(m.group(1))
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name:
            out.append((name, vgpr, int(m.group(1))))
    return out


def build(verbose: bool = True) -> str:
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, os.path.basename(s) + ".o") for s in srcs]
    report = []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        for s, (msg, res) in zip(srcs, ex.map(_compile, srcs, objs)):
            if verbose and msg.strip():
                print(f"[{os.path.basename(s)}]\n{msg}", file=sys.stderr)
            report += [f"{os.path.basename(s)} {k} vgpr={v} scratch={sc}" for k, v, sc in res]
    with open(RESOURCE_REPORT, "w") as f:
        f.write("\n".join(report) + "\n")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
