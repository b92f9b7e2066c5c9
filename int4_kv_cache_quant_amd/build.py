"""Build libotq.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc.

Flags:
  --offload-arch=gfx950           MI355X only; no other targets are built.
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                  no packed fp32 VALU instructions are emitted.
  -fhip-fp32-correctly-rounded-divide-sqrt, -fno-gpu-flush-denormals-to-zero
                                  IEEE fp32 division and denormals, which the
                                  bit-exact quantiser relies on.
  -ffp-contract=off (quantiser)   one rounding per fp32 operation.
  -mllvm -amdgpu-mfma-vgpr-form (MFMA split kernel)
                                  accumulators stay in VGPRs instead of being
                                  copied to and from AGPRs around every rescale.
"""
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libotq.so")
ROOT = os.path.dirname(HERE)

SOURCES = ["api.hip", "quantize.hip", "sdpa_vec.hip", "sdpa_mfma.hip", "combine.hip", "order.hip", "bits.hip",
           "wide.hip", "probe.hip", "bits_mfma.hip"]
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
          "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]
PER_FILE = {"quantize.hip": ["-ffp-contract=off"], "bits.hip": ["-ffp-contract=off"],
            "wide.hip": ["-ffp-contract=off"],
            # keep MFMA accumulators in VGPRs: they are rescaled by VALU ops
            "sdpa_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
            "bits_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else shutil.which("hipcc")


def build(verbose: bool = False, jobs: int = 5) -> str:
    hipcc = _hipcc()
    if not hipcc:
        raise RuntimeError("hipcc not found: cannot build libotq for gfx950")
    tmp = tempfile.mkdtemp(prefix="otq_build_")
    try:
        procs, objs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = [hipcc, *COMMON, *PER_FILE.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
            if len([p for _, p in procs if p.poll() is None]) >= jobs:
                procs[0][1].wait()
        for src, p in procs:
            out, _ = p.communicate()
            if p.returncode != 0:
                sys.stderr.write(out.decode(errors="replace"))
                raise RuntimeError(f"hipcc failed on {src}")
            if verbose and out:
                sys.stderr.write(out.decode(errors="replace"))
        cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(LIB + ".tmp", LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
