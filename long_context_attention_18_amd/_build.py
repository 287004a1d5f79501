"""Builds liblca.so (the HIP library behind include/lca.h) for gfx950.

hipcc cross-compiles here without a GPU. Flags:
  -ffp-contract=off   every floating-point operator is one IEEE operation
                      (the compressor's fp64 pooling must be reproducible);
                      fused multiply-adds are written explicitly.
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      keep the compiler from forming packed fp32 VALU ops.
  -mllvm --amdgpu-mfma-vgpr-form
                      MFMA accumulators in VGPRs: an accumulator the VALU
                      also touches (attention's output rescale) is otherwise
                      copied between AGPRs and VGPRs on every loop trip.
"""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblca.so")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(force: bool = True, verbose: bool = False) -> str:
    deps = sources() + glob.glob(os.path.join(CSRC, "*.h")) + [os.path.join(HERE, "..", "include", "lca.h")]
    if not force and os.path.exists(LIB) and all(os.path.getmtime(LIB) >= os.path.getmtime(d) for d in deps):
        return LIB
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    procs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = ["hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "--amdgpu-mfma-vgpr-form",
               "-Wall", "-Wno-unused-function", "-c", src, "-o", obj]
        procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT), src))
        objs.append(obj)
    failed = []
    for p, src in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # the host pass does not know the GPU target feature; that warning is harmless
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l or "error" in l)
        if verbose or p.returncode != 0:
            if text.strip():
                print(text)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp = LIB + ".tmp"
    subprocess.run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
