"""Build libmxq.so in-tree with hipcc for gfx950.

    python -m microscaling_quantization_block_amd.build

Every source is compiled each time (a build is seconds per file).  Flags:
  -ffp-contract=off                      no fused multiply-add where the format
                                         contract names two roundings
  -fno-gpu-flush-denormals-to-zero       keep binary32 subnormals
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE division for the scale chain
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed-FP32 instructions
"""

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmxq.so")
SOURCES = ["api.cpp", "quant_mxfp8.hip", "quant_nvfp4.hip", "dequant.hip", "gemm.hip", "gemm_fp8s.hip"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


COMMON = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
          "-fno-gpu-flush-denormals-to-zero", "-fhip-fp32-correctly-rounded-divide-sqrt",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


def build(verbose=False, jobs=8):
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="mxq_build_")
    try:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".", "_") + ".o")
            cmd = [cc] + COMMON + (["-x", "hip"] if src.endswith(".cpp") else []) + \
                  ["-c", os.path.join(CSRC, src), "-o", obj]
            objs.append(obj)
            procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                     stderr=subprocess.STDOUT)))
        failed = False
        for src, cmd, p in procs:
            out, _ = p.communicate()
            text = out.decode(errors="replace")
            # the host pass does not know the packed-fp32 feature: harmless
            lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
            if p.returncode != 0:
                failed = True
                sys.stderr.write(f"[mxq build] {src} failed:\n" + "\n".join(lines) + "\n")
            elif verbose and lines:
                sys.stderr.write("\n".join(lines) + "\n")
        if failed:
            raise RuntimeError("libmxq build failed")
        tmp_lib = LIB + ".tmp"
        link = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_lib] + objs + \
               ["-Wl,-rpath,/opt/rocm/lib"]
        r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if r.returncode != 0:
            raise RuntimeError("libmxq link failed:\n" + r.stdout.decode(errors="replace"))
        os.replace(tmp_lib, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
