"""Build libdqk.so (gfx950) in-tree with hipcc.

Every translation unit is compiled with -ffp-contract=off (fused multiply-adds
only where the source writes them) and with packed fp32 instructions disabled.
"""
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdqk.so")
ARCH = os.environ.get("DQK_OFFLOAD_ARCH", "gfx950")

SOURCES = ["dqk_api.cpp", "dqk_select.hip", "dqk_append.hip", "dqk_decode.hip", "dqk_decode_blk.hip", "dqk_tiers.hip",
           "dqk_vrot.hip"]
# MFMA accumulators in ordinary VGPRs: the decode loop reads and rescales them
# with VALU instructions, which would otherwise copy them out of AGPRs
EXTRA = {"dqk_decode_blk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="dqk_build_") as tmp:
        procs, objs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            objs.append(obj)
            lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
            cmd = [hipcc, *COMMON, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip()]
            if p.returncode != 0:
                failed.append(src)
                sys.stderr.write("\n".join(lines) + "\n")
            elif lines and verbose:
                print("\n".join(lines))
        if failed:
            raise RuntimeError(f"hipcc failed for {failed}")
        tmp_lib = LIB + ".tmp"
        cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp_lib, *objs]
        subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
