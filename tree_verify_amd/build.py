"""Build the HIP library (liblucev.so) for gfx950 in the package directory."""
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["api.hip", "gemm_q4.hip", "attention.hip", "attention_q8.hip", "misc.hip", "split.hip"]
LIB = os.path.join(HERE, "liblucev.so")

# Packed-fp32 VALU forms are kept out of the generated code on purpose.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-result"]
# Per-file additions.  The tree attention keeps its MFMA operands and
# accumulators in VGPRs (its softmax reads every score, which would otherwise
# travel through AGPR copies) and runs without IEEE NaN quieting, so a max
# is one instruction (no input here is NaN; the int8 quantiser beside the
# int8 attention takes only finite inputs, and its divisions and roundings
# stay IEEE-exact in either mode).
_ATTN = ["-mllvm", "-amdgpu-mfma-vgpr-form=true", "-mno-amdgpu-ieee", "-fno-honor-nans"]
EXTRA = {"attention.hip": _ATTN, "attention_q8.hip": _ATTN}


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I", os.path.join(HERE, "..", "include")]
    with tempfile.TemporaryDirectory() as tmpd:
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmpd, src + ".o")
            cmd = [hipcc] + HIPCC_FLAGS + EXTRA.get(src, []) + inc + ["-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError("hipcc failed on %s" % src)
            objs.append(obj)
        tmp = LIB + ".tmp"
        cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError("hipcc failed linking liblucev.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
