"""Build the HIP library (liblucev.so) for gfx950 in the package directory."""
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["api.hip", "gemm_q4.hip", "attention.hip", "attention_kvq.hip", "misc.hip", "split.hip"]
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
EXTRA = {"attention.hip": _ATTN, "attention_kvq.hip": _ATTN}


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I", os.path.join(HERE, "..", "include")]
    import concurrent.futures
    with tempfile.TemporaryDirectory() as tmpd:
        def one(src):
            obj = os.path.join(tmpd, src + ".o")
            cmd = [hipcc] + HIPCC_FLAGS + EXTRA.get(src, []) + inc + ["-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError("hipcc failed on %s" % src)
            return obj

        # the sources compile independently (one hipcc each, in parallel)
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(6, len(SOURCES))) as ex:
            objs = list(ex.map(one, SOURCES))
        tmp = LIB + ".tmp"
        cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError("hipcc failed linking liblucev.so")
    os.replace(tmp, LIB)
    return LIB


def asan_runtime() -> str:
    """The ASan runtime of the ROCm clang (it carries the UBSan handlers too)."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/lib/llvm")
    return hits[-1]


def build_host_sanitized(out_dir: str) -> str:
    """The library with AddressSanitizer and UndefinedBehaviorSanitizer on its
    host code (argument validation, the host packer, planning, workspace
    sizing), for CPU tests that launch no kernel: the device code is built
    unoptimised, only so the objects link.  Load it with asan_runtime()
    preloaded."""
    import concurrent.futures
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I", os.path.join(HERE, "..", "include")]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

    def one(src):
        obj = os.path.join(out_dir, src + ".o")
        cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-Wno-unused-result",
               "-Xarch_device", "-O0"] + san + inc + ["-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc (sanitized) failed on %s:\n%s" % (src, res.stdout + res.stderr))
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(6, len(SOURCES))) as ex:
        objs = list(ex.map(one, SOURCES))
    out = os.path.join(out_dir, "liblucev_host_san.so")
    res = subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + san + objs + ["-o", out],
                         capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("linking the sanitized build failed")
    return out


if __name__ == "__main__":
    print(build(verbose=True))
