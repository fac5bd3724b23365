"""Build the HIP library libgla.so in-tree for gfx950.

The device code is compiled by hipcc with packed-fp32 instructions disabled;
the host API layer is plain C++.  The result lands next to this file so that
it travels with the source tree.
"""

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgla.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


# per-source additions: the backward chunk kernel keeps its matrix-core
# accumulators in ordinary vector registers (the default form parks them in
# accumulation registers and copies every result out, ~300 extra VALU
# instructions per wave there)
EXTRA_FLAGS = {
    # the persistent chunk kernel's LDS-writing loads are assembly that sets
    # m0 (which nothing else in it uses)
    "gla_bwd_kernels.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-Wno-inline-asm"],
    # the single-pass kernel's likewise
    "gla_fused.hip": ["-Wno-inline-asm"],
}


def flags_for(src):
    """hipcc flags of one device source file (its base name)."""
    return HIP_FLAGS + EXTRA_FLAGS.get(src, [])


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build step failed: %s\n%s" % (" ".join(cmd), out))
    return out


# Host sanitizer build (CPU checking of the C-ABI layer): with sanitize=True
# (command line: --sanitize) gla_api.cpp, the only host-logic source, is also
# compiled by g++ with AddressSanitizer and UndefinedBehaviorSanitizer and
# linked with the same device objects into libgla_san.so.  Load it with the
# sanitizer runtimes preloaded, e.g.
#   LD_PRELOAD="$(gcc -print-file-name=libasan.so) $(gcc -print-file-name=libubsan.so)" \
#   ASAN_OPTIONS=detect_leaks=0 GLA_LIBRARY=recurrent_vision_token_amd/libgla_san.so \
#   python -m pytest tests/test_abi.py tests/test_host_logic.py -m "not gpu"
LIB_SAN = os.path.join(PKG, "libgla_san.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]


def build(verbose=False, sanitize=False):
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    os.makedirs(BUILD, exist_ok=True)
    k_obj = os.path.join(BUILD, "gla_kernels.o")
    a_obj = os.path.join(BUILD, "gla_api.o")
    logs = []
    s_obj = os.path.join(BUILD, "swiglu_kernels.o")
    g_obj = os.path.join(BUILD, "saga_kernels.o")
    b_obj = os.path.join(BUILD, "gla_bwd_kernels.o")
    f_obj = os.path.join(BUILD, "gla_fused.o")
    n_obj = os.path.join(BUILD, "gla_noalloc.o")
    logs.append(_run([hipcc] + flags_for("gla_kernels.hip") + ["-I", INCLUDE, "-I", CSRC, "-c",
                                            os.path.join(CSRC, "gla_kernels.hip"), "-o", k_obj]))
    logs.append(_run([hipcc] + flags_for("swiglu_kernels.hip") + ["-I", INCLUDE, "-I", CSRC, "-c",
                                            os.path.join(CSRC, "swiglu_kernels.hip"), "-o", s_obj]))
    logs.append(_run([hipcc] + flags_for("saga_kernels.hip") + ["-I", INCLUDE, "-I", CSRC, "-c",
                                            os.path.join(CSRC, "saga_kernels.hip"), "-o", g_obj]))
    logs.append(_run([hipcc] + flags_for("gla_bwd_kernels.hip") + ["-I", INCLUDE, "-I", CSRC, "-c",
                                            os.path.join(CSRC, "gla_bwd_kernels.hip"), "-o", b_obj]))
    logs.append(_run([hipcc] + flags_for("gla_fused.hip") + ["-I", INCLUDE, "-I", CSRC, "-c",
                                            os.path.join(CSRC, "gla_fused.hip"), "-o", f_obj]))
    logs.append(_run([hipcc] + flags_for("gla_noalloc.hip") + ["-I", INCLUDE, "-I", CSRC, "-c",
                                            os.path.join(CSRC, "gla_noalloc.hip"), "-o", n_obj]))
    api_flags = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__",
                 "-I", os.path.join(ROCM, "include"), "-I", INCLUDE, "-I", CSRC]
    dev_objs = [k_obj, s_obj, g_obj, b_obj, f_obj, n_obj]
    logs.append(_run(["g++"] + api_flags + ["-c", os.path.join(CSRC, "gla_api.cpp"), "-o", a_obj]))
    tmp = LIB + ".tmp"
    logs.append(_run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + dev_objs + [a_obj,
                      "-o", tmp]))
    os.replace(tmp, LIB)
    if sanitize:
        # the same device objects, the host layer instrumented; g++ links its
        # own sanitizer runtimes
        san_obj = os.path.join(BUILD, "gla_api_san.o")
        logs.append(_run(["g++"] + SAN_FLAGS + api_flags +
                         ["-c", os.path.join(CSRC, "gla_api.cpp"), "-o", san_obj]))
        tmp = LIB_SAN + ".tmp"
        logs.append(_run(["g++", "-shared"] + SAN_FLAGS + dev_objs + [san_obj] +
                         ["-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-o", tmp]))
        os.replace(tmp, LIB_SAN)
    if verbose:
        print("\n".join(x for x in logs if x.strip()))
    return LIB


if __name__ == "__main__":
    import sys
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))
