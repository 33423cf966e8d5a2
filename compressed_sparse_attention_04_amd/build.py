"""Build libcsa.so (the C-ABI library) from the HIP sources in csrc/.

Every .hip file is compiled for gfx950 with hipcc into an object, and the
objects are linked into one shared library against the HIP runtime that torch
itself loads, so that a process holding torch tensors and this library runs a
single HIP runtime (torch's libamdhip64.so carries no SONAME; linking it as
``-l:libamdhip64.so`` makes the library's dependency resolve to the copy torch
has already loaded).
"""

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libcsa.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    # packed-FP32 VALU ops stay off in every kernel of this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
    # MFMA results in ordinary VGPRs (gfx950 allows either): the indexer
    # epilogues then read their accumulators without v_accvgpr_read copies
    # (pooled scoring 779 -> 715 VALU instructions per wave, the decode scan
    # 1,582 -> 1,486); no kernel spills with it
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


# Host-side sanitizers for the checked build (the device code is unchanged):
# every -fsanitize= right after -Xarch_host, so only the host pass gets it.
SANITIZE_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                  "-Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer").split()
SAN_DIR = os.path.join(BUILD_DIR, "san")
SAN_LIB_PATH = os.path.join(SAN_DIR, "libcsa_san.so")


def sanitizer_runtime():
    """The clang ASan runtime (its shared library also carries the UBSan
    handlers), preloaded into a process that loads the checked build."""
    import glob
    libs = glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))
    return sorted(libs)[-1] if libs else None


def torch_lib_dir():
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.origin:
        return None
    d = os.path.join(os.path.dirname(spec.origin), "lib")
    return d if os.path.exists(os.path.join(d, "libamdhip64.so")) else None


def _compile(src, obj, extra):
    cmd = [HIPCC] + HIP_FLAGS + ["-I" + INCLUDE, "-I" + CSRC] + extra + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature; drop that noise
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, " ".join(cmd), err


def build(verbose=False, extra_flags=None, jobs=None, sanitize=False):
    """Compile every csrc/*.hip and link libcsa.so; returns the library path.

    sanitize=True builds the checked variant instead (host code under
    AddressSanitizer and UBSan, objects in _build/san, library
    _build/san/libcsa_san.so); load it with the runtime from
    sanitizer_runtime() preloaded."""
    obj_dir = SAN_DIR if sanitize else BUILD_DIR
    lib_path = SAN_LIB_PATH if sanitize else LIB_PATH
    os.makedirs(obj_dir, exist_ok=True)
    extra = list(extra_flags or []) + (SANITIZE_FLAGS if sanitize else [])
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    if not srcs:
        raise RuntimeError("no HIP sources found in " + CSRC)
    objs = []
    jobs = jobs or min(8, len(srcs))
    with cf.ThreadPoolExecutor(jobs) as ex:
        futs = {}
        for s in srcs:
            obj = os.path.join(obj_dir, s[:-4] + ".o")
            objs.append(obj)
            futs[ex.submit(_compile, os.path.join(CSRC, s), obj, extra)] = s
        failed = []
        for f in cf.as_completed(futs):
            rc, cmd, err = f.result()
            if verbose or rc != 0:
                print(cmd)
                if err.strip():
                    print(err)
            if rc != 0:
                failed.append(futs[f])
    if failed:
        raise RuntimeError("HIP compile failed: " + ", ".join(sorted(failed)))
    tdir = torch_lib_dir()
    link = [CLANG, "-shared", "-fPIC", "-o", lib_path + ".tmp"] + objs
    if tdir:
        link += ["-L" + tdir, "-l:libamdhip64.so", "-Wl,-rpath," + tdir]
    else:
        link += ["-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
                 "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    # the checked build leaves the sanitizer runtime's symbols to the preloaded runtime
    link += ["-lstdc++"] if sanitize else ["-Wl,--no-undefined", "-lstdc++"]
    r = subprocess.run(link, capture_output=True, text=True)
    if verbose or r.returncode != 0:
        print(" ".join(link))
        print(r.stderr)
    if r.returncode != 0:
        raise RuntimeError("link failed")
    os.replace(lib_path + ".tmp", lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
