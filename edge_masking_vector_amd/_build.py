"""Build libtilemap.so in-tree with hipcc for gfx950.

Every source is compiled to an object in parallel, then linked into one shared library next to
this file.  Flags:
  --offload-arch=gfx950                      MI355X only
  -O3 -ffp-contract=off                      no implicit contraction; the kernels call fmaf
                                             explicitly where the map is fused
  -fno-gpu-flush-denormals-to-zero           f32 subnormals are kept, as on the CPU
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                             no packed-f32 instructions in device code
  -fvisibility=hidden                        only the tm_* C ABI is exported
"""
import concurrent.futures
import os
import shutil
import subprocess
import sysconfig

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtilemap.so")
# The CPython extension that binds the C ABI (csrc/pyext.c), next to the library it links.
EXT = os.path.join(HERE, "_tilemap" + sysconfig.get_config_var("EXT_SUFFIX"))
SOURCES = ["plan.cpp", "map.hip", "mapflat.hip", "rowred.hip", "colred.hip", "transpose.hip", "api.hip",
           "noalloc.hip"]
# Per-source flags.  mapflat.hip: its kernels' arguments are preloaded into scalar registers at
# wave launch (gfx940-family kernel-argument preloading; the code object keeps the plain argument
# loads as a prologue for firmware without it), so a short-lived wave starts its load sooner.
EXTRA_FLAGS = {"mapflat.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=6"]}

ARCH = "gfx950"
FLAGS = [
    "-std=c++17", "-O3", "-fPIC", "-fvisibility=hidden", "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wextra", "-Wno-unused-parameter",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: libtilemap.so needs ROCm's hipcc to build")


def _compile(hipcc, src):
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [hipcc, "--offload-arch=" + ARCH, *FLAGS, *EXTRA_FLAGS.get(src, []), "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-f32 feature name; that warning is harmless.
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, err))
    return obj, err


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libtilemap.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(OBJDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: _compile(hipcc, s), SOURCES))
    for _, err in results:
        if verbose and err.strip():
            print(err)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *[o for o, _ in results], "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    build_ext()
    return LIB


def build_ext() -> str:
    """Compile csrc/pyext.c with the host C compiler into the `_tilemap` extension module, linked
    against libtilemap.so and finding it through an $ORIGIN run path."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no host C compiler (gcc) to build the _tilemap extension")
    tmp = EXT + ".tmp%d" % os.getpid()
    cmd = [cc, "-std=c11", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"), "-I", sysconfig.get_paths()["include"],
           os.path.join(CSRC, "pyext.c"), "-L", HERE, "-ltilemap", "-Wl,-rpath,$ORIGIN", "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building the _tilemap extension failed:\n" + r.stderr)
    os.replace(tmp, EXT)
    return EXT


if __name__ == "__main__":
    print(build(verbose=True))
