"""Build libalnp.so (the HIP producers and their C ABI) for gfx950 in-tree,
libalnp_floor.so (memory-only counterparts of the producers, which the
benchmark times beside them; linked against libalnp.so for its row shapes),
libalnp_timeline.so (measurement only: the same library with the FP8 row and
table kernels writing per-wave clock records, csrc/timeline.hpp), and the
compiled binding _torch_binding (the package's functions in C++ over the C
ABI: host code only, built with the C++ compiler against torch).

    python -m dit_adaptive_layernorm_amd.build      # or build() from Python

Every call recompiles.  Flags: -O3; -ffp-contract=off so that the modulation
and quantization arithmetic is evaluated exactly in the written order
(explicit __builtin_fmaf only in the variance accumulation); packed-fp32
instructions disabled in the device code generator.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libalnp.so")
FLOOR_LIB = os.path.join(PKG, "libalnp_floor.so")
TIMELINE_LIB = os.path.join(PKG, "libalnp_timeline.so")
SOURCES = ["producers.hip", "fp4.hip", "rmsmod.hip", "modulation6.hip", "residual.hip", "abi.hip"]
FLOOR_SOURCE = "floor.hip"
BINDING_SOURCE = "torch_binding.cpp"
CXX = os.environ.get("CXX", "g++")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", f"-I{INCLUDE}", f"-I{CSRC}",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # The host compiler pass warns that it does not know the packed-fp32
    # feature; that is expected.  Show anything else.
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l and l.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def _binding_commands(obj: str, tmp_so: str):
    """Compile and link commands of the compiled binding."""
    import sysconfig

    import torch

    tdir = os.path.dirname(torch.__file__)
    cflags = [
        "-O2", "-std=c++17", "-fPIC", "-Wall",
        "-DTORCH_EXTENSION_NAME=_torch_binding", "-DTORCH_API_INCLUDE_EXTENSION_H",
        f"-D_GLIBCXX_USE_CXX11_ABI={int(torch._C._GLIBCXX_USE_CXX11_ABI)}",
        # torch's ROCm headers (c10/hip/HIPStream.h) and the HIP runtime
        # headers under them expect the macros of a ROCm build of torch when
        # the compiler is not hipcc.
        "-DUSE_ROCM=1", "-D__HIP_PLATFORM_AMD__=1",
        f"-I{tdir}/include", f"-I{tdir}/include/torch/csrc/api/include",
        f"-I{sysconfig.get_paths()['include']}", "-I/opt/rocm/include", f"-I{INCLUDE}",
    ]
    compile_cmd = [CXX, *cflags, "-c", os.path.join(CSRC, BINDING_SOURCE), "-o", obj]
    link_cmd = [CXX, "-shared", obj, "-o", tmp_so, f"-L{tdir}/lib", "-lc10", "-lc10_hip",
                "-ltorch", "-ltorch_cpu", "-ltorch_hip", "-ltorch_python", f"-L{PKG}", "-lalnp",
                "-Wl,-rpath,$ORIGIN", f"-Wl,-rpath,{tdir}/lib"]
    return compile_cmd, link_cmd


def binding_path() -> str:
    import sysconfig
    return os.path.join(PKG, "_torch_binding" + sysconfig.get_config_var("EXT_SUFFIX"))


def build(verbose: bool = False, jobs: int = 7) -> str:
    with tempfile.TemporaryDirectory(prefix="alnp_build_") as tmp:
        objs, procs = [], []
        for src in SOURCES + [FLOOR_SOURCE]:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            if src != FLOOR_SOURCE:
                objs.append(obj)
            procs.append((src, [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]))
        # The timeline build's producers next to the product's, both the
        # longest compiles, so that they start together.
        tl_obj = os.path.join(tmp, "producers_timeline.o")
        procs.insert(1, ("producers.hip (timeline)",
                         [HIPCC, *FLAGS, "-DALNP_TIMELINE", "-c", os.path.join(CSRC, "producers.hip"),
                          "-o", tl_obj]))
        binding_so = binding_path()
        bind_compile, bind_link = _binding_commands(os.path.join(tmp, "torch_binding.o"),
                                                    binding_so + ".tmp")
        procs.append((BINDING_SOURCE, bind_compile))
        # Compile the translation units in parallel.
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max(1, jobs)) as ex:
            list(ex.map(lambda p: _run(p[1], verbose), procs))
        tmp_lib = LIB + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib], verbose)
        os.replace(tmp_lib, LIB)
        tmp_floor = FLOOR_LIB + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC",
              os.path.join(tmp, FLOOR_SOURCE.replace(".hip", ".o")), f"-L{PKG}", "-lalnp",
              "-Wl,-rpath,$ORIGIN", "-o", tmp_floor], verbose)
        os.replace(tmp_floor, FLOOR_LIB)
        tmp_tl = TIMELINE_LIB + ".tmp"
        tl_objs = [tl_obj if o.endswith(os.sep + "producers.o") else o for o in objs]
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *tl_objs, "-o", tmp_tl], verbose)
        os.replace(tmp_tl, TIMELINE_LIB)
        _run(bind_link, verbose)
        os.replace(binding_so + ".tmp", binding_so)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
