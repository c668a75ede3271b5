"""Build the plain C client of libkvscore (kvscore_c_client.c) with gcc, C99, against
include/kvscore.h and the HIP runtime's C API; the executable finds libkvscore.so in the
package directory through its rpath. Run by the repository's build step, not by a test."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "kvscore_c_client.c")
EXE = os.path.join(HERE, "kvscore_c_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    pkg = os.path.join(ROOT, "kv_cache_eviction_kvscore_amd")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}", SRC, "-o", EXE + ".tmp",
           f"-L{pkg}", "-lkvscore", f"-L{ROCM}/lib", "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../kv_cache_eviction_kvscore_amd", f"-Wl,-rpath,{ROCM}/lib"]
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    if verbose:
        print(f"built {EXE}")
    return EXE


if __name__ == "__main__":
    build(verbose=True)
