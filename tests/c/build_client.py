"""Build tests/c/fs_c_client (a plain C consumer of include/fs.h) with gcc,
linked against the built libfsstate.so and the HIP runtime."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "fs_c_client.c")
OUT = os.path.join(HERE, "fs_c_client")
LIBDIR = os.path.join(ROOT, "fsdp_sharded_state_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(force: bool = True) -> str:
    lib = os.path.join(LIBDIR, "libfsstate.so")
    if not force and os.path.exists(OUT) and os.path.getmtime(OUT) >= max(os.path.getmtime(SRC),
                                                                           os.path.getmtime(lib)):
        return OUT
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}", SRC, "-o", OUT,
           f"-L{LIBDIR}", "-lfsstate", f"-Wl,-rpath,{LIBDIR}", f"-L{ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,{ROCM}/lib", "-lm"]
    subprocess.run(cmd, check=True)
    return OUT


if __name__ == "__main__":
    print(build())
