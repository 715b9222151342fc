"""Build the plain C consumer of the C-ABI (qgemv_c_client.c) with gcc,
against include/qgemv.h, the built libqgemv.so and the HIP runtime library.
Used by __graft_entry__.build() and by the CPU test that checks it links."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
LIBDIR = os.path.join(ROOT, "weight_quantized_decode_q8_amd")
SRC = os.path.join(HERE, "qgemv_c_client.c")
OUT = os.path.join(HERE, "_build", "qgemv_c_client")


def build(out: str = OUT) -> str:
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           SRC, "-o", out,
           "-L", LIBDIR, "-lqgemv", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/" + os.path.relpath(LIBDIR, os.path.dirname(os.path.abspath(out))),
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build())
