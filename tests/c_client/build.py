"""Builds the C client of the device calls (pa_device_client.c) next to
its source: plain C99 with gcc, the ROCm headers as system headers, linked
with libpa.so and the HIP runtime.  Run by __graft_entry__.build(), so that
the GPU test only runs the program."""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
EXE = os.path.join(HERE, "pa_device_client")


def build(lib_dir: str):
    """Returns the program's path, or None (with a note) if there is no C
    compiler; the GPU test then fails and says so."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        print("note: no C compiler, the C client of the device calls is not built")
        return None
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-isystem", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "pa_device_client.c"), "-o", EXE, "-L", lib_dir, "-lpa",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           # libpa.so found relative to the program, so the tree can move
           "-Wl,-rpath,$ORIGIN/" + os.path.relpath(lib_dir, HERE),
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C client build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return EXE
