"""Build libmxfp4.so (HIP, gfx950) in-tree.

    python -m mxfp4_fake_quantization_amd.build

Each .hip file of the library under csrc/ is compiled by hipcc for gfx950
into _build/, then linked into mxfp4_fake_quantization_amd/libmxfp4.so.
csrc/probe_kernels.hip (streaming probes the benchmark times next to the
kernels; not part of the C ABI) becomes libmxfp4_probe.so.  Packed-FP32 VALU
instructions are disabled (-packed-fp32-ops); no fast-math.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmxfp4.so")
PROBE_LIB = os.path.join(HERE, "libmxfp4_probe.so")
PROBE_SOURCES = ["probe_kernels.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ["api.hip", "row_kernels.hip", "col_kernels.hip", "ste_kernels.hip",
           "kmajor_kernels.hip", "mxfp8_kernels.hip", "mxgemm_kernels.hip"]
CFLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES) + len(PROBE_SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    _link(objs[len(SOURCES):], PROBE_LIB)
    return _link(objs[:len(SOURCES)], LIB)


def _link(objs, lib) -> str:
    tmp = lib + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    # a kernel whose host-side launch stub was not generated links fine into a
    # shared library and only fails when loaded: refuse it here
    r = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [ln.split()[-1] for ln in r.stdout.splitlines() if "__device_stub__" in ln]
    if missing:
        os.remove(tmp)
        raise RuntimeError("kernel launch stubs missing from the host objects: " + ", ".join(missing))
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build())
    sys.exit(0)
