"""Host-side check of the compiled gfx950 kernels (no GPU): the streaming
kernels' common paths for bf16 and every grouped-matmul kernel keep
everything in registers.  Register
spills go to scratch memory, whose stores are HBM writes the algorithmic
bytes do not count (a spill of five registers in the K-major pack once added
40 % to its writes).  Each source is compiled to gfx950 assembly and, for
every bf16 kernel of the vector (16-byte aligned) form, the instructions up
to its first s_endpgm -- the path taken when no block needs the generic
snap -- must not touch scratch."""
import concurrent.futures as cf
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp4_fake_quantization_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
# kernel name fragment -> symbol pattern of its bf16 (DT = 1) vector forms
FILES = {
    "mxgemm_kernels": r"mxgemm_kernel",
    "row_kernels": r"row_fwd_kernelILi1E",
    "col_kernels": r"col_fwd_kernelILi1E.*Lb1EEEv",
    "ste_kernels": r"ste_(row|col)_kernelILi1E",
    "kmajor_kernels": r"(kmajor_pack_kernelILi1E.*Lb1EEEv|dequant_\w+_kernelILi1E)",
    "mxfp8_kernels": r"mxfp8_\w+_kernelILi1E",
}


def hot_path_scratch(asm: str, pattern: str):
    out, cur, hot, done = {}, None, 0, False
    for line in asm.split("\n"):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            if cur:
                out[cur] = hot
            cur, hot, done = m.group(1), 0, False
            continue
        if cur and not done:
            if "s_endpgm" in line:
                done = True
            elif "scratch_" in line:
                hot += 1
    if cur:
        out[cur] = hot
    return {k: v for k, v in out.items() if re.search(pattern, k)}


def compile_asm(name, tmp):
    out = os.path.join(tmp, name + ".s")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", "--cuda-device-only", "-S", os.path.join(CSRC, name + ".hip"),
                    "-I", CSRC, "-o", out], check=True, capture_output=True)
    with open(out) as f:
        return f.read()


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    tmp = str(tmp_path_factory.mktemp("asm"))
    with cf.ThreadPoolExecutor(max_workers=len(FILES)) as ex:
        return dict(zip(FILES, ex.map(lambda n: compile_asm(n, tmp), FILES)))


@pytest.mark.parametrize("name", sorted(FILES))
def test_bf16_common_paths_do_not_spill(asm, name):
    found = hot_path_scratch(asm[name], FILES[name])
    assert found, f"no bf16 kernels matched in {name}"
    spilled = {k: v for k, v in found.items() if v}
    assert not spilled, f"scratch accesses on the common path: {spilled}"


def test_fp32_kmajor_pack_touches_no_scratch(asm):
    """The fp32 K-major pack holds 8 rows x 4 columns per lane (one 16-byte
    piece per row, as bf16 does with 8 columns): no scratch anywhere, the
    generic snap included (with 8 fp32 columns per lane it spilled)."""
    out, cur, n = {}, None, 0
    for line in asm["kmajor_kernels"].split("\n"):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            if cur:
                out[cur] = n
            cur, n = m.group(1), 0
        elif cur and "scratch_" in line:
            n += 1
    if cur:
        out[cur] = n
    fp32 = {k: v for k, v in out.items() if re.search(r"kmajor_pack_kernelILi0E", k)}
    assert len(fp32) == 16, sorted(fp32)
    assert not any(fp32.values()), {k: v for k, v in fp32.items() if v}


def test_matmul_kernels_touch_no_scratch(asm):
    """Every grouped-matmul instantiation (fp8 or E2M1 B, dword-aligned scale
    rows or not, 256 x 256 or the 128 x 128 tail shape) keeps its
    accumulators, prefetch and addresses in registers: no scratch access
    anywhere in the kernel."""
    out, cur, n = {}, None, 0
    for line in asm["mxgemm_kernels"].split("\n"):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            if cur:
                out[cur] = n
            cur, n = m.group(1), 0
        elif cur and "scratch_" in line:
            n += 1
    if cur:
        out[cur] = n
    gemm = {k: v for k, v in out.items() if "mxgemm_kernel" in k}
    assert len(gemm) == 24, sorted(gemm)
    assert not any(gemm.values()), {k: v for k, v in gemm.items() if v}
