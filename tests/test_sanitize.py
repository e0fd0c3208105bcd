"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU).

Builds tests/sanitize_driver.cpp against host.cpp (the planner and the C ABI) and oracle.c,
both compiled with -fsanitize=address,undefined for the host only, plus the library's
instantiation tables (their device code is not instrumented), and runs it. The driver
makes and queries thousands of plans (valid and refused), runs the int4 repack and the LDS
permutation view over their whole domains, the attention entry's argument checks and the
oracle's C functions; any sanitizer report aborts the run."""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "dense_gemm_operand_amd")
ROCM = "/opt/rocm"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _objects():
    objs = [os.path.join(PKG, "_build", f + ".o") for f in
            ("inst_f16.hip", "inst_bf16.hip", "inst_f8.hip", "inst_misc.hip", "inst_attn.hip",
             "noalloc.hip")]
    if not all(os.path.exists(o) for o in objs):
        from dense_gemm_operand_amd import build
        build.build(oversync=False)
    return objs


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "bin", "hipcc")), reason="no ROCm toolchain")
def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    objs = _objects()
    host_o = str(tmp_path / "host_san.o")
    # host.cpp holds no device code; the sanitizers are passed to its host compilation only
    cmd = [os.path.join(ROCM, "bin", "hipcc"), "-x", "hip", "-O1", "-g", "-std=c++20", "-fPIC",
           "--offload-arch=gfx950", "-c", os.path.join(PKG, "csrc", "host.cpp"), "-o", host_o]
    for f in SAN:
        cmd[1:1] = ["-Xarch_host", f]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    oracle_o = str(tmp_path / "oracle_san.o")
    subprocess.run([clang, "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", *SAN, "-c",
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", oracle_o],
                   check=True, capture_output=True, text=True)
    exe = str(tmp_path / "sanitize_driver")
    subprocess.run([clang + "++", "-O1", "-g", "-std=c++17", *SAN, os.path.join(ROOT, "tests", "sanitize_driver.cpp"),
                    host_o, oracle_o, *objs, "-fopenmp", f"-L{ROCM}/lib", "-lamdhip64",
                    f"-Wl,-rpath,{ROCM}/lib", "-o", exe], check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, f"rc {r.returncode}\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    assert "ok: 0 failed checks" in r.stdout
