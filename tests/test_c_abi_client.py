"""A client of the C ABI in plain C (tests/host/c_abi_roundtrip.c): no Python
binding and no torch in that process. On the CPU it must compile against
include/kvtier.h as C11; on the GPU it runs every layout and path against the C
oracle compiled into it."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "hierarchical_kv_cache_backup_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(out):
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"),
           os.path.join(HERE, "host", "c_abi_roundtrip.c"),
           os.path.join(ROOT, "oracle", "kv_oracle.c"), "-o", str(out),
           "-L" + PKG, "-lkvtier", "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + PKG]
    subprocess.check_call(cmd)


def test_c_client_compiles_as_c11(tmp_path):
    if not os.path.exists(os.path.join(PKG, "libkvtier.so")):
        pytest.skip("libkvtier.so is not built")
    _build(tmp_path / "c_abi_roundtrip")


@pytest.mark.gpu
def test_c_client_round_trip(tmp_path):
    exe = tmp_path / "c_abi_roundtrip"
    _build(exe)
    print("c client: every layout x path, backup + load + kv_load_layer", flush=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failures" in res.stdout, res.stdout


def test_headers_are_c11(tmp_path):
    """Every header of the C ABI compiles in a C11 translation unit, with the
    compiler's warnings as errors."""
    src = tmp_path / "headers.c"
    src.write_text('#include "kvtier.h"\n#include "kvslots.h"\n#include "kvghost.h"\n'
                   "int main(void) { return (int)sizeof(kv_calib_t) == 0; }\n")
    subprocess.check_call(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
                           "-I" + os.path.join(ROOT, "include"), str(src), "-o",
                           str(tmp_path / "headers")])
