"""The host code of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
the library's host part is built with both (decoder_only_transformer_amd.build_lib,
sanitize=True; device code untouched) and tests/host_sanitize/abi_hostile.c drives every entry
point with hostile arguments -- bad shapes, NULL and misaligned pointers, short workspaces,
the largest accepted shape's size arithmetic, NaN and infinite scalars."""
import os
import shutil
import subprocess

import pytest

from decoder_only_transformer_amd import build_lib

HERE = os.path.dirname(os.path.abspath(__file__))
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.timeout(600)
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    if not (os.path.exists(build_lib.HIPCC) and os.path.exists(CLANG)):
        pytest.skip("no ROCm toolchain")
    import torch
    lib = build_lib.build(verbose=False, sanitize=True)
    exe = str(tmp_path / "abi_hostile")
    cmd = [CLANG, "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           "-g", "-O1", os.path.join(HERE, "host_sanitize", "abi_hostile.c"), lib,
           f"-Wl,-rpath,{os.path.dirname(lib)}", "-Wl,-rpath,/opt/rocm/lib", "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               LD_LIBRARY_PATH="/opt/rocm/lib:" + os.environ.get("LD_LIBRARY_PATH", ""))
    if not torch.cuda.is_available():
        env["ABI_HOSTILE_NO_DEVICE"] = "1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    print(out[-4000:])
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0 and "abi_hostile: 0 failures" in out, out[-4000:]
