"""The backward's workspace cache (csrc/workspace.hip) built for the host alone with
AddressSanitizer and UndefinedBehaviorSanitizer, linked against stand-ins for the HIP runtime
calls it makes (tests/native/workspace_rules.cpp) instead of the runtime itself: events stay
pending until the test finishes their stream, so each rule of the cache (idle buffer, same
stream, new slot, GPU-side wait on the oldest, replacement of the smallest, capture fallback,
error paths, the lock between host threads) is taken deterministically."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "online_softmax_fwd_flash_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"
# host-side sanitizers only: each -fsanitize= directly follows -Xarch_host
SANITIZE = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
            "-Xarch_host -fno-sanitize-recover=all").split()


@pytest.mark.skipif(not os.path.exists(HIPCC) or not os.path.exists(CLANG),
                    reason="needs hipcc and the ROCm clang for the host-only build")
def test_workspace_cache_rules(tmp_path):
    objs = []
    for src in (os.path.join(CSRC, "workspace.hip"),
                os.path.join(HERE, "native", "workspace_rules.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = ([HIPCC, "-x", "hip", "--offload-host-only", "-O1", "-g", "-fno-omit-frame-pointer",
                "-Werror=unused-value"] + SANITIZE +
               ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", obj])
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr
        objs.append(obj)
    exe = str(tmp_path / "workspace_rules")
    # linked without the HIP runtime: the stand-ins are the only definitions
    r = subprocess.run([CLANG] + objs + ["-o", exe, "-fsanitize=address,undefined", "-lpthread"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "workspace-rules ok" in r.stdout, r.stdout + r.stderr
