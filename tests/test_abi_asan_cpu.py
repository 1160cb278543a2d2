"""The C-ABI layer (csrc/api.hip, with the workspace cache csrc/workspace.hip) built for the
host alone with AddressSanitizer and
UndefinedBehaviorSanitizer, its kernel launchers replaced by recording stubs
(tests/native/abi_asan.cpp): every validation path, the dispatch to each launcher, the
window normalisation and the host-side block classifier run under the sanitizers, which
abort on the first finding.  No device code is built and no HIP device is made visible."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "online_softmax_fwd_flash_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# host-side sanitizers only: each -fsanitize= directly follows -Xarch_host
SANITIZE = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
            "-Xarch_host -fno-sanitize-recover=all").split()


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                    reason="needs hipcc for the host-only build")
def test_abi_layer_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_asan")
    cmd = ([HIPCC, "-x", "hip", "--offload-host-only", "-O1", "-g", "-fno-omit-frame-pointer"]
           + SANITIZE + ["-I", os.path.join(ROOT, "include"), "-I", CSRC,
                         os.path.join(CSRC, "api.hip"), os.path.join(CSRC, "workspace.hip"),
                         os.path.join(HERE, "native", "abi_asan.cpp"),
                         "-o", exe])
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1")
    env.pop("FA_LOG", None)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi-asan ok" in r.stdout, r.stdout + r.stderr
