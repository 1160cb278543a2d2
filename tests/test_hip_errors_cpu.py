"""HIP runtime failures map to FA_ERR_HIP through the C ABI, and FA_LOG names the kernel
instantiation a call chose.

Each case runs in a fresh interpreter whose environment hides every HIP device
(HIP_VISIBLE_DEVICES=-1) before the library loads.  The child first asks the HIP runtime how
many devices it sees and calls nothing else unless that is none, so no call can reach a GPU:
the entry points then pass validation and fail in the runtime (hipGetDevice, hipMallocAsync
or the launch), which each must report as FA_ERR_HIP (3) without raising."""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = textwrap.dedent('''
    import ctypes, sys
    sys.path.insert(0, {root!r})
    hip = ctypes.CDLL("libamdhip64.so")
    n = ctypes.c_int(0)
    if hip.hipGetDeviceCount(ctypes.byref(n)) == 0 and n.value > 0:
        print("DEVICE-VISIBLE")
        sys.exit(5)
    from online_softmax_fwd_flash_amd import _lib
    L = _lib.lib()
    A = ctypes.c_void_p(0x1000)   # aligned; never dereferenced (no device exists)
    S0 = ctypes.c_void_p(0)
    lay_q = _lib.Layout(16 * 4 * 64, 4 * 64, 64)
    lay_k = _lib.Layout(16 * 2 * 64, 2 * 64, 64)
    for dt, D in ((1, 128), (2, 64), (0, 64), (0, 8)):
        dims = (1, 16, 4, 2, D, 0.125, 1, 0, dt, S0)
        print("fwd", dt, D, L.flash_attn_fwd(A, A, A, A, A, *dims))
        print("bwd", dt, D, L.flash_attn_bwd(*([A] * 9), *dims))
        print("bwd_noalloc", dt, D, L.flash_attn_bwd_noalloc(*([A] * 9), *dims))
        print("dkdv", dt, D, L.flash_attn_bwd_dkdv(*([A] * 8), *dims, 0, 0))
        print("dq_dvec", dt, D, L.flash_attn_bwd_dq_dvec(*([A] * 8), *dims, 0, 0))
    print("pre", L.flash_attn_bwd_preprocess(A, A, A, 1, 16, 4, 64, 1, S0))
    print("fwd_strided", L.flash_attn_fwd_strided(A, A, A, A, A, 1, 16, 16, 4, 2, 64, 0.125, 1,
                                                  0, 1, S0, lay_q, lay_k))
    print("rope", L.flash_attn_qk_norm_rope(A, 8 * 64, 64, A, A, 64, A, A, 16, 4, 64, 64, 0, 0,
                                            1, S0))
    # beyond the fixed scratch: refused (FA_ERR_UNSUPPORTED) before any HIP call
    print("noalloc_too_big", L.flash_attn_bwd_noalloc(*([A] * 9), 2, _lib.FA_NOALLOC_MAX_DVEC // 16
                                                       + 1, 8, 2, 64, 0.125, 1, 0, 1, S0))
    print("DONE")
''')


def run_child(env_extra):
    env = dict(os.environ)
    env.pop("FA_LOG", None)
    env.update(env_extra)
    env["HIP_VISIBLE_DEVICES"] = "-1"
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT)], capture_output=True,
                       text=True, timeout=120, env=env)
    if r.returncode == 5 and "DEVICE-VISIBLE" in r.stdout:
        pytest.skip("a HIP device stayed visible; the failure cannot be forced safely")
    assert r.returncode == 0, r.stdout + r.stderr
    assert "DONE" in r.stdout
    return r


def test_runtime_failures_map_to_fa_err_hip():
    r = run_child({})
    lines = [line.split() for line in r.stdout.splitlines() if line and line != "DONE"]
    codes = {" ".join(x[:-1]): x[-1] for x in lines}
    assert len(codes) == 24
    assert codes.pop("noalloc_too_big") == "2"
    assert set(codes.values()) == {"3"}, r.stdout
    assert "flash_attn:" not in r.stderr


def test_fa_log_names_the_instantiation():
    r = run_child({"FA_LOG": "1"})
    # the f32 kernels need no LDS attribute, so their launch is attempted (and fails) and
    # logged; the log names the tiling and head-dim instantiation chosen for D = 64 and D = 8
    assert "flash_attn: fwd_f32_kernel<DP=64,BQ=64,BK=64> elem=f32 D=64" in r.stderr
    assert "flash_attn: fwd_f32_kernel<DP=8,BQ=64,BK=64> elem=f32 D=8" in r.stderr
    assert "flash_attn: bwd_preprocess_kernel elem=bf16 D=64" in r.stderr
    assert "flash_attn: qk_norm_rope_kernel elem=bf16 D=64" in r.stderr
