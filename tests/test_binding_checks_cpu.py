"""The Python binding rejects tensors the kernels cannot take before any library call: CPU
tensors (whose host pointers would reach the kernels as device addresses), and, on the GPU,
mixed dtypes, non-contiguous inputs, V of another shape than K, and L / Dvec / gradient
buffers of the wrong shape or dtype.  The library is replaced by a stand-in that fails the
test if it is ever reached."""
import pytest
import torch

import online_softmax_fwd_flash_amd as fa
from online_softmax_fwd_flash_amd import _lib


class _NoLib:
    def __getattr__(self, name):
        raise AssertionError(f"library entry point {name} reached despite invalid tensors")


@pytest.fixture
def no_lib(monkeypatch):
    monkeypatch.setattr(_lib, "lib", lambda: _NoLib())


def _cpu_inputs(dtype=torch.bfloat16):
    B, T, H, HKV, D = 1, 16, 4, 2, 64
    q = torch.zeros(B, T, H, D, dtype=dtype)
    k = torch.zeros(B, T, HKV, D, dtype=dtype)
    v = torch.zeros(B, T, HKV, D, dtype=dtype)
    do = torch.zeros(B, T, H, D, dtype=dtype)
    o = torch.zeros(B, T, H, D, dtype=dtype)
    lse = torch.zeros(B, H, T)
    dvec = torch.zeros(B, H, T)
    return q, k, v, do, o, lse, dvec


def _calls(q, k, v, do, o, lse, dvec):
    return {
        "fwd": lambda: fa.flash_attn_fwd(q, k, v),
        "bwd": lambda: fa.flash_attn_bwd(q, k, v, o, lse, do),
        "bwd_dkdv": lambda: fa.flash_attn_bwd_dkdv(q, k, v, do, lse, dvec),
        "bwd_dq": lambda: fa.flash_attn_bwd_dq(q, k, v, do, lse, dvec),
        "bwd_dq_dvec": lambda: fa.flash_attn_bwd_dq_dvec(q, k, v, o, do, lse),
        "bwd_preprocess": lambda: fa.flash_attn_bwd_preprocess(o, do),
        "fwd_strided": lambda: fa.flash_attn_fwd_strided(q, k, v),
        "bwd_strided": lambda: fa.flash_attn_bwd_strided(q, k, v, o, lse, do),
        "bwd_grad16": lambda: fa.flash_attn_bwd_grad16(q, k, v, o, lse, do),
    }


@pytest.mark.parametrize("entry", list(_calls(*_cpu_inputs())))
def test_cpu_tensors_never_reach_the_library(no_lib, entry):
    with pytest.raises(ValueError):
        _calls(*_cpu_inputs())[entry]()


def test_unsupported_dtype_rejected(no_lib):
    ins = _cpu_inputs(torch.float64)
    for name, call in _calls(*ins).items():
        with pytest.raises(ValueError):
            call()


def test_non_tensor_rejected(no_lib):
    q, k, v, do, o, lse, dvec = _cpu_inputs()
    with pytest.raises(ValueError):
        fa.flash_attn_fwd(None, k, v)
    with pytest.raises(ValueError):
        fa.flash_attn_qk_norm_rope(None, lse, lse, 2)


def _gpu_mismatches():
    """(entry, description, call factory) for every mismatch the backward entry points must
    catch; each factory builds valid CUDA tensors and spoils exactly one."""
    B, T, H, HKV, D = 1, 64, 4, 2, 64

    def make(**spoil):
        dev = "cuda"
        bf = torch.bfloat16
        t = dict(q=torch.zeros(B, T, H, D, dtype=bf, device=dev),
                 k=torch.zeros(B, T, HKV, D, dtype=bf, device=dev),
                 v=torch.zeros(B, T, HKV, D, dtype=bf, device=dev),
                 do=torch.zeros(B, T, H, D, dtype=bf, device=dev),
                 o=torch.zeros(B, T, H, D, dtype=bf, device=dev),
                 lse=torch.zeros(B, H, T, device=dev),
                 dvec=torch.zeros(B, H, T, device=dev))
        for name, fn in spoil.items():
            t[name] = fn(t[name])
        return t

    spoils = {
        "q fp32 with bf16 k/v": dict(q=lambda x: x.float()),
        "k fp32": dict(k=lambda x: x.float()),
        "v fp16": dict(v=lambda x: x.half()),
        "k non-contiguous": dict(k=lambda x: x.transpose(1, 2).contiguous().transpose(1, 2)),
        "v shape differs from k": dict(v=lambda x: x[:, :, :1].contiguous()),
        "do non-contiguous": dict(do=lambda x: x.transpose(1, 2).contiguous().transpose(1, 2)),
        "do fp32": dict(do=lambda x: x.float()),
        "o fp16": dict(o=lambda x: x.half()),
        "lse bf16": dict(lse=lambda x: x.bfloat16()),
        "lse short": dict(lse=lambda x: x[:, :, :-1].contiguous()),
        "dvec bf16": dict(dvec=lambda x: x.bfloat16()),
        "dvec short": dict(dvec=lambda x: x[:, :, :-1].contiguous()),
        "q on the host": dict(q=lambda x: x.cpu()),
        "lse on the host": dict(lse=lambda x: x.cpu()),
    }
    entries = {
        "bwd": lambda t: fa.flash_attn_bwd(t["q"], t["k"], t["v"], t["o"], t["lse"], t["do"]),
        "bwd_dkdv": lambda t: fa.flash_attn_bwd_dkdv(t["q"], t["k"], t["v"], t["do"], t["lse"],
                                                    t["dvec"]),
        "bwd_dq": lambda t: fa.flash_attn_bwd_dq(t["q"], t["k"], t["v"], t["do"], t["lse"],
                                                t["dvec"]),
        "bwd_dq_dvec": lambda t: fa.flash_attn_bwd_dq_dvec(t["q"], t["k"], t["v"], t["o"],
                                                          t["do"], t["lse"], dvec=t["dvec"]),
    }
    uses = {"bwd": {"q", "k", "v", "o", "lse", "do"},
            "bwd_dkdv": {"q", "k", "v", "do", "lse", "dvec"},
            "bwd_dq": {"q", "k", "v", "do", "lse", "dvec"},
            "bwd_dq_dvec": {"q", "k", "v", "o", "do", "lse", "dvec"}}
    out = []
    for ename, call in entries.items():
        for desc, sp in spoils.items():
            if set(sp) <= uses[ename]:
                out.append((ename, desc, sp, call, make))
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("case", _gpu_mismatches(), ids=lambda c: f"{c[0]}:{c[1]}")
def test_backward_mismatch_rejected_before_library(no_lib, case):
    ename, desc, spoil, call, make = case
    t = make(**spoil)
    with pytest.raises(ValueError):
        call(t)
