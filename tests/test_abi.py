"""The C-ABI library without a GPU: it loads, exports what include/xfa.h
declares, and rejects bad arguments before making any GPU call."""

import ctypes
import math
import os
import re

import pytest

import transformer_attention_xfa_amd as xfa

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "xfa.h")

OK, INVAL, UNSUP = xfa.XFA_OK, xfa.XFA_ERR_INVALID_ARGUMENT, xfa.XFA_ERR_UNSUPPORTED
A = 0x10000  # a 16-byte-aligned non-null address; never dereferenced by these calls


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(xfa_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert names == sorted(["xfa_fwd", "xfa_bwd_preprocess", "xfa_bwd", "xfa_bwd_workspace_bytes",
                            "xfa_fwd_dropout", "xfa_bwd_dropout", "xfa_status_string"])
    lib = ctypes.CDLL(xfa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in (OK, INVAL, UNSUP, xfa.XFA_ERR_HIP):
        assert xfa.xfa_status_string(s).startswith("xfa: ")
    assert "unknown" in xfa.xfa_status_string(99)


def _fwd(**kw):
    a = dict(q=A, k=A, v=A, out=A, lse=A, B=1, H=2, S=64, hd=64, scale=0.125, causal=1, dtype=1)
    a.update(kw)
    return xfa.lib().xfa_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["S"],
                             a["hd"], a["scale"], a["causal"], a["dtype"], None)


def _pre(**kw):
    a = dict(out=A, dout=A, delta=A, B=1, H=2, S=64, hd=64, scale=0.125, causal=1, dtype=1)
    a.update(kw)
    return xfa.lib().xfa_bwd_preprocess(a["out"], a["dout"], a["delta"], a["B"], a["H"], a["S"],
                                        a["hd"], a["scale"], a["causal"], a["dtype"], None)


def _bwd(**kw):
    a = dict(q=A, k=A, v=A, dout=A, lse=A, delta=A, dq=A, dk=A, dv=A,
             B=1, H=2, S=64, hd=64, scale=0.125, causal=1, dtype=1)
    a.update(kw)
    return xfa.lib().xfa_bwd(a["q"], a["k"], a["v"], a["dout"], a["lse"], a["delta"], a["dq"],
                             a["dk"], a["dv"], a.get("ws"), a["B"], a["H"], a["S"], a["hd"], a["scale"],
                             a["causal"], a["dtype"], None)


def _fwd_drop(**kw):
    a = dict(q=A, k=A, v=A, out=A, lse=A, B=1, H=2, S=64, hd=64, scale=0.125, causal=1, p=0.1, seed=7, dtype=1)
    a.update(kw)
    return xfa.lib().xfa_fwd_dropout(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["S"],
                                     a["hd"], a["scale"], a["causal"], a["p"], a["seed"], a["dtype"], None)


def _bwd_drop(**kw):
    a = dict(q=A, k=A, v=A, dout=A, lse=A, delta=A, dq=A, dk=A, dv=A,
             B=1, H=2, S=64, hd=64, scale=0.125, causal=1, p=0.1, seed=7, dtype=1)
    a.update(kw)
    return xfa.lib().xfa_bwd_dropout(a["q"], a["k"], a["v"], a["dout"], a["lse"], a["delta"], a["dq"],
                                     a["dk"], a["dv"], a.get("ws"), a["B"], a["H"], a["S"], a["hd"],
                                     a["scale"], a["causal"], a["p"], a["seed"], a["dtype"], None)


@pytest.mark.parametrize("call", [_fwd, _pre, _bwd, _fwd_drop, _bwd_drop])
def test_rejects_bad_arguments(call):
    assert call(dtype=2) == INVAL
    assert call(dtype=-1) == INVAL
    assert call(B=-1) == INVAL
    assert call(S=-5) == INVAL
    assert call(hd=0) == INVAL
    assert call(hd=48) == UNSUP
    assert call(hd=256) == UNSUP
    assert call(scale=0.0) == INVAL
    assert call(scale=-1.0) == INVAL
    assert call(scale=math.nan) == INVAL
    assert call(scale=math.inf) == INVAL
    assert call(causal=2) == INVAL
    assert call(S=(1 << 30) + 1) == UNSUP
    assert call(B=1 << 40, H=1 << 30) == UNSUP


@pytest.mark.parametrize("call,ptrs", [
    (_fwd, ["q", "k", "v", "out", "lse"]),
    (_pre, ["out", "dout", "delta"]),
    (_bwd, ["q", "k", "v", "dout", "lse", "delta", "dq", "dk", "dv"]),
    (_fwd_drop, ["q", "k", "v", "out", "lse"]),
    (_bwd_drop, ["q", "k", "v", "dout", "lse", "delta", "dq", "dk", "dv"]),
])
def test_rejects_null_and_misaligned_pointers(call, ptrs):
    for p in ptrs:
        assert call(**{p: None}) == INVAL, p
        assert call(**{p: A + 8}) == INVAL, p


def test_size_limits():
    # S * hd * 4 bytes (one head at fp32 width) must fit a signed 32-bit offset,
    # whatever the dtype; accepted sizes are not tried here (they would launch)
    for dtype in (0, 1):
        assert _fwd(S=1 << 22, hd=128, dtype=dtype) == UNSUP
        assert _pre(S=1 << 22, hd=128, dtype=dtype) == UNSUP
        assert _bwd(S=1 << 22, hd=128, dtype=dtype) == UNSUP
        assert _bwd(S=1 << 23, hd=64, dtype=dtype) == UNSUP
        # the staging past the end counts too: S*hd*4 < 2^31 but (S+256)*hd*4 is not
        assert _fwd(S=(1 << 22) - 200, hd=128, dtype=dtype) == UNSUP
        assert _fwd_drop(S=(1 << 22) - 200, hd=128, dtype=dtype) == UNSUP
        assert _bwd(S=(1 << 22) - 200, hd=128, dtype=dtype) == UNSUP
        # one 1-D dispatch per kernel: B * H * ceil(S / 128) workgroups of 256
        # work-items must stay below 2^24 (the work-item count is 32-bit)
        for call in (_fwd, _pre, _bwd, _fwd_drop, _bwd_drop):
            assert call(B=2, H=1 << 13, S=1 << 17, hd=16, dtype=dtype) == UNSUP
            assert call(B=1, H=1 << 14, S=(1 << 17) - 127, hd=16, dtype=dtype) == UNSUP


@pytest.mark.parametrize("call", [_fwd_drop, _bwd_drop])
def test_dropout_rejects_bad_probability(call):
    # p must lie in [0, 1); p = 1 would drop everything and divide by zero
    for p in (-0.1, -1e-30, 1.0, 1.5, math.nan, math.inf, -math.inf):
        assert call(p=p) == INVAL, p
    # the probability is checked before the pointers: nothing valid is needed
    assert call(p=1.0, q=None) == INVAL
    # any 64-bit seed is accepted (an empty problem returns before launching)
    for seed in (0, 1, (1 << 64) - 1, 0x9E3779B97F4A7C15):
        assert call(seed=seed, S=0) == OK


@pytest.mark.parametrize("call", [_fwd, _pre, _bwd, _fwd_drop, _bwd_drop])
def test_empty_problem_is_a_no_op(call):
    # nothing to do: succeeds without touching (null) pointers or the GPU
    nulls = {"fwd": ["q", "k", "v", "out", "lse"], "pre": ["out", "dout", "delta"],
             "bwd": ["q", "k", "v", "dout", "lse", "delta", "dq", "dk", "dv"]}
    nulls["fwd_drop"], nulls["bwd_drop"] = nulls["fwd"], nulls["bwd"]
    key = call.__name__[1:]
    args = {p: None for p in nulls[key]}
    assert call(S=0, **args) == OK
    assert call(B=0, **args) == OK
    assert call(H=0, **args) == OK


def test_op_rejects_host_tensors():
    # no CPU fallback: the op refuses tensors that are not on the GPU
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 8, 16)
    with pytest.raises(ValueError, match="GPU"):
        xfa.flash_attention(q, q, q)


def test_flash_attention_rejects_unknown_core():
    import torch
    import transformer_attention_xfa_amd as xfa
    t = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ValueError):
        xfa.flash_attention(t, t, t, core="fp16")
    assert xfa.CORES == ("native", "fp32")


@pytest.mark.parametrize("p", [-0.5, 1.0, 2.0])
def test_flash_attention_rejects_bad_dropout_probability(p):
    import torch
    t = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ValueError, match="dropout_p"):
        xfa.flash_attention(t, t, t, dropout_p=p)


@pytest.mark.parametrize("dtype", [0, 1])
@pytest.mark.parametrize("B,H,S,hd", [(1, 1, 64, 16), (8, 16, 4096, 128), (1, 32, 16384, 128), (2, 3, 1, 64),
                                      (0, 4, 100, 32)])
def test_workspace_bytes_is_zero(B, H, S, hd, dtype):
    # the shipped backward forms dQ in its own query-outer kernel: no
    # workspace for any shape, so NULL is a valid workspace argument
    assert xfa.lib().xfa_bwd_workspace_bytes(B, H, S, hd, dtype) == 0
    assert xfa.xfa_bwd_workspace_bytes(B, H, S, hd, dtype) == 0


def test_workspace_pointer_is_not_checked_when_size_is_zero():
    # with no workspace needed, NULL and any other value pass the checks
    # (an empty problem returns before any GPU call)
    assert _bwd(ws=None, S=0) == OK
    assert _bwd(ws=A, S=0) == OK
    assert _bwd_drop(ws=None, S=0) == OK
    assert _bwd(ws=None, hd=48) == UNSUP
