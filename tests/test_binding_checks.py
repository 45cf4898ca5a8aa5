"""The Python binding's argument checks, on the host (no GPU): the C ABI receives bare
pointers and cannot see a tensor's size, dtype or residency, so the binding rejects a
mismatch before any launch. Every case below is wrong in exactly one way (tensors on
the CPU have the right shape unless the case is about shape), and the check must
raise before anything is launched: host tensors never reach a kernel."""
from __future__ import annotations

import os

import pytest
import torch

from flash_attention_train_amd import binding as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libfa_train.so not built")

Bn, Hq, Hkv, S, D = 1, 4, 2, 64, 64


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def _qkv(dtype=torch.bfloat16):
    return _t(Bn, Hq, S, D, dtype=dtype), _t(Bn, Hkv, S, D, dtype=dtype), _t(Bn, Hkv, S, D, dtype=dtype)


def _stats():
    return _t(Bn, Hq, S, dtype=torch.float32), _t(Bn, Hq, S, dtype=torch.float32)


def _fwd(**kw):
    q, k, v = _qkv()
    a = dict(q=q, k=k, v=v, out=_t(Bn, Hq, S, D), lse=_t(Bn, Hq, S, dtype=torch.float32))
    a.update(kw)
    return B.fwd(a.pop("q"), a.pop("k"), a.pop("v"), **a)


FWD_CASES = [
    ("k dtype differs from q", dict(k=_t(Bn, Hkv, S, D, dtype=torch.float32)), TypeError, "^k "),
    ("v shorter than k", dict(v=_t(Bn, Hkv, S - 1, D)), ValueError, "^v "),
    ("k head dim differs", dict(k=_t(Bn, Hkv, S, 2 * D), v=_t(Bn, Hkv, S, 2 * D)), ValueError, "^k "),
    ("out in fp32 with bf16 q", dict(out=_t(Bn, Hq, S, D, dtype=torch.float32)), TypeError, "^out "),
    ("out one row short", dict(out=_t(Bn, Hq, S - 1, D)), ValueError, "^out "),
    ("lse in bf16", dict(lse=_t(Bn, Hq, S)), TypeError, "^lse "),
    ("lse one row short", dict(lse=_t(Bn, Hq, S - 1, dtype=torch.float32)), ValueError, "^lse "),
    ("q is a host tensor", {}, ValueError, "device tensor"),
]


@pytest.mark.parametrize("name,kw,exc,match", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_fwd_rejects(name, kw, exc, match):
    with pytest.raises(exc, match=match):
        _fwd(**kw)


def _bwd(**kw):
    q, k, v = _qkv()
    lse, delta = _stats()
    a = dict(q=q, k=k, v=v, dout=_t(Bn, Hq, S, D), lse=lse, delta=delta, dq=_t(Bn, Hq, S, D),
             dk=_t(Bn, Hkv, S, D), dv=_t(Bn, Hkv, S, D))
    a.update(kw)
    return B.bwd(a.pop("q"), a.pop("k"), a.pop("v"), a.pop("dout"), a.pop("lse"), a.pop("delta"), **a)


BWD_CASES = [
    ("dout one row short", dict(dout=_t(Bn, Hq, S - 1, D)), ValueError, "^dout "),
    ("dout in fp32", dict(dout=_t(Bn, Hq, S, D, dtype=torch.float32)), TypeError, "^dout "),
    ("lse short", dict(lse=_t(Bn, Hq, S - 8, dtype=torch.float32)), ValueError, "^lse "),
    ("delta in bf16", dict(delta=_t(Bn, Hq, S)), TypeError, "^delta "),
    ("dq in fp32 with bf16 q", dict(dq=_t(Bn, Hq, S, D, dtype=torch.float32)), TypeError, "^dq "),
    ("dk one row short", dict(dk=_t(Bn, Hkv, S - 1, D)), ValueError, "^dk "),
    ("dv with Hq heads", dict(dv=_t(Bn, Hq, S, D)), ValueError, "^dv "),
    ("v shorter than k", dict(v=_t(Bn, Hkv, S - 1, D)), ValueError, "^v "),
    ("every operand on the host", {}, ValueError, "device tensor"),
]


@pytest.mark.parametrize("name,kw,exc,match", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_bwd_rejects(name, kw, exc, match):
    with pytest.raises(exc, match=match):
        _bwd(**kw)


def _chunked(**kw):
    q, k, v = _qkv()
    lse, delta = _stats()
    a = dict(q=q, k=k, v=v, dout=_t(Bn, Hq, S, D), lse=lse, delta=delta,
             dk_acc=_t(Bn, Hkv, 2 * S, D, dtype=torch.float32), dv_acc=_t(Bn, Hkv, 2 * S, D, dtype=torch.float32),
             dq=_t(Bn, Hq, S, D))
    a.update(kw)
    return B.bwd_chunked(a.pop("q"), a.pop("k"), a.pop("v"), a.pop("dout"), a.pop("lse"), a.pop("delta"),
                         a.pop("dk_acc"), a.pop("dv_acc"), **a)


CHUNKED_CASES = [
    ("dk_acc has fewer rows than the keys", dict(dk_acc=_t(Bn, Hkv, S - 1, D, dtype=torch.float32)), ValueError,
     "^dk_acc "),
    ("dv_acc with another head count", dict(dv_acc=_t(Bn, Hq, 2 * S, D, dtype=torch.float32)), ValueError,
     "^dv_acc "),
    ("dk_acc in bf16", dict(dk_acc=_t(Bn, Hkv, 2 * S, D)), TypeError, "accumulators"),
    ("dq one row short", dict(dq=_t(Bn, Hq, S - 1, D)), ValueError, "^dq "),
    ("lse short", dict(lse=_t(Bn, Hq, S - 1, dtype=torch.float32)), ValueError, "^lse "),
    ("every operand on the host", {}, ValueError, "device tensor"),
]


@pytest.mark.parametrize("name,kw,exc,match", CHUNKED_CASES, ids=[c[0] for c in CHUNKED_CASES])
def test_bwd_chunked_rejects(name, kw, exc, match):
    with pytest.raises(exc, match=match):
        _chunked(**kw)


def test_preprocess_rejects():
    o = _t(Bn, Hq, S, D)
    with pytest.raises(ValueError):
        B.bwd_preprocess(o, _t(Bn, Hq, S - 1, D))  # dout short
    with pytest.raises(TypeError):
        B.bwd_preprocess(o, _t(Bn, Hq, S, D, dtype=torch.float32))  # dout dtype
    with pytest.raises(ValueError):
        B.bwd_preprocess(o, _t(Bn, Hq, S, D), delta=_t(Bn, Hq, S - 1, dtype=torch.float32))  # delta short
    with pytest.raises(ValueError):
        B.bwd_preprocess(o, _t(Bn, Hq, S, D))  # host tensors


def test_sinks_rejects():
    lse, delta = _stats()
    sinks = _t(Hq, dtype=torch.float32)
    with pytest.raises(ValueError):
        B.bwd_sinks(lse, _t(Bn, Hq, S - 1, dtype=torch.float32), sinks)  # delta short
    with pytest.raises(ValueError):
        B.bwd_sinks(lse, delta, _t(Hq - 1, dtype=torch.float32))  # sinks short
    with pytest.raises(ValueError):
        B.bwd_sinks(lse, delta, sinks, dsink=_t(Hq - 1, dtype=torch.float32))  # accumulator short
    with pytest.raises(ValueError):
        B.bwd_sinks(lse, delta, sinks, dsink=_t(Hq, dtype=torch.float32))  # host tensors


def test_window_conversions_reject():
    qs = torch.zeros((Bn, Hkv, S, D), dtype=torch.int8)
    d = torch.zeros((Bn, Hkv, S, D // 32), dtype=torch.float16)
    with pytest.raises(ValueError):
        B.dequant_q8_0(qs, d, out=_t(Bn, Hkv, S - 1, D))  # out short
    with pytest.raises(TypeError):
        B.dequant_q8_0(qs, d, out=_t(Bn, Hkv, S, D, dtype=torch.float32))  # out dtype
    with pytest.raises(ValueError):
        B.dequant_q8_0(qs, d, out=_t(Bn, Hkv, S, D))  # host tensors
    src = torch.zeros((Bn, Hkv, S, D), dtype=torch.float16)
    with pytest.raises(ValueError):
        B.convert_f16(src, out=_t(Bn, Hkv, S, D - 8))  # out shape
    with pytest.raises(ValueError):
        B.convert_f16(src, out=_t(Bn, Hkv, S, D))  # host tensors


def test_structured_and_modifier_arrays_reject():
    q, k, v = _qkv()
    with pytest.raises(ValueError):
        _fwd(key_len=torch.zeros(Bn + 1, dtype=torch.int32))  # one length per batch entry
    with pytest.raises(ValueError):
        _fwd(alibi=torch.zeros(Hq - 1, dtype=torch.float32))
    with pytest.raises(ValueError):
        _fwd(mask=torch.zeros((1, S, S - 1), dtype=torch.float32))
