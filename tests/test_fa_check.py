"""The checked build (libfa_train_check.so, -DFA_CHECK) on the host, no GPU: its checker
enumerates every workgroup the bf16 forward and backward would launch for a problem, with the
kernels' own unit decoding, ranges and LDS offsets, and verifies that every staged row, LDS
offset, stored row and workspace slice stays inside its buffer and that the units cover every
output row exactly once (once per split). Swept over the workloads at full size, their shrunk
and ragged forms, GQA, causal offsets, every split hint, both dK/dV walks, structured lengths
and windows, and the 64 chunks of the long-window walk."""
from __future__ import annotations

import ctypes
import os

import pytest

from flash_attention_train_amd import binding as B
from flash_attention_train_amd import build

pytestmark = pytest.mark.skipif(not os.path.exists(build.CHECK_LIB), reason="libfa_train_check.so not built")

_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build.CHECK_LIB)
        _lib.fa_train_check_launch.argtypes = [ctypes.POINTER(B.FaAttnParams), ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_char_p, ctypes.c_size_t]
        _lib.fa_train_check_launch.restype = ctypes.c_int
    return _lib


def params(**kw):
    a = dict(B=1, Hq=4, Hkv=2, Sq=64, Sk=64, D=128, dtype=B.FA_BF16, causal=0, q_offset=0, scale=0.125, mask=None,
             mask_stride_b=0, mask_stride_q=0, mask_tiles=None, fwd_variant=0, kv_split=0, q_split=0, fwd_split=0,
             key_len=None, q_len=None, window_left=-1, window_right=-1, bwd_dq_launch=0, sinks=None, alibi=None,
             q_split_tiles=0, mask_stride_h=0, softcap=0.0, bwd_kv_walk=0, kv_format=0, k_scale=B.FaView(),
             v_scale=B.FaView(), dbias=None, dbias_stride_b=0, dbias_stride_h=0, dbias_stride_q=0)
    a.update(kw)
    if a["causal"] and "q_offset" not in kw:
        a["q_offset"] = a["Sk"] - a["Sq"]
    return B.FaAttnParams(*(a[f] for f, _ in B.FaAttnParams._fields_))


def check(p, key_len=None, q_len=None):
    rep = ctypes.create_string_buffer(256)
    kl = (ctypes.c_int32 * len(key_len))(*key_len) if key_len else None
    ql = (ctypes.c_int32 * len(q_len))(*q_len) if q_len else None
    st = lib().fa_train_check_launch(ctypes.byref(p), kl, ql, rep, len(rep))
    return st, rep.value.decode()


SHAPES = {
    "dit_sa": dict(B=1, Hq=16, Hkv=8, Sq=1542, Sk=1542),
    "dit_ca": dict(B=2, Hq=16, Hkv=16, Sq=1542, Sk=512),
    "lm_causal": dict(B=1, Hq=32, Hkv=8, Sq=4096, Sk=4096, causal=1),
    "ragged_gqa4": dict(B=2, Hq=4, Hkv=1, Sq=333, Sk=201),
    "causal_offset": dict(B=1, Hq=4, Hkv=2, Sq=100, Sk=356, causal=1, q_offset=256),
    "causal_before_keys": dict(B=1, Hq=2, Hkv=2, Sq=80, Sk=40, causal=1, q_offset=-40),
    "one_one": dict(B=1, Hq=2, Hkv=1, Sq=1, Sk=1),
    "d64": dict(B=2, Hq=4, Hkv=4, Sq=200, Sk=129, D=64),
}
SPLITS = [dict(), dict(kv_split=2, q_split=2, q_split_tiles=6), dict(kv_split=3, q_split=5),
          dict(kv_split=1, q_split=4, q_split_tiles=1), dict(fwd_split=7), dict(bwd_kv_walk=2, kv_split=2),
          dict(bwd_dq_launch=3), dict(bwd_dq_launch=3, kv_split=2, q_split=3, q_split_tiles=3)]


@pytest.mark.parametrize("split", range(len(SPLITS)))
@pytest.mark.parametrize("name", list(SHAPES))
def test_launch_index_space(name, split):
    st, rep = check(params(**SHAPES[name], **SPLITS[split]))
    assert st == 0, rep


@pytest.mark.parametrize("dq_launch", [0, 3])
@pytest.mark.parametrize("window", [(-1, -1), (256, 256), (0, 0), (100, -1)])
def test_structured_lengths_and_windows(window, dq_launch):
    p = params(B=2, Hq=16, Hkv=8, Sq=1542, Sk=1542, window_left=window[0], window_right=window[1],
               bwd_dq_launch=dq_launch)
    for kl, ql in (([1388, 1388], None), ([1542, 1101], [1542, 700]), ([0, 1], [5, 0])):
        st, rep = check(p, key_len=kl, q_len=ql)
        assert st == 0, (kl, ql, rep)


@pytest.mark.parametrize("dq_launch", [0, 3])
def test_long_window_chunks(dq_launch):
    W, C = 32768, 512
    for c in range(W // C):
        p0 = c * C
        st, rep = check(params(B=1, Hq=16, Hkv=4, Sq=C, Sk=p0 + C, causal=1, q_offset=p0, bwd_dq_launch=dq_launch))
        assert st == 0, (c, rep)


def test_fp32_is_not_covered():
    assert check(params(dtype=B.FA_F32))[0] == 7
