"""The C ABI on the host, no GPU: the library loads, exports every symbol the
headers declare, and rejects bad arguments before any launch. Pointers here are
fake addresses; every call below is invalid in exactly one way, so validation
returns before anything touches a device."""
from __future__ import annotations

import ctypes
import glob
import os
import re

import pytest

from flash_attention_train_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libfa_train.so not built")


def declared_functions():
    """Functions declared by the op's headers (the checked build's own header is separate)."""
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        if os.path.basename(h) == "fa_train_check.h":
            continue
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(fa_train_\w+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported_and_bound():
    L = B.lib()
    names = declared_functions()
    assert "fa_train_fwd" in names and "fa_train_bwd_chunked" in names
    for n in names:
        assert hasattr(L, n), n
        assert n in B.SIGNATURES, f"{n} has no ctypes signature in the binding"
    assert L.fa_train_version() == 14


BASE = 0x7F0000000000  # fake, 256-byte aligned device addresses


def params(**kw):
    a = dict(B=1, Hq=4, Hkv=2, Sq=64, Sk=64, D=64, dtype=B.FA_BF16, causal=0, q_offset=0, scale=0.125, mask=None,
             mask_stride_b=0, mask_stride_q=0, mask_tiles=None, fwd_variant=0, kv_split=0, q_split=0, fwd_split=0, key_len=None, q_len=None,
             window_left=-1, window_right=-1, bwd_dq_launch=0, sinks=None, alibi=None,
             q_split_tiles=0, mask_stride_h=0, softcap=0.0, bwd_kv_walk=0, kv_format=0, k_scale=B.FaView(),
             v_scale=B.FaView(), dbias=None, dbias_stride_b=0, dbias_stride_h=0, dbias_stride_q=0)
    a.update(kw)
    return B.FaAttnParams(*(a[f] for f, _ in B.FaAttnParams._fields_))


def view(i, H=4, S=64, D=64, elt=2, **kw):
    a = dict(data=BASE + i * (1 << 24), stride_b=H * S * D, stride_h=S * D, stride_s=D)
    a.update(kw)
    return B.FaView(a["data"], a["stride_b"], a["stride_h"], a["stride_s"])


def lse_view(i, H=4, S=64):
    return B.FaView(BASE + i * (1 << 24), H * S, S, 1)


def fwd_call(p, q=None, k=None, v=None, o=None, lse=None):
    q = q or view(0)
    k = k or view(1, H=2)
    v = v or view(2, H=2)
    o = o or view(3)
    lse = lse or lse_view(4)
    return B.lib().fa_train_fwd(ctypes.byref(p) if p is not None else None, q, k, v, o, lse, None)


FWD_ERRORS = [
    ("null params", None, {}, 1),
    ("Hq not a multiple of Hkv", params(Hq=3), {}, 2),
    ("zero length", params(Sq=0), {}, 2),
    ("bad dtype", params(dtype=7), {}, 3),
    ("head dim 96", params(D=96), {}, 7),
    ("misaligned q", params(), {"q": view(0, data=BASE + 8)}, 5),
    ("stride not 16B", params(), {"k": view(1, H=2, stride_s=68)}, 5),
    ("o rows overlap", params(), {"o": view(3, stride_s=32)}, 4),
    ("o aliases q", params(), {"o": view(0)}, 6),
    ("lse aliases o", params(), {"lse": B.FaView(BASE + 3 * (1 << 24), 256, 64, 1)}, 6),
    ("lse not contiguous", params(), {"lse": B.FaView(BASE + 4 * (1 << 24), 512, 128, 2)}, 4),
    ("null data", params(), {"v": view(2, H=2, data=0)}, 1),
    ("causal flag 2", params(causal=2), {}, 2),
    ("negative scale", params(scale=-0.5), {}, 2),
    ("unknown forward variant", params(fwd_variant=9), {}, 2),
    ("split out of range", params(kv_split=65), {}, 2),
    ("window bound -2", params(window_left=-2), {}, 2),
    ("unknown dQ launch hint", params(bwd_dq_launch=5), {}, 2),
    ("negative q_split_tiles", params(q_split_tiles=-1), {}, 2),
    ("per-head mask with a block map", params(mask=BASE + 9 * (1 << 24), mask_stride_q=64, mask_stride_h=64 * 64,
                                              mask_tiles=BASE + 10 * (1 << 24)), {}, 7),
    ("misaligned sinks", params(sinks=BASE + 2), {}, 5),
    ("misaligned alibi", params(alibi=BASE + 2), {}, 5),
    ("misaligned key_len", params(key_len=BASE + 2), {}, 5),
    ("mask stride too small", params(mask=BASE + 9 * (1 << 24), mask_stride_q=32), {}, 4),
    ("row stride 2^24", params(), {"k": view(1, H=2, stride_s=1 << 24, stride_h=(1 << 24) * 64,
                                                stride_b=(1 << 24) * 128)}, 4),
]


@pytest.mark.parametrize("name,p,over,code", FWD_ERRORS, ids=[e[0] for e in FWD_ERRORS])
def test_forward_rejects(name, p, over, code):
    st = fwd_call(p, **over)
    assert st == code, (st, B.lib().fa_train_last_error())
    assert B.lib().fa_train_last_error() != b""
    assert B.lib().fa_train_status_str(st) not in (b"", b"ok")


def test_split_forward_workspace_and_rejects():
    L = B.lib()
    # splits x B x Hq x Sq x (2 D + 8) bytes: the bf16 partial rows plus their fp32 base and row sum
    p2 = params(Sk=640, fwd_split=2)
    assert L.fa_train_fwd_workspace_bytes(ctypes.byref(p2)) == 2 * 1 * 4 * 64 * (2 * 64 + 8)
    # automatic: 4 query-tile workgroups, 64 key tiles -> 5 splits (each at least 12 tiles)
    assert L.fa_train_fwd_workspace_bytes(ctypes.byref(params(Sk=4096))) == 5 * 1 * 4 * 64 * (2 * 64 + 8)
    assert L.fa_train_fwd_workspace_bytes(ctypes.byref(params())) == 0  # one key tile: nothing to split
    assert L.fa_train_fwd_workspace_bytes(ctypes.byref(params(Sk=640, fwd_split=1))) == 0
    assert L.fa_train_fwd_workspace_bytes(None) == ctypes.c_size_t(-1).value
    assert L.fa_train_fwd_workspace_bytes(ctypes.byref(params(fwd_split=65))) == ctypes.c_size_t(-1).value
    kk, vv = view(1, H=2, S=640), view(2, H=2, S=640)
    need = 2 * 1 * 4 * 64 * (2 * 64 + 8)
    ws = BASE + 12 * (1 << 24)

    def fws(p, ws=ws, nbytes=need, **over):
        v = {"q": view(0), "k": kk, "v": vv, "o": view(3), "lse": lse_view(4)}
        v.update(over)
        return L.fa_train_fwd_ws(ctypes.byref(p), v["q"], v["k"], v["v"], v["o"], v["lse"], ws, nbytes, None)

    assert fwd_call(p2, k=kk, v=vv) == 8  # the plain forward never splits
    assert fws(p2, ws=None) == 8
    assert fws(p2, nbytes=need - 1) == 8
    assert fws(p2, ws=ws + 64) == 5
    assert fws(p2, ws=BASE) == 6  # workspace over Q
    assert fws(params(Sk=640, fwd_split=65)) == 2


def bwd_call(p, accumulate=False, ws=None, ws_bytes=None, **over):
    L = B.lib()
    v = {"q": view(0), "k": view(1, H=2), "v": view(2, H=2), "do": view(3), "lse": lse_view(4), "delta": lse_view(5),
         "dq": view(6), "dk": view(7, H=2, elt=4 if accumulate else 2), "dv": view(8, H=2)}
    v.update(over)
    need = L.fa_train_bwd_workspace_bytes(ctypes.byref(p))
    ws = BASE + 12 * (1 << 24) if ws is None else ws
    ws_bytes = need if ws_bytes is None else ws_bytes
    f = L.fa_train_bwd_chunked if accumulate else L.fa_train_bwd
    return f(ctypes.byref(p), v["q"], v["k"], v["v"], v["do"], v["lse"], v["delta"], v["dq"], v["dk"], v["dv"], ws,
             ws_bytes, None)


def test_backward_rejects():
    # split walks keep one fp32 slice per split: dQ slices [q_split][B, Hq, Sq, D], dK and
    # dV slices [kv_split][B, Hkv, Sk, D] each
    p = params(q_split=2, kv_split=1)
    assert B.lib().fa_train_bwd_workspace_bytes(ctypes.byref(p)) == 2 * (1 * 4 * 64 * 64 * 4)
    assert B.lib().fa_train_bwd_workspace_bytes(ctypes.byref(params(q_split=1, kv_split=1))) == 0
    assert B.lib().fa_train_bwd_workspace_bytes(ctypes.byref(params(q_split=1, kv_split=2))) == 2 * 2 * (2 * 64 * 64 * 4)
    # a split tail keeps full-length dQ slices (only the split tiles' rows are written and summed)
    assert B.lib().fa_train_bwd_workspace_bytes(ctypes.byref(params(q_split=2, kv_split=1, q_split_tiles=1))) == \
        B.lib().fa_train_bwd_workspace_bytes(ctypes.byref(params(q_split=2, kv_split=1)))
    # dQ from stored dS: 16 KB per (batch entry, query head, 64-row tile, 128-key tile) after the
    # slices; ignored (the dQ walk, no dS) for a stored K/V window, a mask gradient or the role walk
    ds = 1 * 4 * 1 * 1 * 16384
    assert B.lib().fa_train_bwd_workspace_bytes(ctypes.byref(params(q_split=1, kv_split=1, bwd_dq_launch=3))) == ds
    assert B.lib().fa_train_bwd_workspace_bytes(ctypes.byref(params(q_split=2, kv_split=1, bwd_dq_launch=3))) == \
        2 * (1 * 4 * 64 * 64 * 4) + ds
    big = params(B=2, Hq=4, Sq=300, Sk=260, q_split=1, kv_split=1, bwd_dq_launch=3)
    assert B.lib().fa_train_bwd_workspace_bytes(ctypes.byref(big)) == 2 * 4 * 5 * 3 * 16384
    assert B.lib().fa_train_bwd_workspace_bytes(ctypes.byref(params(q_split=1, kv_split=1, bwd_dq_launch=3,
                                                                    bwd_kv_walk=2))) == 0
    # the automatic choice takes stored dS from 512 128-row tiles on, while dS fits 2 GB
    lm = params(Hq=32, Hkv=8, Sq=4096, Sk=4096, causal=1, q_split=1, kv_split=1)
    assert B.lib().fa_train_bwd_workspace_bytes(ctypes.byref(lm)) == 32 * 64 * 32 * 16384
    long = params(Hq=32, Hkv=8, Sq=32768, Sk=32768, causal=1, q_split=1, kv_split=1)
    assert B.lib().fa_train_bwd_workspace_bytes(ctypes.byref(long)) == 0
    long.bwd_dq_launch = 3
    assert B.lib().fa_train_bwd_workspace_bytes(ctypes.byref(long)) == 32 * 512 * 256 * 16384
    assert bwd_call(p, ws=0) == 8
    assert bwd_call(p, ws_bytes=100) == 8
    assert bwd_call(p, ws=BASE + 12 * (1 << 24) + 16) == 5
    assert bwd_call(p, dq=view(0)) == 6          # dQ over Q
    assert bwd_call(p, dk=view(8, H=2)) == 6     # dK over dV
    assert bwd_call(p, dv=view(4, H=2)) == 6  # dV over the LSE input
    assert bwd_call(p, ws=BASE + 4 * (1 << 24)) == 6  # workspace over LSE
    assert bwd_call(p, dk=view(7, H=2, stride_h=0)) == 4  # dK heads collapse onto each other
    assert bwd_call(params(Hkv=3)) == 2
    assert bwd_call(p, accumulate=True, dk=view(7, H=2, data=BASE + 7 * (1 << 24) + 4)) == 5
    assert B.lib().fa_train_bwd_workspace_bytes(None) == ctypes.c_size_t(-1).value


def test_preprocess_rejects():
    L = B.lib()
    p = params()
    assert L.fa_train_bwd_preprocess(ctypes.byref(p), view(0), view(1), B.FaView(BASE + 0 * (1 << 24), 256, 64, 1),
                                     None) == 6
    assert L.fa_train_bwd_preprocess(ctypes.byref(params(D=32)), view(0), view(1), lse_view(2), None) == 7
    assert L.fa_train_bwd_preprocess(None, view(0), view(1), lse_view(2), None) == 1


def test_mask_tiles_host_checks():
    L = B.lib()
    assert L.fa_train_mask_tiles_bytes(ctypes.byref(params())) == 0  # no mask
    m = params(Sq=130, Sk=70, mask=BASE + 9 * (1 << 24), mask_stride_q=72, mask_stride_b=0)
    assert L.fa_train_mask_tiles_bytes(ctypes.byref(m)) == 256 + 2 * (3 * 2) * 64 * 8
    mb = params(B=2, Sq=130, Sk=70, mask=BASE + 9 * (1 << 24), mask_stride_q=72, mask_stride_b=130 * 72)
    assert L.fa_train_mask_tiles_bytes(ctypes.byref(mb)) == 256 + 2 * (2 * 3 * 2) * 64 * 8
    assert L.fa_train_mask_tiles(ctypes.byref(params()), BASE, None) == 1
    assert L.fa_train_mask_tiles(ctypes.byref(m), None, None) == 1
    assert L.fa_train_mask_tiles(ctypes.byref(m), BASE + 9 * (1 << 24) + 64, None) == 6
    assert L.fa_train_mask_tiles(ctypes.byref(m), BASE + 3, None) == 5


def test_probe_rejects_bad_arguments():
    L = B.lib()
    assert L.fa_train_probe_mfma(9, 1, BASE, BASE, BASE, None) == 2
    assert L.fa_train_probe_mfma(0, 0, BASE, BASE, BASE, None) == 2
    assert L.fa_train_probe_mfma(0, 1, None, BASE, BASE, None) == 1
    assert L.fa_train_probe_ds_read_tr16(0, BASE, BASE, None) == 2


def test_window_conversions_reject():
    L = B.lib()
    # f16 -> fp32 / bf16
    assert L.fa_train_convert_f16(1, 4, 64, 64, view(0), view(0), B.FA_F32, None) == 6  # out overlaps src
    assert L.fa_train_convert_f16(1, 4, 64, 64, view(0), view(2, elt=4), 2, None) == 3
    assert L.fa_train_convert_f16(1, 4, 64, 96, view(0, D=96), view(2, D=96), B.FA_BF16, None) == 7
    assert L.fa_train_convert_f16(0, 4, 64, 64, view(0), view(2), B.FA_BF16, None) == 2
    assert L.fa_train_convert_f16(1, 4, 64, 64, None, view(2), B.FA_BF16, None) == 1
    assert L.fa_train_convert_f16(1, 4, 64, 64, view(0, stride_s=68), view(2), B.FA_BF16, None) == 5
    assert L.fa_train_convert_f16(1, 4, 64, 64, view(0), view(2, stride_s=32), B.FA_BF16, None) == 4
    # q8_0 -> bf16: quants [1, 4, 64, 64] int8, scales [1, 4, 64, 2] fp16
    qs = B.FaView(BASE, 4 * 64 * 64, 64 * 64, 64)
    d = B.FaView(BASE + (1 << 24), 4 * 64 * 2, 64 * 2, 2)
    assert L.fa_train_dequant_q8_0(1, 4, 64, 64, qs, B.FaView(BASE + (1 << 24), 4 * 64, 64, 1), view(2), None) == 4
    assert L.fa_train_dequant_q8_0(1, 4, 64, 64, qs, d, view(0), None) == 6  # out overlaps qs
    assert L.fa_train_dequant_q8_0(1, 4, 64, 48, qs, d, view(2), None) == 7


def test_softcap_params_rejected():
    L = B.lib()
    lse, dlt = lse_view(5), lse_view(6)
    bad = [(dict(softcap=-1.0), 2), (dict(softcap=float("inf")), 2), (dict(softcap=float("nan")), 2)]
    for kw, code in bad:
        p = params(**kw)
        assert L.fa_train_fwd(ctypes.byref(p), view(0), view(1, H=2), view(2, H=2), view(3), lse, None) == code, kw
        assert L.fa_train_bwd(ctypes.byref(p), view(0), view(1, H=2), view(2, H=2), view(3), lse, dlt, view(8),
                              view(9, H=2), view(10, H=2), None, 0, None) == code, kw
    # a softcap backward keeps the bf16 matrix-core kernels' plan also under a dense mask or ALiBi
    # (no workspace for this unsplit shape); fp32 runs on the generic kernels, whose workspace is
    # the fp32 dQ accumulator; the bf16 forward keeps its split walks
    masked = dict(softcap=30.0, mask=BASE + 11 * (1 << 24), mask_stride_q=64)
    slopes = dict(softcap=30.0, alibi=BASE + 11 * (1 << 24))
    for kw in (masked, slopes):
        assert L.fa_train_bwd_workspace_bytes(ctypes.byref(params(dtype=B.FA_BF16, kv_split=1, q_split=1, **kw))) == 0
        assert L.fa_train_bwd_workspace_bytes(ctypes.byref(params(dtype=B.FA_F32, **kw))) == 1 * 4 * 64 * 64 * 4
    assert L.fa_train_bwd_workspace_bytes(ctypes.byref(params(softcap=30.0, kv_split=1, q_split=1))) == \
        L.fa_train_bwd_workspace_bytes(ctypes.byref(params(kv_split=1, q_split=1))) == 0
    # (the automatic split of this small non-causal grid: dK/dV walks two ways, fp32 dK and dV slices)
    assert L.fa_train_bwd_workspace_bytes(ctypes.byref(params())) == 2 * 2 * (1 * 2 * 64 * 64 * 4)
    long_keys = dict(softcap=30.0, Sk=4096)
    assert L.fa_train_fwd_workspace_bytes(ctypes.byref(params(**long_keys))) == \
        L.fa_train_fwd_workspace_bytes(ctypes.byref(params(Sk=4096))) > 0
    assert L.fa_train_fwd_workspace_bytes(ctypes.byref(params(dtype=B.FA_F32, **long_keys))) == 0


def test_backward_noalloc_rejects_before_any_launch():
    """fa_train_bwd_noalloc runs fa_train_bwd's checks, and rejects a problem whose workspace
    exceeds its static scratch, all on the host before it looks up the scratch or launches."""
    L = B.lib()
    far = 1 << 34  # fake regions far enough apart for LM-sized views

    def v(i, H, S, D=128):
        return view(0, H=H, S=S, D=D, data=BASE + i * far)

    def call(p, **over):
        a = {"q": v(0, 32, 4096), "k": v(1, 8, 4096), "v": v(2, 8, 4096), "do": v(3, 32, 4096),
             "lse": B.FaView(BASE + 4 * far, 32 * 4096, 4096, 1), "delta": B.FaView(BASE + 5 * far, 32 * 4096, 4096, 1),
             "dq": v(6, 32, 4096), "dk": v(7, 8, 4096), "dv": v(8, 8, 4096)}
        a.update(over)
        return L.fa_train_bwd_noalloc(ctypes.byref(p) if p is not None else None, a["q"], a["k"], a["v"], a["do"],
                                      a["lse"], a["delta"], a["dq"], a["dk"], a["dv"], None)

    lm = dict(Hq=32, Hkv=8, Sq=4096, Sk=4096, D=128, causal=1)
    big = params(kv_split=8, q_split=8, **lm)
    assert L.fa_train_bwd_workspace_bytes(ctypes.byref(big)) > B.NOALLOC_SCRATCH_BYTES
    assert call(big) == 8, B.lib().fa_train_last_error()
    assert b"scratch" in B.lib().fa_train_last_error()
    assert call(None) == 1
    assert call(params(Hkv=3, **{k: x for k, x in lm.items() if k != "Hkv"})) == 2
    assert call(params(kv_split=2, **lm), dq=v(0, 32, 4096)) == 6  # dQ over Q


def test_kv_walk_hint_range():
    assert fwd_call(params(bwd_kv_walk=3)) == 2
    assert fwd_call(params(bwd_kv_walk=-1)) == 2


def test_stored_kv_formats_rejected_where_unsupported():
    """K / V stored as fp16 or q8_0: bf16 problems only, no dense mask, ALiBi or softcap; q8_0 needs
    its fp16 scale planes, [B, Hkv, Sk, D / 32] with rows covering their D / 32 scales."""
    def kv8(i):  # int8 quants [1, 2, 64, 64]
        return view(i, H=2, elt=1)

    def scales(i, **kw):
        a = dict(data=BASE + i * (1 << 24), stride_b=2 * 64 * 2, stride_h=64 * 2, stride_s=2)
        a.update(kw)
        return B.FaView(a["data"], a["stride_b"], a["stride_h"], a["stride_s"])

    q8 = dict(kv_format=2, k_scale=scales(10), v_scale=scales(11), kv_split=1, q_split=1)  # (unsplit: no workspace)
    assert fwd_call(params(kv_format=3)) == 3
    assert fwd_call(params(dtype=B.FA_F32, kv_format=1)) == 7
    assert fwd_call(params(kv_format=1, mask=BASE + 9 * (1 << 24), mask_stride_q=64)) == 7
    assert fwd_call(params(kv_format=1, alibi=BASE + 9 * (1 << 24))) == 7
    assert fwd_call(params(kv_format=1, softcap=30.0)) == 7
    assert fwd_call(params(kv_format=2), k=kv8(1), v=kv8(2)) == 1  # no scale planes
    assert fwd_call(params(kv_format=2, k_scale=scales(10, stride_s=1), v_scale=scales(11)), k=kv8(1), v=kv8(2)) == 4
    assert fwd_call(params(kv_format=2, k_scale=scales(10, data=BASE + 10 * (1 << 24) + 1), v_scale=scales(11)),
                    k=kv8(1), v=kv8(2)) == 5
    assert fwd_call(params(kv_format=2, k_scale=scales(3), v_scale=scales(11)), k=kv8(1), v=kv8(2)) == 6  # over O
    p = params(**q8)
    assert B.lib().fa_train_bwd(ctypes.byref(p), view(0), kv8(1), kv8(2), view(3), lse_view(4), lse_view(5),
                                view(6), view(7, H=2), view(11, H=2), None, 0, None) == 6  # dV over v_scale


def test_mask_gradient_params_rejected():
    """dbias (the mask's gradient) needs a dense mask, fp32-aligned rows of at least Sk entries, the
    mask's broadcast over batch and heads, no overlap with the inputs, and no softcap in bf16; all
    checked before any launch."""
    L = B.lib()
    lse, dlt = lse_view(5), lse_view(6)
    m = dict(mask=BASE + 11 * (1 << 24), mask_stride_q=64)
    db = dict(dbias=BASE + 12 * (1 << 24), dbias_stride_q=64)
    bad = [(dict(**db), 2),                                         # no mask
           (dict(**m, **db, softcap=30.0), 7),                      # bf16 softcap
           (dict(**m, dbias=BASE + 12 * (1 << 24), dbias_stride_q=32), 4),  # rows shorter than Sk
           (dict(**m, **db, dbias_stride_h=64 * 64), 4),            # per-head gradient of a shared mask
           (dict(**m, mask_stride_h=64 * 64, **db), 4),             # shared gradient of a per-head mask
           (dict(**m, dbias=BASE + 12 * (1 << 24) + 2, dbias_stride_q=64), 5),  # misaligned
           (dict(**m, dbias=BASE + 11 * (1 << 24), dbias_stride_q=64), 6)]      # the mask itself
    for kw, code in bad:
        p = params(kv_split=1, q_split=1, **kw)  # (unsplit: no workspace)
        got = L.fa_train_bwd(ctypes.byref(p), view(0), view(1, H=2), view(2, H=2), view(3), lse, dlt, view(8),
                             view(9, H=2), view(10, H=2), None, 0, None)
        assert got == code, (kw, got)
    # accepted on the host: fp32 with a softcap, and a per-head gradient of a per-head mask (the
    # problem stops at the missing workspace of the fp32 path, after every other check)
    ok = [dict(**m, **db, dtype=B.FA_F32, softcap=30.0),
          dict(**m, mask_stride_h=64 * 64, dbias=BASE + 12 * (1 << 24), dbias_stride_h=64 * 64, dbias_stride_q=64,
               dtype=B.FA_F32)]
    for kw in ok:
        p = params(**kw)
        got = L.fa_train_bwd(ctypes.byref(p), view(0, elt=4), view(1, H=2), view(2, H=2), view(3), lse, dlt,
                             view(8), view(9, H=2), view(10, H=2), None, 0, None)
        assert got == 8, (kw, got)  # FA_ERR_WORKSPACE
