"""Guard bands around every output: each output view (O, LSE, Delta, dQ, dK, dV, the window
accumulators, the sink gradient) is carved out of a larger buffer whose every other element
holds a sentinel (a NaN payload for floats), on ragged shapes with padded strides. After the
calls, the sentinels must be untouched: no kernel writes outside the views it was given
(rows past the end, padding between rows and heads, the space before and after). The values
inside are checked against the oracle as well."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from flash_attention_train_amd import binding, configs
from flash_attention_train_amd.inputs import make_case
from parity_util import compare_full, host64, say, upload

pytestmark = pytest.mark.gpu

SENTINEL_F32 = 0x7FC0BEEF  # a quiet NaN with a payload no kernel produces
SENTINEL_BF16 = 0x7FCB


def _guarded(shape, dtype, pad_s=8, pad_h=3, margin=4096):
    """A view of `shape` ([B, H, S, D] or [B, H, S]) inside a sentinel-filled buffer: rows padded by
    pad_s elements (a multiple of 8, keeping 16-byte rows), pad_h spare rows per head, and
    `margin` spare elements before and after."""
    four = len(shape) == 4
    B, H, S = shape[:3]
    D = shape[3] if four else 1
    row = D + (pad_s if four else 0)
    head = (S + pad_h) * row
    n = margin + B * H * head + margin
    ints = torch.int32 if dtype == torch.float32 else torch.int16
    sent = SENTINEL_F32 if dtype == torch.float32 else SENTINEL_BF16
    if ints == torch.int16:
        sent = sent - (1 << 16) if sent >= (1 << 15) else sent
    buf = torch.full((n,), sent, dtype=ints, device="cuda").view(dtype)
    base = buf[margin:margin + B * H * head]
    if four:
        v = base.view(B, H, S + pad_h, row)[:, :, :S, :D]
    else:
        v = base.view(B, H, S + pad_h)[:, :, :S]
    return buf, v


def _inside_mask(buf, v):
    """Boolean host array over the buffer: True on the elements the view covers."""
    m = torch.zeros(buf.numel(), dtype=torch.bool)
    off = v.storage_offset() - buf.storage_offset()
    idx = torch.arange(v.numel()).view(v.shape)
    # element offsets of the view inside the buffer
    strides = v.stride()
    pos = torch.zeros(v.shape, dtype=torch.int64) + off
    for d, st in enumerate(strides):
        shape = [1] * v.dim()
        shape[d] = v.shape[d]
        pos = pos + (torch.arange(v.shape[d]) * st).view(shape)
    m[pos.reshape(-1)] = True
    del idx
    return m


def _check_band(name, buf, v):
    ints = torch.int32 if buf.dtype == torch.float32 else torch.int16
    raw = buf.view(ints).cpu()
    sent = SENTINEL_F32 if buf.dtype == torch.float32 else SENTINEL_BF16
    if ints == torch.int16:
        sent = sent - (1 << 16) if sent >= (1 << 15) else sent
    outside = ~_inside_mask(buf, v)
    bad = (raw[outside] != sent).sum().item()
    assert bad == 0, f"{name}: {bad} elements outside the view were written"
    assert (raw[~outside] != sent).all(), f"{name}: some elements inside the view were not written"


CASES = {
    "dit_sa_ragged_bf16": lambda: configs.make("dit_sa", Hq=4, Hkv=2, Sq=300, Sk=300),
    "dit_ca_masked_rows": lambda: configs.make("dit_ca", B=2, Hq=2, Hkv=2, Sq=130, Sk=96),
    "causal_gqa_offset": lambda: make_case("guard_causal", B=1, Hq=4, Hkv=1, Sq=77, Sk=141, D=128, dtype="bf16",
                                           seed=91, causal=True),
    "f32_d64": lambda: make_case("guard_f32", B=2, Hq=2, Hkv=1, Sq=70, Sk=90, D=64, dtype="f32", seed=92,
                                 mask="ca_keypad", mask_args={"lo": 10, "hi": 60, "masked_rows": 2}),
}


@pytest.mark.parametrize("splits", [(0, 0), (3, 2)])
@pytest.mark.parametrize("name", list(CASES))
def test_outputs_stay_inside_their_views(name, splits):
    c = CASES[name]()
    kv, qs = splits
    say(f"case {name}: guard bands, kv_split {kv} q_split {qs}")
    t = upload(c)
    dt = t["q"].dtype
    ob, o = _guarded(t["q"].shape, dt)
    lb, lse = _guarded(t["q"].shape[:3], torch.float32)
    db, delta = _guarded(t["q"].shape[:3], torch.float32)
    qb_, dq = _guarded(t["q"].shape, dt)
    kb_, dk = _guarded(t["k"].shape, dt)
    vb_, dv = _guarded(t["v"].shape, dt)
    binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal, q_offset=c.q_offset,
                out=o, lse=lse)
    binding.bwd_preprocess(o, t["do"], delta=delta)
    binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=t["mask"], scale=c.scale, causal=c.causal,
                q_offset=c.q_offset, dq=dq, dk=dk, dv=dv, kv_split=kv, q_split=qs)
    torch.cuda.synchronize()
    for n, b, v in (("O", ob, o), ("LSE", lb, lse), ("Delta", db, delta), ("dQ", qb_, dq), ("dK", kb_, dk),
                    ("dV", vb_, dv)):
        _check_band(n, b, v)
    m = None if c.mask is None else c.mask.astype(np.float64)
    ref = oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), m, scale=c.scale, causal=c.causal,
                          q_offset=c.q_offset)
    compare_full(c, {"O": host64(o), "LSE": host64(lse), "Delta": host64(delta), "dQ": host64(dq),
                     "dK": host64(dk), "dV": host64(dv)}, ref)


def test_window_accumulators_stay_inside_their_views():
    """The chunked walk adds into padded fp32 window accumulators: rows past the chunk's keys, the
    padding and the margins keep their sentinels, and the sink gradient's neighbours too."""
    W, C = 384, 128
    c = make_case("guard_window", B=1, Hq=4, Hkv=2, Sq=W, Sk=W, D=128, dtype="bf16", seed=93, causal=True)
    t = upload(c)
    kb_, dk_acc = _guarded(t["k"].shape, torch.float32)
    vb_, dv_acc = _guarded(t["k"].shape, torch.float32)
    dk_acc.zero_()
    dv_acc.zero_()
    for p0, n, sk in configs.chunk_plan(W, C):
        q, do = t["q"][:, :, p0:p0 + n], t["do"][:, :, p0:p0 + n]
        kk, vv = t["k"][:, :, :sk], t["v"][:, :, :sk]
        o, lse = binding.fwd(q, kk, vv, scale=c.scale, causal=True, q_offset=p0)
        delta = binding.bwd_preprocess(o, do)
        binding.bwd_chunked(q, kk, vv, do, lse, delta, dk_acc, dv_acc, scale=c.scale, causal=True, q_offset=p0,
                            kv_split=2, q_split=2)
    torch.cuda.synchronize()
    _check_band("dK_acc", kb_, dk_acc)
    _check_band("dV_acc", vb_, dv_acc)
    ref = oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), scale=c.scale, causal=True, q_offset=0)
    compare_full(c, {"dK": dk_acc.cpu().numpy().astype(np.float64), "dV": dv_acc.cpu().numpy().astype(np.float64)},
                 ref, names=("dK", "dV"))
    # the sink gradient is added into a 4-float slot between sentinels
    sinks = torch.linspace(-1.0, 1.0, c.Hq, device="cuda")
    sb = torch.full((c.Hq + 64,), SENTINEL_F32, dtype=torch.int32, device="cuda").view(torch.float32)
    dsink = sb[32:32 + c.Hq]
    dsink.zero_()
    o, lse = binding.fwd(t["q"], t["k"], t["v"], scale=c.scale, causal=True, q_offset=0, sinks=sinks)
    delta = binding.bwd_preprocess(o, t["do"])
    binding.bwd_sinks(lse, delta, sinks, dsink=dsink)
    torch.cuda.synchronize()
    raw = sb.view(torch.int32).cpu()
    assert (raw[:32] == SENTINEL_F32).all() and (raw[32 + c.Hq:] == SENTINEL_F32).all()
