"""GPU parity of K/V windows read in place (llama.cpp pull request 57: a q8_0 cache trains in
place; an f16 cache too, its backward casting each tile it reads): the window stays in its
stored format (fp16 values, or q8_0 int8 quants with an fp16 scale per 32 values) and every
kernel that reads a K or V tile converts it to bf16 on the way, so no bf16 copy of the window
exists. The conversion is the same as the conversion entry points' (fp16 widened exactly,
the q8_0 product exact in fp32, one rounding to nearest even), so:

* the exact walk over a stored window, each chunk forward -> preprocess -> chunked backward,
  equals the one-shot oracle run on the window's stored values (fp16, or d * q), within the
  bf16 tolerance, fully masked rows and dead columns exactly zero;
* it gives the same bits as the same walk over a bf16 copy made by the conversion entry
  points (same values, same kernels, same summation order);
* a plain forward / backward over a stored K/V (D = 64 and 128, GQA, causal or not, a key
  length) matches the oracle, and the library rejects the combinations it does not take.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from flash_attention_train_amd import binding, configs
from flash_attention_train_amd.inputs import make_case, quantize_q8_0
from parity_util import compare_full, host64, say, upload

pytestmark = pytest.mark.gpu


def _stored(c, fmt):
    """The case's K/V as a stored window on the device, the oracle's view of its values, and
    the keyword arguments of the calls."""
    k, v = c.f64("k").astype(np.float32), c.f64("v").astype(np.float32)
    if fmt == "f16":
        k16, v16 = k.astype(np.float16), v.astype(np.float16)
        dev = {"k": torch.from_numpy(k16).cuda(), "v": torch.from_numpy(v16).cuda()}
        ref = {"k": k16.astype(np.float64), "v": v16.astype(np.float64)}
        return dev, ref, {}
    (kq, kd), (vq, vd) = quantize_q8_0(k), quantize_q8_0(v)
    dev = {"k": torch.from_numpy(kq).cuda(), "v": torch.from_numpy(vq).cuda()}
    kw = {"k_scale": torch.from_numpy(kd).cuda(), "v_scale": torch.from_numpy(vd).cuda()}
    ref = {"k": oracle.dequant_q8_0(kq, kd), "v": oracle.dequant_q8_0(vq, vd)}
    return dev, ref, kw


def _walk(c, t, k, v, W, C, kw, dq_launch=0):
    dk_acc = torch.zeros((1, c.Hkv, W, c.D), dtype=torch.float32, device="cuda")
    dv_acc = torch.zeros_like(dk_acc)
    O, dQ = torch.empty_like(t["q"]), torch.empty_like(t["q"])
    LSE = torch.empty((1, c.Hq, W), dtype=torch.float32, device="cuda")
    Delta = torch.empty_like(LSE)
    for p0, n, sk in configs.chunk_plan(W, C):
        q, do = t["q"][:, :, p0:p0 + n], t["do"][:, :, p0:p0 + n]
        skw = {name: x[:, :, :sk] for name, x in kw.items()}
        o, lse = binding.fwd(q, k[:, :, :sk], v[:, :, :sk], scale=c.scale, causal=True, q_offset=p0,
                             out=O[:, :, p0:p0 + n], lse=LSE[:, :, p0:p0 + n], **skw)
        delta = binding.bwd_preprocess(o, do, delta=Delta[:, :, p0:p0 + n])
        binding.bwd_chunked(q, k[:, :, :sk], v[:, :, :sk], do, lse, delta, dk_acc, dv_acc, scale=c.scale,
                            causal=True, q_offset=p0, dq=dQ[:, :, p0:p0 + n], dq_launch=dq_launch, **skw)
    torch.cuda.synchronize()
    return {"O": O, "LSE": LSE, "Delta": Delta, "dQ": dQ, "dK": dk_acc, "dV": dv_acc}


@pytest.mark.parametrize("dq_launch", [1, 2])
@pytest.mark.parametrize("fmt", ["f16", "q8_0"])
def test_window_walk_in_place(fmt, dq_launch):
    W, C = 1024, 256
    c = configs.make("long_window", W=W, Hq=4, Hkv=1)
    say(f"{fmt} window read in place: W={W}, chunks of {C}, Hq={c.Hq} Hkv={c.Hkv}, dq_launch {dq_launch}")
    t = upload(c)
    dev, ref_kv, kw = _stored(c, fmt)
    got = _walk(c, t, dev["k"], dev["v"], W, C, kw, dq_launch)
    ref = oracle.backward(c.f64("q"), ref_kv["k"], ref_kv["v"], c.f64("do"), scale=c.scale, causal=True, q_offset=0)
    compare_full(c, {n: host64(x) for n, x in got.items()}, ref)
    # the conversion-pass walk over a bf16 copy of the same window: the same bits
    if fmt == "f16":
        kb, vb = binding.convert_f16(dev["k"]), binding.convert_f16(dev["v"])
    else:
        kb, vb = binding.dequant_q8_0(dev["k"], kw["k_scale"]), binding.dequant_q8_0(dev["v"], kw["v_scale"])
    copy = _walk(c, t, kb, vb, W, C, {}, dq_launch)
    for n in got:
        assert torch.equal(got[n], copy[n]), f"{n}: in-place walk differs from the walk over the bf16 copy"


CASES = {
    "gqa_causal_d128": dict(B=1, Hq=4, Hkv=2, Sq=300, Sk=300, D=128, causal=True),
    "noncausal_d64_ragged": dict(B=2, Hq=2, Hkv=1, Sq=130, Sk=200, D=64, causal=False),
    "chunk_offset": dict(B=1, Hq=4, Hkv=2, Sq=100, Sk=356, D=128, causal=True, q_offset=256),
}


@pytest.mark.parametrize("fmt", ["f16", "q8_0"])
@pytest.mark.parametrize("name", list(CASES))
def test_fwd_bwd_in_place(name, fmt):
    c = make_case(f"in_place_{name}", dtype="bf16", seed=81, **CASES[name])
    say(f"case {name}: {fmt} K/V read in place")
    t = upload(c)
    dev, ref_kv, kw = _stored(c, fmt)
    kl = None
    if name == "noncausal_d64_ragged":  # with a structured key length too
        kl = torch.tensor([150, 200], dtype=torch.int32, device="cuda")
    o, lse = binding.fwd(t["q"], dev["k"], dev["v"], scale=c.scale, causal=c.causal, q_offset=c.q_offset,
                         key_len=kl, **kw)
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], dev["k"], dev["v"], t["do"], lse, delta, scale=c.scale, causal=c.causal,
                             q_offset=c.q_offset, key_len=kl, **kw)
    torch.cuda.synchronize()
    m = None
    if kl is not None:
        m = oracle.structured_mask(c.B, c.Sq, c.Sk, key_len=[150, 200])
        c.mask = m.astype(np.float32)  # for the exact-zero checks of dead key columns
    ref = oracle.backward(c.f64("q"), ref_kv["k"], ref_kv["v"], c.f64("do"), m, scale=c.scale, causal=c.causal,
                          q_offset=c.q_offset)
    got = {"O": host64(o), "LSE": host64(lse), "Delta": host64(delta), "dQ": host64(dq), "dK": host64(dk),
           "dV": host64(dv)}
    compare_full(c, got, ref)


def test_in_place_rejections():
    """Stored formats take bf16 problems without a dense mask, ALiBi or softcap; q8_0 needs its scales."""
    c = make_case("in_place_reject", B=1, Hq=2, Hkv=1, Sq=64, Sk=64, D=64, dtype="bf16", seed=82)
    t = upload(c)
    dev, _, kw = _stored(c, "q8_0")
    with pytest.raises(ValueError):  # quants without scales
        binding.fwd(t["q"], dev["k"], dev["v"], scale=c.scale)
    mask = torch.zeros((1, 64, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(binding.FaError) as e:
        binding.fwd(t["q"], dev["k"], dev["v"], scale=c.scale, mask=mask, **kw)
    assert e.value.status == 7
    with pytest.raises(binding.FaError) as e:
        binding.fwd(t["q"], dev["k"], dev["v"], scale=c.scale, softcap=20.0, **kw)
    assert e.value.status == 7
    f16 = {n: x.float().half() for n, x in (("k", t["k"]), ("v", t["v"]))}
    with pytest.raises(TypeError):  # an fp32 problem takes no stored format
        binding.fwd(t["q"].float(), f16["k"], f16["v"], scale=c.scale)
