"""fa_train_bwd_noalloc, the backward for callers that cannot allocate: its workspace is
the library's static device scratch. Through the C ABI it must give fa_train_bwd's
results on two calls in a row, the second on a smaller problem (the scratch keeps the
first call's contents), in bf16 with split walks (fp32 slices in the scratch) and in
fp32 (the dQ accumulator in the scratch, which must start from zero on every call);
and a problem whose workspace exceeds the array is rejected before any launch."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from flash_attention_train_amd import binding, configs
from flash_attention_train_amd.inputs import make_case
from parity_util import compare_full, host64, say, upload

pytestmark = pytest.mark.gpu


def _pair(c, t, **kw):
    """fa_train_bwd with a caller workspace, then fa_train_bwd_noalloc, on the same inputs."""
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal,
                         q_offset=c.q_offset)
    delta = binding.bwd_preprocess(o, t["do"])
    ref = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=t["mask"], scale=c.scale, causal=c.causal,
                      q_offset=c.q_offset, **kw)
    got = binding.bwd_noalloc(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=t["mask"], scale=c.scale,
                              causal=c.causal, q_offset=c.q_offset, **kw)
    torch.cuda.synchronize()
    outs = {"O": host64(o), "LSE": host64(lse), "Delta": host64(delta)}
    return outs, ref, got


def _check(c, outs, ref, got, bitwise):
    m = None if c.mask is None else c.mask.astype(np.float64)
    want = oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), m, scale=c.scale, causal=c.causal,
                           q_offset=c.q_offset)
    res = dict(outs)
    res.update({"dQ": host64(got[0]), "dK": host64(got[1]), "dV": host64(got[2])})
    compare_full(c, res, want)
    for name, a, b in zip(("dQ", "dK", "dV"), ref, got):
        if bitwise:
            assert torch.equal(a, b), f"{name}: fa_train_bwd_noalloc differs from fa_train_bwd"
        else:  # fp32 dQ is summed with atomics: equal up to summation order
            e = (a.double() - b.double()).abs().max().item() / max(a.double().abs().max().item(), 1e-30)
            assert e <= 1e-5, (name, e)


def test_noalloc_matches_bwd_two_calls():
    # first call: DiT self-attention structure with split walks, so that fp32 slices live in the scratch
    c1 = configs.make("dit_sa", Hq=8, Hkv=4, Sq=700, Sk=700)
    say(f"noalloc call 1: B={c1.B} Hq={c1.Hq} Sq={c1.Sq} bf16, kv_split 2, q_split 2")
    t1 = upload(c1)
    split = dict(kv_split=2, q_split=2)
    p = binding.make_params(t1["q"], t1["k"], scale=c1.scale, causal=c1.causal, q_offset=c1.q_offset,
                            mask=t1["mask"], **split)
    need = int(binding.lib().fa_train_bwd_workspace_bytes(p))
    assert 0 < need <= binding.NOALLOC_SCRATCH_BYTES
    outs, ref, got = _pair(c1, t1, **split)
    _check(c1, outs, ref, got, bitwise=True)
    # second call: a smaller problem right after, same splits (the scratch still holds call 1's slices)
    c2 = make_case("noalloc_small", B=1, Hq=4, Hkv=2, Sq=300, Sk=260, D=128, dtype="bf16", seed=91, causal=True,
                   q_offset=-40)
    say(f"noalloc call 2: B={c2.B} Hq={c2.Hq} Sq={c2.Sq} Sk={c2.Sk} bf16 causal, kv_split 2, q_split 2")
    t2 = upload(c2)
    outs, ref, got = _pair(c2, t2, **split)
    _check(c2, outs, ref, got, bitwise=True)


def test_noalloc_fp32_accumulator_starts_at_zero():
    # fp32: the dQ accumulator lives in the scratch; the second call must not see the first's sums
    c1 = make_case("noalloc_f32_a", B=1, Hq=4, Hkv=2, Sq=200, Sk=180, D=64, dtype="f32", seed=92, mask="ca_keypad",
                   mask_args={"lo": 40, "hi": 170, "masked_rows": 2})
    c2 = make_case("noalloc_f32_b", B=1, Hq=2, Hkv=1, Sq=90, Sk=70, D=64, dtype="f32", seed=93, causal=True)
    for c in (c1, c2):
        say(f"noalloc fp32 call: B={c.B} Hq={c.Hq} Sq={c.Sq} Sk={c.Sk}")
        t = upload(c)
        outs, ref, got = _pair(c, t)
        _check(c, outs, ref, got, bitwise=False)


def test_noalloc_rejects_beyond_the_scratch():
    # a split whose fp32 slices exceed the static array: rejected on the host, outputs untouched
    c = configs.make("lm_causal", Hq=32, Hkv=8, Sq=4096, Sk=4096)
    t = upload(c)
    lse = torch.zeros(c.B, c.Hq, c.Sq, dtype=torch.float32, device="cuda")
    delta = torch.zeros_like(lse)
    dq = torch.full_like(t["q"], 7.0)
    with pytest.raises(binding.FaError) as e:
        binding.bwd_noalloc(t["q"], t["k"], t["v"], t["do"], lse, delta, scale=c.scale, causal=True, q_offset=0,
                            dq=dq, kv_split=8, q_split=8)
    assert e.value.status == 8  # FA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((dq == 7.0).all())
