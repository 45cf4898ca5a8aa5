"""GPU parity of the logit softcap (score (b, h, i, j) = c tanh(scale <q_i, k_j> / c) + the
mask value) against the oracle, in fp32 and bf16: every output element by element, with the
exact-zero checks for fully masked rows and dead key columns. The bf16 forward and backward run
the cap in their MFMA kernels (every work decomposition; under a dense mask the backward caps a
whole block before adding the mask values); fp32 runs on the generic kernels. Cases: the causal GQA layer, a
dense key-padding mask with fully masked rows, a score bias per head, and the chunked walk
over a window (each chunk adding into the fp32 dK / dV accumulators). The caps are small
enough (1 to 4 score units) that tanh is well inside its bend for N(0, 1) inputs."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from flash_attention_train_amd import binding, configs
from flash_attention_train_amd.inputs import BF16, F32, make_case
from parity_util import compare_full, host64, say, upload
from test_gpu_head_bias import _case as head_bias_case, compare as head_bias_compare

pytestmark = pytest.mark.gpu


def _case(name, dtype):
    if name == "lm_causal_gqa4":
        return make_case(name, B=1, Hq=8, Hkv=2, Sq=300, Sk=300, D=128, dtype=dtype, seed=131, causal=True), 1.0
    if name == "ca_keypad_rows_d64":
        return make_case(name, B=2, Hq=4, Hkv=4, Sq=200, Sk=150, D=64, dtype=dtype, seed=132, mask="ca_keypad",
                         mask_args={"lo": 40, "hi": 150, "masked_rows": 2}), 2.0
    if name == "plain_d64":  # no mask, not causal, ragged tiles
        return make_case(name, B=2, Hq=4, Hkv=2, Sq=190, Sk=250, D=64, dtype=dtype, seed=135), 2.0
    if name == "head_bias":  # [B, Hq, Sq, Sk] biases with rows and key columns hidden per head
        return head_bias_case(name, B=2, Hq=4, Hkv=2, Sq=130, Sk=190, D=128, dtype=dtype, seed=133), 4.0
    raise KeyError(name)


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("name", ["lm_causal_gqa4", "plain_d64", "ca_keypad_rows_d64", "head_bias"])
@pytest.mark.parametrize("split", [0, 3])
def test_softcap_parity(name, dtype, split):
    c, cap = _case(name, dtype)
    say(f"case {name} ({dtype}): softcap {cap}, forward split {split}")
    bias = c.meta.get("bias")
    m = bias if bias is not None else c.mask
    ref = oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), None if m is None else m.astype(np.float64),
                          scale=c.scale, causal=c.causal, q_offset=c.q_offset, softcap=cap)
    t = upload(c)
    if bias is not None:
        t["mask"] = torch.from_numpy(bias).cuda()
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal,
                         q_offset=c.q_offset, softcap=cap, split=split)
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=t["mask"], scale=c.scale,
                             causal=c.causal, q_offset=c.q_offset, softcap=cap)
    torch.cuda.synchronize()
    got = {"O": host64(o), "LSE": host64(lse), "Delta": host64(delta), "dQ": host64(dq), "dK": host64(dk),
           "dV": host64(dv)}
    if bias is not None:
        head_bias_compare(c, got, ref)
    else:
        compare_full(c, got, ref)


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_softcap_chunked_window(dtype):
    W, C, cap = 512, 128, 1.5
    c = configs.make("long_window", W=W, Hq=4, Hkv=1, D=64, dtype=dtype)
    say(f"softcap chunked walk ({dtype}): W={W}, chunks of {C}, softcap {cap}")
    t = upload(c)
    dk_acc = torch.zeros((1, c.Hkv, W, c.D), dtype=torch.float32, device="cuda")
    dv_acc = torch.zeros_like(dk_acc)
    O, dQ = torch.empty_like(t["q"]), torch.empty_like(t["q"])
    LSE = torch.empty((1, c.Hq, W), dtype=torch.float32, device="cuda")
    Delta = torch.empty_like(LSE)
    for p0, n, sk in configs.chunk_plan(W, C):
        q, do = t["q"][:, :, p0:p0 + n], t["do"][:, :, p0:p0 + n]
        kk, vv = t["k"][:, :, :sk], t["v"][:, :, :sk]
        o, lse = binding.fwd(q, kk, vv, scale=c.scale, causal=True, q_offset=p0, out=O[:, :, p0:p0 + n],
                             lse=LSE[:, :, p0:p0 + n], softcap=cap)
        delta = binding.bwd_preprocess(o, do, delta=Delta[:, :, p0:p0 + n])
        binding.bwd_chunked(q, kk, vv, do, lse, delta, dk_acc, dv_acc, scale=c.scale, causal=True, q_offset=p0,
                            dq=dQ[:, :, p0:p0 + n], softcap=cap)
    torch.cuda.synchronize()
    ref = oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), scale=c.scale, causal=True, q_offset=0,
                          softcap=cap)
    got = {"O": host64(O), "LSE": host64(LSE), "Delta": host64(Delta), "dQ": host64(dQ),
           "dK": dk_acc.cpu().numpy().astype(np.float64), "dV": dv_acc.cpu().numpy().astype(np.float64)}
    compare_full(c, got, ref)


@pytest.mark.parametrize("variant", [2, 3])
def test_softcap_forward_variants(variant):
    """The other configurations of the bf16 forward kernel (64 rows per wave with 32-key tiles;
    keys split over two halves of the workgroup) apply the cap the same way."""
    c, cap = _case("ca_keypad_rows_d64", BF16)
    say(f"case ca_keypad_rows_d64 (bf16): softcap {cap}, forward variant {variant}")
    ref = oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), c.mask.astype(np.float64), scale=c.scale,
                          causal=c.causal, q_offset=c.q_offset, softcap=cap)
    t = upload(c)
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal,
                         q_offset=c.q_offset, softcap=cap, split=1, variant=variant)
    torch.cuda.synchronize()
    compare_full(c, {"O": host64(o), "LSE": host64(lse)}, ref, names=("O", "LSE"))


@pytest.mark.parametrize("kv_split,q_split,q_split_tiles,dq_launch", [(1, 1, 0, 1), (2, 1, 0, 2), (3, 2, 0, 1),
                                                                      (2, 2, 1, 1), (1, 3, 2, 2)])
@pytest.mark.parametrize("name", ["lm_causal_gqa4", "plain_d64"])
def test_softcap_backward_decompositions(name, kv_split, q_split, q_split_tiles, dq_launch):
    """The capped bf16 backward in the MFMA kernels: split dK/dV and dQ walks (with their reduce
    passes), the split tail, and the dQ walk in the shared or its own launch."""
    c, cap = _case(name, BF16)
    say(f"case {name} (bf16): softcap {cap}, splits {kv_split}x{q_split}x{q_split_tiles}, dq launch {dq_launch}")
    ref = oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), scale=c.scale, causal=c.causal,
                          q_offset=c.q_offset, softcap=cap)
    t = upload(c)
    o, lse = binding.fwd(t["q"], t["k"], t["v"], scale=c.scale, causal=c.causal, q_offset=c.q_offset, softcap=cap)
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, scale=c.scale, causal=c.causal,
                             q_offset=c.q_offset, softcap=cap, kv_split=kv_split, q_split=q_split,
                             q_split_tiles=q_split_tiles, dq_launch=dq_launch)
    torch.cuda.synchronize()
    got = {"O": host64(o), "LSE": host64(lse), "Delta": host64(delta), "dQ": host64(dq), "dK": host64(dk),
           "dV": host64(dv)}
    compare_full(c, got, ref)


def test_softcap_with_sinks_and_structured_masks():
    """Without a dense mask the cap combines with attention sinks and with structured masks (key
    lengths, a sliding window): the capped MFMA kernels, against the oracle with the same sinks and
    the structured mask written out densely."""
    from flash_attention_train_amd.inputs import sink_logits
    c = make_case("sinks_band", B=2, Hq=4, Hkv=2, Sq=200, Sk=200, D=128, dtype=BF16, seed=136)
    cap, sinks = 2.0, sink_logits(137, 4)
    key_len, window = [200, 160], (48, 48)  # every row keeps a visible key; keys past 160 are dead
    say(f"case sinks_band (bf16): softcap {cap}, sinks {sinks}, key lengths {key_len}, window {window}")
    dense = oracle.structured_mask(c.B, c.Sq, c.Sk, key_len=key_len, window_left=window[0], window_right=window[1])
    ref = oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), dense, scale=c.scale, softcap=cap,
                          sinks=sinks.astype(np.float64))
    t = upload(c)
    kl = torch.tensor(key_len, dtype=torch.int32, device="cuda")
    sk = torch.from_numpy(sinks).cuda()
    o, lse = binding.fwd(t["q"], t["k"], t["v"], scale=c.scale, softcap=cap, sinks=sk, key_len=kl, window=window)
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, scale=c.scale, softcap=cap, key_len=kl,
                             window=window)
    dsink = binding.bwd_sinks(lse, delta, sk)
    torch.cuda.synchronize()
    c.mask = dense.astype(np.float32)  # the dense form, for the exact-zero checks
    got = {"O": host64(o), "LSE": host64(lse), "Delta": host64(delta), "dQ": host64(dq), "dK": host64(dk),
           "dV": host64(dv)}
    compare_full(c, got, ref)
    # the sink gradient: a sum of terms of both signs, measured against the sum of their sizes
    terms = np.exp(sinks.astype(np.float64)[None, :, None] - ref["LSE"]) * np.abs(ref["Delta"])
    err = np.abs(dsink.cpu().numpy() - ref["dSink"]) / terms.sum(axis=(0, 2))
    say(f"  dSink error against sum |terms|: {err.max():.2e}")
    assert err.max() <= 2e-2
