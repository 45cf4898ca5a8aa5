"""GPU parity of the q8_0 K/V window (llama.cpp pull request 57 trains a q8_0 cache in
place): the dequantisation kernel bit for bit against the oracle's values rounded to bf16
(the fp32 product of an fp16 scale and an int8 quant is exact, so the one rounding is the
bf16 store), and the exact walk over a q8_0 window -- each chunk converting the window rows
it adds, then forward, preprocess and the chunked backward -- against the one-shot oracle
run on the exactly dequantised window."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from flash_attention_train_amd import binding, configs
from flash_attention_train_amd.inputs import f32_to_bf16_bits, quantize_q8_0
from parity_util import compare_full, host64, say, upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D", [64, 128])
def test_dequant_q8_0_bit_exact(D):
    rng = np.random.default_rng(40 + D)
    x = (3.0 * rng.standard_normal((2, 3, 77, D))).astype(np.float32)
    x[0, 1, 5, :32] = 0.0  # an all-zero block (scale 0)
    qs, d = quantize_q8_0(x)
    want = f32_to_bf16_bits(oracle.dequant_q8_0(qs, d).astype(np.float32))
    tq, td = torch.from_numpy(qs).cuda(), torch.from_numpy(d).cuda()
    out = binding.dequant_q8_0(tq, td)
    # a strided destination: rows 10 .. 59 into the middle of a wider window buffer
    win = torch.full((2, 3, 120, D), 7.0, dtype=torch.bfloat16, device="cuda")
    binding.dequant_q8_0(tq[:, :, 10:60], td[:, :, 10:60], out=win[:, :, 30:80])
    torch.cuda.synchronize()
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    w = win.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(w[:, :, 30:80], want[:, :, 10:60])
    seven = f32_to_bf16_bits(np.float32(7.0))
    assert np.all(w[:, :, :30] == seven) and np.all(w[:, :, 80:] == seven)  # nothing outside the view


def test_q8_0_window_walk():
    W, C = 1024, 256
    c = configs.make("long_window_q8", W=W, Hq=4, Hkv=1)
    say(f"q8_0 window walk: W={W}, chunks of {C}, Hq={c.Hq} Hkv={c.Hkv}")
    t = upload(c)
    (kq, kd), (vq, vd) = c.meta["q8"]["k"], c.meta["q8"]["v"]
    kq, kd, vq, vd = (torch.from_numpy(a).cuda() for a in (kq, kd, vq, vd))
    k = torch.zeros_like(t["k"])
    v = torch.zeros_like(t["v"])
    dk_acc = torch.zeros((1, c.Hkv, W, c.D), dtype=torch.float32, device="cuda")
    dv_acc = torch.zeros_like(dk_acc)
    O, dQ = torch.empty_like(t["q"]), torch.empty_like(t["q"])
    LSE = torch.empty((1, c.Hq, W), dtype=torch.float32, device="cuda")
    Delta = torch.empty_like(LSE)
    for p0, n, sk in configs.chunk_plan(W, C):
        binding.dequant_q8_0(kq[:, :, p0:sk], kd[:, :, p0:sk], out=k[:, :, p0:sk])
        binding.dequant_q8_0(vq[:, :, p0:sk], vd[:, :, p0:sk], out=v[:, :, p0:sk])
        q, do = t["q"][:, :, p0:p0 + n], t["do"][:, :, p0:p0 + n]
        o, lse = binding.fwd(q, k[:, :, :sk], v[:, :, :sk], scale=c.scale, causal=True, q_offset=p0,
                             out=O[:, :, p0:p0 + n], lse=LSE[:, :, p0:p0 + n])
        delta = binding.bwd_preprocess(o, do, delta=Delta[:, :, p0:p0 + n])
        binding.bwd_chunked(q, k[:, :, :sk], v[:, :, :sk], do, lse, delta, dk_acc, dv_acc, scale=c.scale,
                            causal=True, q_offset=p0, dq=dQ[:, :, p0:p0 + n])
    torch.cuda.synchronize()
    kv = {n: oracle.dequant_q8_0(*c.meta["q8"][n]) for n in ("k", "v")}
    ref = oracle.backward(c.f64("q"), kv["k"], kv["v"], c.f64("do"), scale=c.scale, causal=True, q_offset=0)
    got = {"O": host64(O), "LSE": host64(LSE), "Delta": host64(Delta), "dQ": host64(dQ),
           "dK": dk_acc.cpu().numpy().astype(np.float64), "dV": dv_acc.cpu().numpy().astype(np.float64)}
    compare_full(c, got, ref)
