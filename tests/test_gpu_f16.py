"""GPU parity of the f16 K/V window (llama.cpp pull request 57 trains an f16 cache in place,
casting each tile to F32 in its backward): the conversion kernel bit for bit -- exact into
fp32, nearest-even into bf16 -- and the exact walk over an f16 window, each chunk converting
the window rows it adds, then forward, preprocess and the chunked backward, against the
one-shot oracle run on the window's fp16 values. The fp32 walk is the pages' own arithmetic
(fp16 values cast to F32) and meets the fp32 tolerance; the bf16 walk rounds the window
once more, to bf16, and meets the bf16 one."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from flash_attention_train_amd import binding, configs
from flash_attention_train_amd.inputs import BF16, F32, f32_to_bf16_bits
from parity_util import compare_full, host64, say, upload

pytestmark = pytest.mark.gpu


def _specials(D):
    """fp16 values that stress the conversion: signed zeros, the smallest and largest
    subnormals, the smallest normal, the largest finite value, infinities, values halfway
    between two bf16 values (ties to even both ways)."""
    bits = [0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x0400, 0x7BFF, 0xFBFF, 0x7C00, 0xFC00,
            0x3C04, 0x3C0C, 0x3C02, 0xBC06, 0x3BFF, 0x0155]
    x = np.zeros(D, np.uint16)
    x[:len(bits)] = bits
    return x.view(np.float16)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_convert_f16_bit_exact(D, dtype):
    rng = np.random.default_rng(50 + D)
    x = (3.0 * rng.standard_normal((2, 3, 77, D))).astype(np.float16)
    x[1, 2, 9] = _specials(D)
    f = x.astype(np.float32)  # exact
    if dtype == torch.float32:
        want = f.view(np.uint32)
    else:
        want = f32_to_bf16_bits(f)
    tx = torch.from_numpy(x).cuda()
    out = binding.convert_f16(tx, dtype=dtype)
    # a strided destination: rows 10 .. 59 into the middle of a wider window buffer
    win = torch.full((2, 3, 120, D), 7.0, dtype=dtype, device="cuda")
    binding.convert_f16(tx[:, :, 10:60], out=win[:, :, 30:80])
    torch.cuda.synchronize()
    ints = torch.int32 if dtype == torch.float32 else torch.int16
    u = np.uint32 if dtype == torch.float32 else np.uint16
    got = out.cpu().view(ints).numpy().view(u)
    assert np.array_equal(got, want)
    w = win.cpu().view(ints).numpy().view(u)
    assert np.array_equal(w[:, :, 30:80], want[:, :, 10:60])
    seven = np.float32(7.0).view(np.uint32) if dtype == torch.float32 else f32_to_bf16_bits(np.float32(7.0))
    assert np.all(w[:, :, :30] == seven) and np.all(w[:, :, 80:] == seven)  # nothing outside the view


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_f16_window_walk(dtype):
    W, C = 1024, 256
    c = configs.make("long_window_f16", W=W, Hq=4, Hkv=1, dtype=dtype)
    say(f"f16 window walk ({dtype}): W={W}, chunks of {C}, Hq={c.Hq} Hkv={c.Hkv}")
    t = upload(c)
    k16, v16 = (torch.from_numpy(c.meta["f16"][n]).cuda() for n in ("k", "v"))
    k = torch.zeros_like(t["k"])
    v = torch.zeros_like(t["v"])
    dk_acc = torch.zeros((1, c.Hkv, W, c.D), dtype=torch.float32, device="cuda")
    dv_acc = torch.zeros_like(dk_acc)
    O, dQ = torch.empty_like(t["q"]), torch.empty_like(t["q"])
    LSE = torch.empty((1, c.Hq, W), dtype=torch.float32, device="cuda")
    Delta = torch.empty_like(LSE)
    for p0, n, sk in configs.chunk_plan(W, C):
        binding.convert_f16(k16[:, :, p0:sk], out=k[:, :, p0:sk])
        binding.convert_f16(v16[:, :, p0:sk], out=v[:, :, p0:sk])
        q, do = t["q"][:, :, p0:p0 + n], t["do"][:, :, p0:p0 + n]
        o, lse = binding.fwd(q, k[:, :, :sk], v[:, :, :sk], scale=c.scale, causal=True, q_offset=p0,
                             out=O[:, :, p0:p0 + n], lse=LSE[:, :, p0:p0 + n])
        delta = binding.bwd_preprocess(o, do, delta=Delta[:, :, p0:p0 + n])
        binding.bwd_chunked(q, k[:, :, :sk], v[:, :, :sk], do, lse, delta, dk_acc, dv_acc, scale=c.scale,
                            causal=True, q_offset=p0, dq=dQ[:, :, p0:p0 + n])
    torch.cuda.synchronize()
    # the window the walk saw, written by the conversion, is the case's own K / V
    assert torch.equal(k.cpu(), t["k"].cpu()) and torch.equal(v.cpu(), t["v"].cpu())
    kv = {n: c.meta["f16"][n].astype(np.float64) for n in ("k", "v")}
    ref = oracle.backward(c.f64("q"), kv["k"], kv["v"], c.f64("do"), scale=c.scale, causal=True, q_offset=0)
    got = {"O": host64(O), "LSE": host64(LSE), "Delta": host64(Delta), "dQ": host64(dQ),
           "dK": dk_acc.cpu().numpy().astype(np.float64), "dV": dv_acc.cpu().numpy().astype(np.float64)}
    compare_full(c, got, ref)
