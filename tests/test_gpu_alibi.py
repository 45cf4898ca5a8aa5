"""GPU parity of ALiBi (score (b, h, i, j) gets -a_h |j - (q_offset + i)|, added after the
scale) against the oracle: every output element by element, with the exact-zero checks
for fully masked rows and dead key columns. Cases: the causal GQA layer with the usual
slopes 2^(-8 (h + 1) / H), ALiBi on top of a dense padding mask read through its tile map,
key padding with fully masked rows, the split forward and the other forward variants,
the dQ walk in its own launch, and the chunked walk over a window (positions offset by
each chunk's q_offset)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from flash_attention_train_amd import binding, configs
from flash_attention_train_amd.inputs import make_case
from parity_util import compare_full, host64, say, upload

pytestmark = pytest.mark.gpu


def slopes(H):
    return (2.0 ** (-8.0 * np.arange(1, H + 1) / H)).astype(np.float32)


CASES = {
    "lm_causal_gqa4": lambda: make_case("lm_causal_gqa4", B=1, Hq=8, Hkv=2, Sq=300, Sk=300, D=128, dtype="bf16",
                                        seed=95, causal=True),
    "sa_pad_d64_tiles": lambda: make_case("sa_pad_d64_tiles", B=1, Hq=4, Hkv=2, Sq=260, Sk=260, D=64, dtype="bf16",
                                          seed=96, mask="sa_pad", mask_args={"pad_frac": 0.1}),
    "ca_keypad_rows": lambda: make_case("ca_keypad_rows", B=2, Hq=4, Hkv=4, Sq=200, Sk=150, D=128, dtype="bf16",
                                        seed=97, mask="ca_keypad", mask_args={"lo": 40, "hi": 150, "masked_rows": 2}),
}
_REF = {}


def reference(name):
    if name not in _REF:
        c = CASES[name]()
        a = slopes(c.Hq)
        m = None if c.mask is None else c.mask.astype(np.float64)
        _REF[name] = (c, a, oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), m, scale=c.scale,
                                            causal=c.causal, q_offset=c.q_offset, alibi=a.astype(np.float64)))
    return _REF[name]


def run(c, a, *, split=0, variant=0, dq_launch=0, tiles=False):
    t = upload(c)
    al = torch.from_numpy(a).to("cuda")
    mt = binding.mask_tile_map(t["mask"], t["q"], t["k"]) if tiles and t["mask"] is not None else None
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal,
                         q_offset=c.q_offset, split=split, variant=variant, alibi=al, mask_tiles=mt)
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=t["mask"], scale=c.scale,
                             causal=c.causal, q_offset=c.q_offset, dq_launch=dq_launch, alibi=al, mask_tiles=mt)
    torch.cuda.synchronize()
    return {"O": host64(o), "LSE": host64(lse), "Delta": host64(delta), "dQ": host64(dq), "dK": host64(dk),
            "dV": host64(dv)}


@pytest.mark.parametrize("name", list(CASES))
def test_alibi_parity(name):
    c, a, ref = reference(name)
    say(f"case {name}: alibi slopes {a}")
    compare_full(c, run(c, a, tiles=True), ref)


@pytest.mark.parametrize("split,variant,dq_launch", [(3, 0, 0), (1, 2, 0), (1, 3, 0), (1, 1, 2)])
def test_alibi_paths(split, variant, dq_launch):
    c, a, ref = reference("ca_keypad_rows")
    say(f"case ca_keypad_rows: split {split} variant {variant} dq_launch {dq_launch}")
    compare_full(c, run(c, a, split=split, variant=variant, dq_launch=dq_launch), ref)


def test_alibi_chunked_window():
    W, C = 512, 128
    c = configs.make("long_window", W=W, Hq=4, Hkv=1)
    a = slopes(c.Hq)
    al = torch.from_numpy(a).to("cuda")
    say(f"alibi chunked walk: W={W}, chunks of {C}")
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
                             lse=LSE[:, :, p0:p0 + n], alibi=al)
        delta = binding.bwd_preprocess(o, do, delta=Delta[:, :, p0:p0 + n])
        binding.bwd_chunked(q, kk, vv, do, lse, delta, dk_acc, dv_acc, scale=c.scale, causal=True, q_offset=p0,
                            dq=dQ[:, :, p0:p0 + n], alibi=al)
    torch.cuda.synchronize()
    ref = oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), scale=c.scale, causal=True, q_offset=0,
                          alibi=a.astype(np.float64))
    got = {"O": host64(O), "LSE": host64(LSE), "Delta": host64(Delta), "dQ": host64(dQ),
           "dK": dk_acc.cpu().numpy().astype(np.float64), "dV": dv_acc.cpu().numpy().astype(np.float64)}
    compare_full(c, got, ref)
