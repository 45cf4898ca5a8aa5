"""GPU parity of the backward's dQ from stored dS (bwd_dq_launch = 3): the dK/dV walk writes every
dS = P (dP - Delta) it forms, and a second kernel forms dQ = scale dS K from it (the tiled backward of
llama.cpp pull request 57, commit 86c140d, computes dQ from the same dS). Against the oracle element by
element, on the structures that decide which dS blocks exist: causal diagonals and offsets, a mask
tile map with dead blocks, key lengths with a sliding window, the logit softcap, splits of both walks,
D = 64, and the chunked walk over a window. dK and dV come from the same walk as with the dQ walk,
so they must be bitwise equal to that setting's; fully masked rows keep dQ exactly 0."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from flash_attention_train_amd import binding, configs
from flash_attention_train_amd.inputs import make_case
from parity_util import TOL, host64, rel_err, say, upload

pytestmark = pytest.mark.gpu

# name: (case arguments, modifiers, split hints)
CASES = {
    "causal_gqa_ragged": (dict(B=1, Hq=4, Hkv=2, Sq=300, Sk=300, D=128, dtype="bf16", seed=501, causal=True), {}, {}),
    "causal_offset_chunk": (dict(B=1, Hq=2, Hkv=1, Sq=200, Sk=520, D=128, dtype="bf16", seed=502, causal=True,
                                 q_offset=320), {}, {}),
    "d64_noncausal_batch": (dict(B=2, Hq=2, Hkv=2, Sq=190, Sk=260, D=64, dtype="bf16", seed=503), {}, {}),
    "pad_mask_tile_map": (dict(B=1, Hq=4, Hkv=2, Sq=390, Sk=390, D=128, dtype="bf16", seed=504, mask="sa_pad",
                               mask_args={"pad_frac": 0.1}), {"tiles": True}, {}),
    "keypad_rows_tile_map": (dict(B=2, Hq=2, Hkv=2, Sq=300, Sk=260, D=128, dtype="bf16", seed=505, mask="ca_keypad",
                                  mask_args={"lo": 30, "hi": 200, "masked_rows": 2}), {"tiles": True}, {}),
    "window_key_len": (dict(B=2, Hq=2, Hkv=1, Sq=520, Sk=520, D=128, dtype="bf16", seed=506),
                       {"window": (40, 40), "key_len": [520, 301]}, {}),
    "softcap_causal": (dict(B=1, Hq=2, Hkv=2, Sq=260, Sk=260, D=128, dtype="bf16", seed=507, causal=True),
                       {"softcap": 20.0}, {}),
    "softcap_pad_mask": (dict(B=1, Hq=2, Hkv=1, Sq=200, Sk=200, D=128, dtype="bf16", seed=508, mask="sa_pad",
                              mask_args={"pad_frac": 0.1}), {"softcap": 15.0}, {}),
    "splits": (dict(B=1, Hq=4, Hkv=2, Sq=600, Sk=600, D=128, dtype="bf16", seed=509, causal=True), {},
               dict(kv_split=2, q_split=3, q_split_tiles=2)),
    # whole dK/dV units over a single query row: the other 63 rows of its dS block are zeros
    "one_row": (dict(B=1, Hq=2, Hkv=1, Sq=1, Sk=300, D=128, dtype="bf16", seed=511), {}, {}),
}


def _run(name):
    args, mods, splits = CASES[name]
    c = make_case(f"dqds_{name}", **args)
    t = upload(c)
    kw = dict(mask=t["mask"], scale=c.scale, causal=c.causal, q_offset=c.q_offset)
    m = None if c.mask is None else np.broadcast_to(c.mask, (c.B, c.Sq, c.Sk)).astype(np.float64)
    if "window" in mods:
        wl, wr = mods["window"]
        kl = mods["key_len"]
        kw["window"] = (wl, wr)
        kw["key_len"] = torch.tensor(kl, dtype=torch.int32, device="cuda")
        sm = oracle.structured_mask(c.B, c.Sq, c.Sk, key_len=kl, q_len=None, window_left=wl, window_right=wr,
                                    q_offset=c.q_offset)
        m = sm if m is None else m + sm
    if "softcap" in mods:
        kw["softcap"] = mods["softcap"]
    if mods.get("tiles"):
        kw["mask_tiles"] = binding.mask_tile_map(t["mask"], t["q"], t["k"])
    o, lse = binding.fwd(t["q"], t["k"], t["v"], **kw)
    delta = binding.bwd_preprocess(o, t["do"])
    walk = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, dq_launch=1, **splits, **kw)
    stored = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, dq_launch=3, **splits, **kw)
    torch.cuda.synchronize()
    ref = oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), m, scale=c.scale, causal=c.causal,
                          q_offset=c.q_offset, softcap=mods.get("softcap"))
    return c, m, walk, stored, ref


@pytest.mark.parametrize("name", list(CASES))
def test_dq_from_stored_ds(name):
    c, m, walk, stored, ref = _run(name)
    say(f"case {name}: B={c.B} Hq={c.Hq} Hkv={c.Hkv} Sq={c.Sq} Sk={c.Sk} D={c.D}")
    for a, b in zip(walk[1:], stored[1:]):
        assert torch.equal(a, b), "dK / dV must not depend on how dQ is formed"
    dq = host64(stored[0])
    assert np.isfinite(dq).all()
    vis = np.ones((c.B, c.Sq, c.Sk), bool) if m is None else np.isfinite(m)
    if c.causal:
        vis &= np.arange(c.Sk)[None, None, :] <= (c.q_offset + np.arange(c.Sq))[None, :, None]
    full = ~vis.any(axis=2)
    if full.any():
        rows = np.broadcast_to(full[:, None, :, None], dq.shape)
        assert np.all(dq[rows] == 0), "fully masked rows must get dQ = 0 exactly"
    errs = {"dQ": rel_err(dq, ref["dQ"]), "dK": rel_err(host64(stored[1]), ref["dK"]),
            "dV": rel_err(host64(stored[2]), ref["dV"]), "dQ_vs_walk": rel_err(dq, host64(walk[0]))}
    say("  errors: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert errs["dQ"] <= TOL["bf16"] and errs["dK"] <= TOL["bf16"] and errs["dV"] <= TOL["bf16"], errs


def test_dq_from_stored_ds_chunked_walk():
    """The chunked walk over a window with dQ from stored dS: each chunk's dQ and the window's fp32
    dK / dV accumulators equal the one-shot causal problem's."""
    W, C = 640, 128
    c = make_case("dqds_window", B=1, Hq=4, Hkv=2, Sq=W, Sk=W, D=128, dtype="bf16", seed=510, causal=True)
    t = upload(c)
    dk_acc = torch.zeros((1, c.Hkv, W, c.D), dtype=torch.float32, device="cuda")
    dv_acc = torch.zeros_like(dk_acc)
    dq = torch.empty_like(t["q"])
    for p0, n, sk in configs.chunk_plan(W, C):
        q, do = t["q"][:, :, p0:p0 + n], t["do"][:, :, p0:p0 + n]
        kk, vv = t["k"][:, :, :sk], t["v"][:, :, :sk]
        o, lse = binding.fwd(q, kk, vv, scale=c.scale, causal=True, q_offset=p0)
        delta = binding.bwd_preprocess(o, do)
        dq[:, :, p0:p0 + n] = binding.bwd_chunked(q, kk, vv, do, lse, delta, dk_acc, dv_acc, scale=c.scale,
                                                  causal=True, q_offset=p0, dq_launch=3)
    torch.cuda.synchronize()
    ref = oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), None, scale=c.scale, causal=True,
                          q_offset=0)
    errs = {"dQ": rel_err(host64(dq), ref["dQ"]), "dK": rel_err(dk_acc.cpu().numpy().astype(np.float64), ref["dK"]),
            "dV": rel_err(dv_acc.cpu().numpy().astype(np.float64), ref["dV"])}
    say("  chunked walk errors: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL["bf16"] for v in errs.values()), errs

