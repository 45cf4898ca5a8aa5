"""GPU parity of a score bias per head (mask [Bm, Hq, Sq, Sk], the pull request's KQ bias,
with -inf entries still hiding scores) against the oracle, element by element: both dtypes,
GQA, causal, the split forward, the backward's split tail and the dQ walk in its own
launch. Rows fully masked in one head only must be exactly zero there (and only there);
key columns hidden from every head of a group get exactly zero dK / dV."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from flash_attention_train_amd import binding
from flash_attention_train_amd.inputs import make_case
from parity_util import TOL, host64, rel_err, say, upload

pytestmark = pytest.mark.gpu


def _case(name, *, B, Hq, Hkv, Sq, Sk, D, dtype, seed, causal=False):
    c = make_case(name, B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D, dtype=dtype, seed=seed, causal=causal)
    rng = np.random.default_rng(seed + 500)
    m = (0.8 * rng.standard_normal((B, Hq, Sq, Sk))).astype(np.float32)
    m[0, 1, :, Sk // 3] = -np.inf            # a key column hidden in one head of a group only
    m[-1, -1, Sq // 2, :] = -np.inf          # a row fully masked in one head only
    for h in range(Hq):                      # a key column hidden from every head of KV head 0
        if h // (Hq // Hkv) == 0:
            m[:, h, :, Sk - 1] = -np.inf
    c.meta["bias"] = m
    return c


CASES = {
    "dit_like": lambda: _case("dit_like", B=2, Hq=4, Hkv=2, Sq=260, Sk=200, D=128, dtype="bf16", seed=111),
    "lm_causal_gqa4": lambda: _case("lm_causal_gqa4", B=1, Hq=8, Hkv=2, Sq=300, Sk=300, D=128, dtype="bf16",
                                    seed=112, causal=True),
    "d64_bf16": lambda: _case("d64_bf16", B=1, Hq=2, Hkv=1, Sq=150, Sk=130, D=64, dtype="bf16", seed=113),
    "fp32_small": lambda: _case("fp32_small", B=1, Hq=2, Hkv=1, Sq=70, Sk=90, D=64, dtype="f32", seed=114),
}
_REF = {}


def reference(name):
    if name not in _REF:
        c = CASES[name]()
        _REF[name] = (c, oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"),
                                         c.meta["bias"].astype(np.float64), scale=c.scale, causal=c.causal,
                                         q_offset=c.q_offset))
    return _REF[name]


def run(c, **kw):
    t = upload(c)
    bias = torch.from_numpy(c.meta["bias"]).cuda()
    split = kw.pop("split", 0)
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=bias, scale=c.scale, causal=c.causal, q_offset=c.q_offset,
                         split=split)
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=bias, scale=c.scale,
                             causal=c.causal, q_offset=c.q_offset, **kw)
    torch.cuda.synchronize()
    return {"O": host64(o), "LSE": host64(lse), "Delta": host64(delta), "dQ": host64(dq), "dK": host64(dk),
            "dV": host64(dv)}


def compare(c, got, ref):
    m = c.meta["bias"]
    vis = np.isfinite(m)
    if c.causal:
        vis &= np.arange(c.Sk)[None, None, None, :] <= (c.q_offset + np.arange(c.Sq))[None, None, :, None]
    full = ~vis.any(axis=3)                                                  # [B, Hq, Sq]
    G = c.Hq // c.Hkv
    dead = ~vis.any(axis=2).reshape(c.B, c.Hkv, G, c.Sk).any(axis=2)         # [B, Hkv, Sk]
    assert full.any() and dead.any()
    errs = {}
    for n in ("O", "LSE", "Delta", "dQ", "dK", "dV"):
        g, r = got[n], ref[n]
        keep = np.ones(g.shape, bool)
        if n in ("O", "LSE", "Delta", "dQ"):
            rows = np.broadcast_to(full if g.ndim == 3 else full[..., None], g.shape)
            assert np.all(g[rows] == 0), f"{n}: fully masked rows are not exactly zero"
            keep &= ~rows
        else:
            cols = np.broadcast_to(dead[..., None], g.shape)
            assert np.all(g[cols] == 0), f"{n}: dead key columns are not exactly zero"
            keep &= ~cols
        errs[n] = rel_err(g[keep], r[keep])
    say(f"  {c.name} errors:", {k: f"{v:.2e}" for k, v in errs.items()})
    bad = {k: v for k, v in errs.items() if not v <= TOL[c.dtype]}
    assert not bad, bad


@pytest.mark.parametrize("name", list(CASES))
def test_head_bias_parity(name):
    c, ref = reference(name)
    say(f"case {name}: per-head bias, {c.dtype}")
    compare(c, run(c), ref)


@pytest.mark.parametrize("kw", [dict(split=3), dict(kv_split=2, q_split=2, q_split_tiles=1),
                                dict(kv_split=1, q_split=1, dq_launch=2)])
def test_head_bias_paths(kw):
    c, ref = reference("dit_like")
    say(f"case dit_like: {kw}")
    compare(c, run(c, **dict(kw)), ref)


def test_head_bias_rejects_block_map():
    c = CASES["d64_bf16"]()
    t = upload(c)
    bias = torch.from_numpy(c.meta["bias"]).cuda()
    with pytest.raises(binding.FaError):
        binding.mask_tile_map(bias, t["q"], t["k"])
