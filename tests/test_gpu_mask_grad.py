"""GPU parity of the mask's gradient (a learnable KQ bias, one of the score modifiers whose flash
backward llama.cpp pull request 57 lacked): for every score dL/dM = P (dP - Delta), added into an
fp32 tensor of the mask's shape, summed over the batch entries and heads the mask is shared by.
Compared with the oracle element by element (entries hidden by -inf, causal masking or a
structured mask get exactly 0), on both dtypes: a per-head bias with GQA and causal masking, a
mask shared by the batch and the heads (several heads add into one entry), the split backward
and the dQ walk in its own launch, and the chunked walk over a window, whose chunks sum into one
gradient."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from flash_attention_train_amd import binding, configs
from flash_attention_train_amd.inputs import make_case
from parity_util import TOL, rel_err, say, upload

pytestmark = pytest.mark.gpu


def _per_head(c, seed):
    rng = np.random.default_rng(seed)
    m = (0.8 * rng.standard_normal((c.B, c.Hq, c.Sq, c.Sk))).astype(np.float32)
    m[0, 1, :, c.Sk // 3] = -np.inf  # a key column hidden in one head
    m[-1, -1, c.Sq // 2, :] = -np.inf  # a row fully masked in one head
    return m


CASES = {
    "bf16_per_head_causal_gqa": (dict(B=2, Hq=4, Hkv=2, Sq=200, Sk=200, D=128, dtype="bf16", seed=401, causal=True),
                                 "per_head"),
    "f32_per_head_d64": (dict(B=1, Hq=2, Hkv=1, Sq=96, Sk=130, D=64, dtype="f32", seed=402), "per_head"),
    "bf16_shared_keypad": (dict(B=2, Hq=4, Hkv=4, Sq=150, Sk=120, D=64, dtype="bf16", seed=403, mask="ca_keypad",
                                mask_args={"lo": 40, "hi": 120, "masked_rows": 2}), "case"),
    "bf16_batch_shared_pad": (dict(B=2, Hq=4, Hkv=2, Sq=260, Sk=260, D=128, dtype="bf16", seed=404, mask="sa_pad",
                                   mask_args={"pad_frac": 0.1}), "case"),
    "f32_shared_causal": (dict(B=2, Hq=2, Hkv=2, Sq=70, Sk=90, D=128, dtype="f32", seed=405, causal=True,
                               mask="sa_pad", mask_args={"pad_frac": 0.2}), "case"),
}


def _setup(name):
    args, kind = CASES[name]
    c = make_case(f"mask_grad_{name}", **args)
    if kind == "per_head":
        c.mask = _per_head(c, args["seed"] + 7)
    # a bias with finite values too (the cases' masks are 0 / -inf): the gradient is then not
    # only the visibility pattern
    if kind == "case":
        rng = np.random.default_rng(args["seed"] + 9)
        c.mask = np.where(np.isfinite(c.mask), 0.5 * rng.standard_normal(c.mask.shape), c.mask).astype(np.float32)
    return c


def _check(c, got, want):
    assert got.shape == want.shape and np.isfinite(got).all()
    hidden = np.broadcast_to(~np.isfinite(c.mask), got.shape)
    assert np.all(got[hidden] == 0), "hidden entries must get exactly zero gradient"
    err = rel_err(got, want)
    say(f"  dbias error {err:.2e}")
    assert err <= TOL[c.dtype], err


@pytest.mark.parametrize("splits", [(0, 0, 0), (2, 2, 1), (1, 3, 2)])
@pytest.mark.parametrize("name", list(CASES))
def test_mask_gradient(name, splits):
    c = _setup(name)
    kv, qs, dql = splits
    say(f"case {name}: mask {c.mask.shape}, kv_split {kv} q_split {qs} dq_launch {dql}")
    want = oracle.bias_grad(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), c.mask.astype(np.float64),
                            scale=c.scale, causal=c.causal, q_offset=c.q_offset)
    t = upload(c)
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal, q_offset=c.q_offset)
    delta = binding.bwd_preprocess(o, t["do"])
    db = torch.zeros(t["mask"].shape, dtype=torch.float32, device="cuda")
    binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=t["mask"], scale=c.scale, causal=c.causal,
                q_offset=c.q_offset, kv_split=kv, q_split=qs, dq_launch=dql, dbias=db)
    torch.cuda.synchronize()
    _check(c, db.cpu().numpy().astype(np.float64), want)


def test_mask_gradient_with_tile_map_and_adds_in():
    """With the mask's block map (dead blocks skipped, open blocks not read) the gradient is the
    same; and a second call adds into the first's result."""
    c = _setup("bf16_batch_shared_pad")
    want = oracle.bias_grad(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), c.mask.astype(np.float64),
                            scale=c.scale)
    t = upload(c)
    tiles = binding.mask_tile_map(t["mask"], t["q"], t["k"])
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, mask_tiles=tiles)
    delta = binding.bwd_preprocess(o, t["do"])
    db = torch.zeros(t["mask"].shape, dtype=torch.float32, device="cuda")
    for _ in range(2):
        binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=t["mask"], scale=c.scale, mask_tiles=tiles,
                    dbias=db)
    torch.cuda.synchronize()
    _check(c, db.cpu().numpy().astype(np.float64) / 2, want)


def test_mask_gradient_chunked_window():
    """The chunked walk over a window: each chunk's rows add their gradient into the window's
    [1, W, W] bias gradient (chunk c's rows sit at q_offset = c C), which then equals the
    one-shot causal problem's."""
    W, C = 384, 128
    c = make_case("mask_grad_window", B=1, Hq=4, Hkv=2, Sq=W, Sk=W, D=128, dtype="bf16", seed=406, causal=True)
    rng = np.random.default_rng(407)
    c.mask = (0.5 * rng.standard_normal((1, W, W))).astype(np.float32)
    want = oracle.bias_grad(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), c.mask.astype(np.float64),
                            scale=c.scale, causal=True, q_offset=0)
    t = upload(c)
    db = torch.zeros((1, W, W), dtype=torch.float32, device="cuda")
    dk_acc = torch.zeros((1, c.Hkv, W, c.D), dtype=torch.float32, device="cuda")
    dv_acc = torch.zeros_like(dk_acc)
    for p0, n, sk in configs.chunk_plan(W, C):
        q, do = t["q"][:, :, p0:p0 + n], t["do"][:, :, p0:p0 + n]
        kk, vv = t["k"][:, :, :sk], t["v"][:, :, :sk]
        mk, dbk = t["mask"][:, p0:p0 + n, :sk], db[:, p0:p0 + n, :sk]
        o, lse = binding.fwd(q, kk, vv, mask=mk, scale=c.scale, causal=True, q_offset=p0)
        delta = binding.bwd_preprocess(o, do)
        binding.bwd_chunked(q, kk, vv, do, lse, delta, dk_acc, dv_acc, mask=mk, scale=c.scale, causal=True,
                            q_offset=p0, dbias=dbk)
    torch.cuda.synchronize()
    _check(c, db.cpu().numpy().astype(np.float64), want)
