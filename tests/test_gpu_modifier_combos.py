"""GPU parity of the score modifiers on every dtype and in combination (llama.cpp pull request 57
lists ALiBi, the logit softcap, attention sinks and a KQ bias among the score modifiers whose
explicit path had no flash backward): the fp32 kernels with attention sinks, ALiBi and the
structured masks (key and query lengths, a sliding window), and the logit softcap together with
a dense mask, ALiBi, sinks and structure on both dtypes, all against the oracle element by
element. The oracle's score is cap(scale q.k) + mask + ALiBi; a structured mask enters it as
its dense 0 / -inf equivalent. Rows whose keys are all hidden keep only the sink (O = 0,
dQ = 0, LSE = the sink, or 0 without one) and key columns no row sees get dK = dV = 0,
exactly."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from flash_attention_train_amd import binding
from flash_attention_train_amd.inputs import make_case
from parity_util import TOL, host64, rel_err, say, upload

pytestmark = pytest.mark.gpu


def _slopes(H):
    return (2.0 ** (-8.0 * np.arange(1, H + 1) / H)).astype(np.float32)


def _sinks(H, seed):
    s = (1.0 + 2.0 * np.random.default_rng(seed).standard_normal(H)).astype(np.float32)
    s[-1] = -np.inf  # the last head has no sink
    return s


# name: (case arguments, modifiers); key_len / q_len per batch entry, window (left, right)
CASES = {
    "f32_sinks_causal_gqa": (dict(B=1, Hq=4, Hkv=2, Sq=150, Sk=150, D=64, dtype="f32", seed=301, causal=True),
                             dict(sinks=True)),
    "f32_sinks_keypad_rows": (dict(B=2, Hq=2, Hkv=2, Sq=90, Sk=70, D=128, dtype="f32", seed=302, mask="ca_keypad",
                                   mask_args={"lo": 20, "hi": 70, "masked_rows": 2}), dict(sinks=True)),
    "f32_alibi_causal_gqa": (dict(B=1, Hq=4, Hkv=1, Sq=130, Sk=130, D=128, dtype="f32", seed=303, causal=True),
                             dict(alibi=True)),
    "f32_alibi_pad_mask": (dict(B=1, Hq=2, Hkv=2, Sq=100, Sk=100, D=64, dtype="f32", seed=304, mask="sa_pad",
                                mask_args={"pad_frac": 0.1}), dict(alibi=True)),
    "f32_key_len": (dict(B=2, Hq=2, Hkv=1, Sq=96, Sk=120, D=64, dtype="f32", seed=305),
                    dict(key_len=[120, 77])),
    "f32_q_len_causal_offset": (dict(B=2, Hq=2, Hkv=2, Sq=80, Sk=144, D=128, dtype="f32", seed=306, causal=True,
                                     q_offset=64), dict(q_len=[80, 50], key_len=[144, 100])),
    "f32_window": (dict(B=1, Hq=4, Hkv=2, Sq=160, Sk=160, D=64, dtype="f32", seed=307),
                   dict(window=(24, 9))),
    "f32_everything": (dict(B=2, Hq=4, Hkv=2, Sq=100, Sk=100, D=64, dtype="f32", seed=308, causal=True,
                            mask="sa_pad", mask_args={"pad_frac": 0.1}),
                       dict(softcap=20.0, alibi=True, sinks=True, key_len=[100, 81], window=(40, -1))),
    "bf16_softcap_pad_mask": (dict(B=1, Hq=4, Hkv=2, Sq=260, Sk=260, D=128, dtype="bf16", seed=309, mask="sa_pad",
                                   mask_args={"pad_frac": 0.1}), dict(softcap=15.0)),
    "bf16_softcap_alibi_causal": (dict(B=1, Hq=4, Hkv=1, Sq=200, Sk=200, D=128, dtype="bf16", seed=310,
                                       causal=True), dict(softcap=15.0, alibi=True)),
    "bf16_softcap_everything": (dict(B=2, Hq=4, Hkv=2, Sq=150, Sk=150, D=64, dtype="bf16", seed=311,
                                     mask="ca_keypad", mask_args={"lo": 30, "hi": 150, "masked_rows": 2}),
                                dict(softcap=15.0, alibi=True, sinks=True, key_len=[150, 111], window=(-1, 40))),
}


def _setup(name):
    args, mods = CASES[name]
    c = make_case(f"combo_{name}", **args)
    sinks = _sinks(c.Hq, args["seed"]) if mods.get("sinks") else None
    alibi = _slopes(c.Hq) if mods.get("alibi") else None
    wl, wr = mods.get("window", (-1, -1))
    kl, ql = mods.get("key_len"), mods.get("q_len")
    structured = kl is not None or ql is not None or wl >= 0 or wr >= 0
    # the oracle's dense mask: the case's additive mask plus the structure's 0 / -inf
    m = None if c.mask is None else np.broadcast_to(c.mask, (c.B, c.Sq, c.Sk)).astype(np.float64)
    if structured:
        sm = oracle.structured_mask(c.B, c.Sq, c.Sk, key_len=kl, q_len=ql, window_left=wl, window_right=wr,
                                    q_offset=c.q_offset)
        m = sm if m is None else m + sm
    return c, mods, sinks, alibi, (wl, wr), kl, ql, m


def _visibility(c, m):
    vis = np.ones((c.B, c.Sq, c.Sk), bool)
    if m is not None:
        vis &= np.isfinite(m)
    if c.causal:
        vis &= np.arange(c.Sk)[None, None, :] <= (c.q_offset + np.arange(c.Sq))[None, :, None]
    return ~vis.any(axis=2), ~vis.any(axis=1)


@pytest.mark.parametrize("name", list(CASES))
def test_modifiers_match_oracle(name):
    c, mods, sinks, alibi, window, kl, ql, m = _setup(name)
    say(f"case {name}: {c.dtype} B={c.B} Hq={c.Hq} Hkv={c.Hkv} Sq={c.Sq} Sk={c.Sk} D={c.D} {mods}")
    ref = oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), m, scale=c.scale, causal=c.causal,
                          q_offset=c.q_offset, sinks=None if sinks is None else sinks.astype(np.float64),
                          alibi=None if alibi is None else alibi.astype(np.float64), softcap=mods.get("softcap"))
    t = upload(c)
    kw = dict(mask=t["mask"], scale=c.scale, causal=c.causal, q_offset=c.q_offset, window=window,
              softcap=mods.get("softcap", 0.0),
              key_len=None if kl is None else torch.tensor(kl, dtype=torch.int32, device="cuda"),
              q_len=None if ql is None else torch.tensor(ql, dtype=torch.int32, device="cuda"),
              alibi=None if alibi is None else torch.from_numpy(alibi).to("cuda"))
    sk = None if sinks is None else torch.from_numpy(sinks).to("cuda")
    o, lse = binding.fwd(t["q"], t["k"], t["v"], sinks=sk, **kw)
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, **kw)
    got = {"O": host64(o), "LSE": host64(lse), "Delta": host64(delta), "dQ": host64(dq), "dK": host64(dk),
           "dV": host64(dv)}
    if sinks is not None:
        got["dSink"] = binding.bwd_sinks(lse, delta, sk).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    full, dead = _visibility(c, m)
    tol = TOL[c.dtype]
    errs = {}
    for n in got:
        g, r = got[n], ref[n]
        assert g.shape == r.shape and np.isfinite(g).all(), n
        keep = np.ones(g.shape, bool)
        if n in ("O", "LSE", "Delta", "dQ") and full.any():
            rows = np.broadcast_to(full[:, None, :] if g.ndim == 3 else full[:, None, :, None], g.shape)
            if n == "LSE":  # the sink alone (0 without one)
                s = np.zeros(c.Hq) if sinks is None else np.where(np.isfinite(sinks), sinks, 0).astype(np.float64)
                want = np.broadcast_to(s[None, :, None], g.shape)
                assert np.array_equal(g[rows], want[rows]), "LSE of fully masked rows"
            else:
                assert np.all(g[rows] == 0), f"{n}: fully masked rows are not exactly zero"
            keep &= ~rows
        if n in ("dK", "dV") and dead.any():
            cols = np.broadcast_to(dead[:, None, :, None], g.shape)
            assert np.all(g[cols] == 0), f"{n}: dead key columns are not exactly zero"
            keep &= ~cols
        errs[n] = rel_err(g[keep], r[keep]) if keep.any() else 0.0
    say(f"  errors: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"{name}: {bad} above {tol}"
