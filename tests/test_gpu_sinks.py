"""GPU parity of the attention sinks (one logit per query head joining every row's
softmax denominator, with no value row) against the oracle: O, LSE, Delta, dQ, dK, dV
and the sinks' own gradient, element by element. Rows whose keys are all masked keep
only the sink: O = 0 and dQ = 0 exactly, and LSE equal to the sink's value exactly.
A head whose sink is -inf has no sink. The cases cover the causal GQA layer, key
padding with fully masked rows, D = 64, the split forward and its merge, the other
forward variants, and the dQ walk in either launch."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from flash_attention_train_amd import binding
from flash_attention_train_amd.inputs import make_case
from parity_util import TOL, host64, rel_err, say, upload, visibility

pytestmark = pytest.mark.gpu


def _sinks(Hq, seed):
    s = (1.0 + 2.0 * np.random.default_rng(seed).standard_normal(Hq)).astype(np.float32)
    s[-1] = -np.inf  # the last head has no sink
    return s


CASES = {
    "lm_causal_gqa4": lambda: make_case("lm_causal_gqa4", B=1, Hq=8, Hkv=2, Sq=300, Sk=300, D=128, dtype="bf16",
                                        seed=91, causal=True),
    "ca_keypad_rows": lambda: make_case("ca_keypad_rows", B=2, Hq=4, Hkv=4, Sq=200, Sk=150, D=128, dtype="bf16",
                                        seed=92, mask="ca_keypad", mask_args={"lo": 40, "hi": 150, "masked_rows": 2}),
    "sa_pad_d64": lambda: make_case("sa_pad_d64", B=1, Hq=4, Hkv=2, Sq=260, Sk=260, D=64, dtype="bf16", seed=93,
                                    mask="sa_pad", mask_args={"pad_frac": 0.1}),
}

_REF = {}


def reference(name):
    if name not in _REF:
        c = CASES[name]()
        s = _sinks(c.Hq, 7 + len(_REF))
        m = None if c.mask is None else c.mask.astype(np.float64)
        _REF[name] = (c, s, oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), m, scale=c.scale,
                                            causal=c.causal, q_offset=c.q_offset, sinks=s.astype(np.float64)))
    return _REF[name]


def run(c, sinks, *, split=0, variant=0, dq_launch=0):
    t = upload(c)
    sk = torch.from_numpy(sinks).to("cuda")
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal,
                         q_offset=c.q_offset, split=split, variant=variant, sinks=sk)
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=t["mask"], scale=c.scale,
                             causal=c.causal, q_offset=c.q_offset, dq_launch=dq_launch)
    dsink = binding.bwd_sinks(lse, delta, sk)
    torch.cuda.synchronize()
    return {"O": host64(o), "LSE": host64(lse), "Delta": host64(delta), "dQ": host64(dq), "dK": host64(dk),
            "dV": host64(dv), "dSink": dsink.cpu().numpy().astype(np.float64)}


def compare(c, sinks, got, ref):
    tol = TOL[c.dtype]
    full, dead = visibility(c)
    errs = {}
    for n in ("O", "LSE", "Delta", "dQ", "dK", "dV", "dSink"):
        g, r = got[n], ref[n]
        assert g.shape == r.shape and np.isfinite(g).all(), n
        keep = np.ones(g.shape, bool)
        if n in ("O", "LSE", "Delta", "dQ") and full.any():
            rows = np.broadcast_to(full[:, None, :] if g.ndim == 3 else full[:, None, :, None], g.shape)
            if n == "LSE":  # the sink alone: LSE is the sink's value (0 for a head without one)
                want = np.broadcast_to(np.where(np.isfinite(sinks), sinks, 0).astype(np.float64)[None, :, None],
                                       g.shape)
                assert np.array_equal(g[rows], want[rows]), "LSE of fully masked rows is not the sink"
            else:
                assert np.all(g[rows] == 0), f"{n}: fully masked rows are not exactly zero"
            keep &= ~rows
        if n in ("dK", "dV") and dead.any():
            cols = np.broadcast_to(dead[:, None, :, None], g.shape)
            assert np.all(g[cols] == 0), f"{n}: dead key columns are not exactly zero"
            keep &= ~cols
        if n == "dSink":
            # a sum over rows of terms of both signs (Delta has either sign): its rounding is
            # measured against the sum of the terms' magnitudes, the scale an error in each
            # term (bf16 O inside Delta) propagates at, not against the cancelled total
            keep = np.isfinite(sinks)
            assert np.all(g[~keep] == 0), "a head without a sink has a sink gradient"
            mag = np.array([np.sum(np.exp(float(sinks[h]) - ref["LSE"][:, h]) * np.abs(ref["Delta"][:, h]))
                            for h in range(len(sinks)) if keep[h]])
            errs[n] = float(np.abs(g[keep] - r[keep]).max() / mag.max())
            continue
        errs[n] = rel_err(g[keep], r[keep])
    say(f"  {c.name} errors:", {k: f"{v:.2e}" for k, v in errs.items()})
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{c.name}: above tolerance {tol}: {bad}"


@pytest.mark.parametrize("name", list(CASES))
def test_sinks_parity(name):
    c, s, ref = reference(name)
    say(f"case {name}: sinks {s}")
    compare(c, s, run(c, s), ref)


@pytest.mark.parametrize("split,variant", [(3, 0), (1, 2), (1, 3)])
def test_sinks_forward_paths(split, variant):
    """The split forward (the sink joins in the merge) and the other forward variants."""
    c, s, ref = reference("ca_keypad_rows")
    say(f"case ca_keypad_rows: split {split} variant {variant}")
    compare(c, s, run(c, s, split=split, variant=variant), ref)


def test_sinks_with_own_dq_launch():
    c, s, ref = reference("lm_causal_gqa4")
    compare(c, s, run(c, s, dq_launch=2), ref)


def test_sinks_of_minus_inf_are_no_sinks():
    """Sinks that are all -inf give the same bits as no sinks at all."""
    c = CASES["lm_causal_gqa4"]()
    t = upload(c)
    none = binding.fwd(t["q"], t["k"], t["v"], scale=c.scale, causal=True)
    ninf = binding.fwd(t["q"], t["k"], t["v"], scale=c.scale, causal=True,
                       sinks=torch.full((c.Hq,), -np.inf, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(none[0], ninf[0]) and torch.equal(none[1], ninf[1])
