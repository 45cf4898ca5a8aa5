"""Helpers for the GPU parity tests: upload a seeded case, run the op through the
C ABI, and compare with the oracle element by element.

Error metric per output tensor (over the elements that are not exempt):
    e = max |gpu - oracle| / max |oracle|
and the bar is 1e-4 for fp32 inputs and 2e-2 for bf16 inputs. Exempt elements are
checked for exact equality instead: rows of fully masked queries (O, LSE, dQ all
exactly 0) and key columns no query can see (dK = dV = 0 exactly).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from flash_attention_train_amd import binding
from flash_attention_train_amd.inputs import BF16, Case

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == BF16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def upload(c: Case) -> dict:
    d = {n: dev(getattr(c, n), c.dtype) for n in ("q", "k", "v", "do")}
    d["mask"] = None if c.mask is None else torch.from_numpy(c.mask).to("cuda")
    return d


def run_gpu(c: Case, t: dict | None = None, **bwd_kw) -> dict:
    """fwd -> preprocess -> bwd on the GPU; returns float64 host copies."""
    t = t or upload(c)
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal,
                         q_offset=c.q_offset)
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=t["mask"], scale=c.scale,
                             causal=c.causal, q_offset=c.q_offset, **bwd_kw)
    torch.cuda.synchronize()
    return {"O": host64(o), "LSE": host64(lse), "Delta": host64(delta), "dQ": host64(dq), "dK": host64(dk),
            "dV": host64(dv)}


def visibility(c: Case):
    """(fully_masked_rows [B, Sq], dead_key_columns [B, Sk]) from the mask and causal structure."""
    vis = np.ones((c.B, c.Sq, c.Sk), bool)
    if c.mask is not None:
        m = c.mask if c.mask.shape[0] == c.B else np.broadcast_to(c.mask, (c.B, c.Sq, c.Sk))
        vis &= np.isfinite(m)
    if c.causal:
        vis &= np.arange(c.Sk)[None, None, :] <= (c.q_offset + np.arange(c.Sq))[None, :, None]
    return ~vis.any(axis=2), ~vis.any(axis=1)


def rel_err(g: np.ndarray, r: np.ndarray) -> float:
    den = np.abs(r).max()
    return float(np.abs(g - r).max() / den) if den > 0 else float(np.abs(g - r).max())


def compare_full(c: Case, got: dict, ref: dict, names=("O", "LSE", "Delta", "dQ", "dK", "dV"),
                 zero_ok=()) -> dict:
    """Element-by-element comparison; returns the error per tensor. Raises on failure."""
    tol = TOL[c.dtype]
    full, dead = visibility(c)
    errs = {}
    for n in names:
        g, r = got[n], ref[n]
        assert g.shape == r.shape, (n, g.shape, r.shape)
        keep = np.ones(g.shape, bool)
        if n in ("O", "LSE", "Delta", "dQ") and full.any():
            rows = np.broadcast_to(full[:, None, :] if g.ndim == 3 else full[:, None, :, None], g.shape)
            assert np.all(g[rows] == 0), f"{n}: fully masked rows are not exactly zero"
            keep &= ~rows
        if n in ("dK", "dV") and dead.any():
            cols = np.broadcast_to(dead[:, None, :, None], g.shape)
            assert np.all(g[cols] == 0), f"{n}: dead key columns are not exactly zero"
            keep &= ~cols
        assert np.isfinite(g).all(), f"{n}: non-finite values"
        if n in ("dQ", "dK", "dV") and np.abs(r[keep]).max() == 0:
            # a gradient that is exactly zero by construction (e.g. dQ and dK with a
            # single key): the GPU's must be zero up to rounding, measured against
            # the size of dV, which is not zero there
            assert n in zero_ok, f"{n}: the oracle gradient is zero (the check would be vacuous)"
            errs[n] = float(np.abs(g).max() / np.abs(ref["dV"]).max())
            continue
        errs[n] = rel_err(g[keep], r[keep])
    say(f"  {c.name} errors:", {k: f"{v:.2e}" for k, v in errs.items()})
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{c.name}: above tolerance {tol}: {bad}"
    return errs
