"""Derive and assert the gfx950 lane maps the kernels rely on (the pages' lesson:
an operand's lane map can differ from the accumulator's, so it is probed, not
assumed -- "Flash Attn Training" skill page, section 6, trap 10).

The kernels assume, for the 32x32 matrix-core family:
  A (32 x K): lane l holds row l % 32, register slot j carries k-slot (l // 32, j)
  B (K x 32): lane l holds column l % 32, register slot j carries the same k-slot
  C (32 x 32): lane l, register r holds (row 8 (r // 4) + 4 (l // 32) + r % 4, col l % 32)
The test loads random small-integer matrices under that assumption and requires
the exact product back. Probe results are also written as JSON to the folder named by
FA_PROBE_OUT, when that is set, for reading.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

from parity_util import say

pytestmark = pytest.mark.gpu

OUT = os.environ.get("FA_PROBE_OUT")  # optional folder for the probes' JSON records


def _binding():
    from flash_attention_train_amd import binding
    return binding


def _kslot_32(l, j, kper):
    return kper * (l // 32) + j


def _c_row_32(l, r):
    return 8 * (r // 4) + 4 * (l // 32) + (r % 4)


@pytest.mark.parametrize("kind,kper", [(0, 8), (2, 1)], ids=["32x32x16_bf16", "32x32x2_f32"])
def test_mfma_32x32_layouts(kind, kper):
    B = _binding()
    K = 2 * kper
    rng = np.random.default_rng(5 + kind)
    waves = 8
    A = rng.integers(-3, 4, size=(waves, 32, K)).astype(np.float32)
    Bm = rng.integers(-3, 4, size=(waves, K, 32)).astype(np.float32)
    a = np.zeros((waves, 64, kper), np.float32)
    b = np.zeros((waves, 64, kper), np.float32)
    for l in range(64):
        for j in range(kper):
            a[:, l, j] = A[:, l % 32, _kslot_32(l, j, kper)]
            b[:, l, j] = Bm[:, _kslot_32(l, j, kper), l % 32]
    c = _binding().probe_mfma(kind, torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()).cpu().numpy()
    C = np.einsum("wmk,wkn->wmn", A.astype(np.float64), Bm.astype(np.float64))
    want = np.zeros((waves, 64, 16))
    for l in range(64):
        for r in range(16):
            want[:, l, r] = C[:, _c_row_32(l, r), l % 32]
    if OUT:
        os.makedirs(OUT, exist_ok=True)
        with open(os.path.join(OUT, f"probe_mfma_kind{kind}.json"), "w") as f:
            json.dump({"c_wave0": c[0].tolist(), "want_wave0": want[0].tolist()}, f)
    say(f"mfma kind {kind}: max |c - want| = {np.abs(c - want).max()}")
    assert np.array_equal(c, want)


def test_mfma_16x16x32_bf16_layout():
    # A (16 x 32): lane l row l % 16, slot j -> k 8 (l // 16) + j; B likewise;
    # C: lane l, reg r -> (row 4 (l // 16) + r, col l % 16)
    rng = np.random.default_rng(9)
    waves = 4
    A = rng.integers(-3, 4, size=(waves, 16, 32)).astype(np.float32)
    Bm = rng.integers(-3, 4, size=(waves, 32, 16)).astype(np.float32)
    a = np.zeros((waves, 64, 8), np.float32)
    b = np.zeros((waves, 64, 8), np.float32)
    for l in range(64):
        for j in range(8):
            a[:, l, j] = A[:, l % 16, 8 * (l // 16) + j]
            b[:, l, j] = Bm[:, 8 * (l // 16) + j, l % 16]
    c = _binding().probe_mfma(1, torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()).cpu().numpy()
    C = np.einsum("wmk,wkn->wmn", A.astype(np.float64), Bm.astype(np.float64))
    want = np.zeros((waves, 64, 4))
    for l in range(64):
        for r in range(4):
            want[:, l, r] = C[:, 4 * (l // 16) + r, l % 16]
    say(f"mfma 16x16x32: max |c - want| = {np.abs(c - want).max()}")
    assert np.array_equal(c, want)


def test_ds_read_tr16_record():
    """Record the LDS transpose read's lane map for a few address patterns (LDS holds
    value i at 16-bit element i). Asserts only that each 16-lane group receives
    exactly the elements its own lanes addressed (a transpose moves data within
    the group) and that every result is in range."""
    patterns = {
        "linear": [8 * l for l in range(64)],                           # lane l -> elements 4l..4l+3
        "rows64": [128 * l for l in range(64)],                         # lane l -> row l of a [64][64] matrix
        "rows_by_group": [128 * (l % 16) + 8 * (l // 16) for l in range(64)],
        "quad_rows": [128 * (l % 4) + 8 * (l // 4) for l in range(64)],
    }
    addr = torch.tensor([patterns[k] for k in patterns], dtype=torch.int32).cuda()
    out = _binding().probe_ds_read_tr16(addr).cpu().numpy()
    if OUT:
        os.makedirs(OUT, exist_ok=True)
        rec = {k: {"addr": patterns[k], "out": out[i].tolist()} for i, k in enumerate(patterns)}
        with open(os.path.join(OUT, "probe_ds_read_tr16.json"), "w") as f:
            json.dump(rec, f)
    for i, k in enumerate(patterns):
        say(f"tr16 {k}: lanes 0..7 -> {out[i][:8].tolist()}")
    assert (out >= 0).all() and (out < 4096).all()
    for i, k in enumerate(patterns):
        for grp in range(4):
            lanes = range(16 * grp, 16 * grp + 16)
            loaded = sorted(e for l in lanes for e in range(patterns[k][l] // 2, patterns[k][l] // 2 + 4))
            got = sorted(out[i][16 * grp:16 * grp + 16].reshape(-1).tolist())
            assert got == loaded, (k, grp)
