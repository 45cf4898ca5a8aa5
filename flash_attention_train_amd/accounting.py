"""Work and traffic accounting: unmasked score pairs, FLOPs, algorithmic bytes.

The FLOP convention counts only the score entries a result depends on (the
mask-adjusted count N of unmasked (b, h, i, j) entries): the forward does two
D-long products per entry (QK^T and PV, 4*D*N FLOPs) and the backward five
(the QK^T recompute, dO V^T, P^T dO, dS^T Q and dS K: 10*D*N FLOPs). Masked work a
kernel skips is not counted, and masked work a kernel does anyway is not counted
either.
"""
from __future__ import annotations

import numpy as np

from .inputs import BF16, Case

MI355X_BF16_DENSE_TFLOPS = 2516.6  # 256 CU x 4096 FLOP/clk x 2.4 GHz (dense, no sparsity)
MI355X_FP32_MFMA_TFLOPS = 157.3
MI355X_HBM_GBS = 8000.0


def visible_counts(Sq: int, Sk: int, causal: bool, q_offset: int, mask_b: np.ndarray | None) -> np.ndarray:
    """Number of visible keys for each query row of one batch entry (shape [Sq])."""
    if mask_b is not None:
        vis = np.isfinite(mask_b)
        if causal:
            j = np.arange(Sk)[None, :]
            i = np.arange(Sq)[:, None]
            vis &= j <= (q_offset + i)
        return vis.sum(axis=1).astype(np.int64)
    if causal:
        c = np.arange(Sq, dtype=np.int64) + q_offset + 1
        return np.clip(c, 0, Sk)
    return np.full(Sq, Sk, dtype=np.int64)


def unmasked_pairs(B: int, Hq: int, Sq: int, Sk: int, causal: bool, q_offset: int,
                   mask: np.ndarray | None) -> int:
    total = 0
    for b in range(B):
        mb = None
        if mask is not None:
            mb = mask[b if mask.shape[0] > 1 else 0]
        total += int(visible_counts(Sq, Sk, causal, q_offset, mb).sum())
    return total * Hq


def structured_counts(Sq: int, Sk: int, causal: bool, q_offset: int, key_len: int, q_len: int, window_left: int,
                      window_right: int) -> np.ndarray:
    """Visible keys per query row of one batch entry under a structured mask: row i
    (i < q_len) sees the keys j with max(0, pos - window_left) <= j < min(key_len,
    pos + 1 if causal, pos + window_right + 1), pos = q_offset + i (a bound of -1 is absent)."""
    pos = q_offset + np.arange(Sq, dtype=np.int64)
    lo = np.maximum(pos - window_left, 0) if window_left >= 0 else np.zeros(Sq, np.int64)
    hi = np.full(Sq, min(key_len, Sk), np.int64)
    if causal:
        hi = np.minimum(hi, pos + 1)
    if window_right >= 0:
        hi = np.minimum(hi, pos + window_right + 1)
    n = np.maximum(hi - lo, 0)
    n[q_len:] = 0
    return n


def case_pairs(c: Case) -> int:
    st = c.meta.get("structure")
    if st is None:
        return unmasked_pairs(c.B, c.Hq, c.Sq, c.Sk, c.causal, c.q_offset, c.mask)
    if c.mask is not None:
        raise ValueError("pair counts of a structured case with a dense mask are not defined here")
    total = 0
    for b in range(c.B):
        kl = c.Sk if st["key_len"] is None else int(st["key_len"][b])
        ql = c.Sq if st["q_len"] is None else int(st["q_len"][b])
        total += int(structured_counts(c.Sq, c.Sk, c.causal, c.q_offset, kl, ql, *st["window"]).sum())
    return total * c.Hq


def fwd_flops(n_pairs: int, D: int) -> float:
    return 4.0 * D * n_pairs


def bwd_flops(n_pairs: int, D: int) -> float:
    return 10.0 * D * n_pairs


def elt_bytes(dtype: str) -> int:
    return 2 if dtype == BF16 else 4


def preprocess_bytes(B: int, Hq: int, Sq: int, D: int, dtype: str) -> int:
    """Algorithmic bytes of Delta = rowsum(dO * O): read O and dO, write Delta (fp32)."""
    return 2 * B * Hq * Sq * D * elt_bytes(dtype) + 4 * B * Hq * Sq


def chunked_pairs(Hq: int, W: int, chunk: int) -> int:
    """Unmasked pairs of the causal walk over a W-long window in chunks (equals one-shot causal)."""
    return Hq * sum(int(np.clip(np.arange(chunk) + p0 + 1, 0, p0 + chunk).sum())
                    for p0 in range(0, W, chunk))


def step_bytes(c: Case, mask_passes: int = 3) -> int:
    """Algorithmic HBM bytes of one training step of the op as it is split into passes:
    the forward reads Q, K, V and writes O and the LSE; the preprocess reads O and dO and
    writes Delta; the backward reads Q, K, V, dO, the LSE and Delta and writes dQ, dK and
    dV. A dense mask is read once by each of `mask_passes` passes (the block map, the
    forward, the backward). Each tensor counts once per pass that needs it; nothing a
    kernel re-reads counts twice."""
    e = elt_bytes(c.dtype)
    q = c.B * c.Hq * c.Sq * c.D * e
    kv = c.B * c.Hkv * c.Sk * c.D * e
    row = 4 * c.B * c.Hq * c.Sq
    mask = 0 if c.mask is None else int(np.prod(c.mask.shape)) * 4
    fwd = q + 2 * kv + q + row
    pre = 2 * q + row
    bwd = q + 2 * kv + q + 2 * row + q + 2 * kv
    return int(fwd + pre + bwd + mask_passes * mask)
