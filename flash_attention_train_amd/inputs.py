"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This module holds no attention arithmetic. It only draws numbers and builds
additive masks, so both sides of every parity check start from the very same
stored values:

* every tensor is drawn with ``numpy.random.Generator(PCG64(seed))`` as float64
  standard normals, multiplied by its standard deviation and cast to float32;
* bf16 tensors are then rounded to nearest-even on the bit pattern (no library
  conversion is involved), and kept as ``uint16`` bit patterns;
* draw order is Q, K, V, dO, then whatever the mask needs.

Masks are additive fp32 arrays ``[Bm, Sq, Sk]`` (``Bm`` is 1 for a mask shared by
the batch), holding 0 where a key is open and ``-inf`` where it is masked. The two
mask families follow the pages' DiT trainer (Flash Attn Training skill page,
section 6, traps 8 and 9; HOT-Step TRAINING.md, the batching paragraph on
padded query rows):

* ``sa_pad``: self-attention padding. The last ~10 % of positions are padding;
  real query rows cannot see pad keys, pad query rows stay fully open, so no key
  column is ever fully masked.
* ``ca_keypad``: cross-attention key padding. Sample ``b`` keeps its first
  ``L_b`` encoder keys, ``L_b`` uniform on ``[lo, hi]``; on top of that a few query
  rows per sample are masked completely, which exercises the convention that a
  fully masked row yields O = 0 and LSE = 0.

Two test-only families: ``random`` (finite biases with ``-inf`` holes and a few fully
masked rows and columns) and ``blocks`` (64 x 64 blocks drawn whole as hidden, open,
0 / ``-inf`` or finite biases, so long walks cross every block class).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


# ----------------------------------------------------------------------------
# bf16 bit helpers (round to nearest even, no library dependence)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def stored_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored tensor (float32 array or bf16 bits)."""
    if dtype == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# the case record
# ----------------------------------------------------------------------------
@dataclass
class Case:
    """One attention problem: shapes, options and the stored input values.

    Tensors are contiguous ``[B, H, S, D]``; ``q``/``do`` have ``Hq`` heads and
    ``Sq`` rows, ``k``/``v`` have ``Hkv`` heads and ``Sk`` rows. For ``bf16`` the
    arrays hold uint16 bit patterns, for ``f32`` float32 values.
    """

    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    D: int
    dtype: str
    scale: float
    causal: bool
    q_offset: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray
    mask: Optional[np.ndarray] = None  # float32 [Bm, Sq, Sk] or None
    seed: int = 0
    meta: dict = field(default_factory=dict)

    def f64(self, which: str) -> np.ndarray:
        return stored_to_f64(getattr(self, which), self.dtype)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float64)
    if std != 1.0:
        x *= std
    return x.astype(np.float32)


def stored(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 values as a case stores them: bf16 bit patterns (nearest even) or fp32 itself."""
    return f32_to_bf16_bits(x) if dtype == BF16 else x


_store = stored


def sa_pad_mask(Sq: int, Sk: int, pad_frac: float = 0.1) -> tuple[np.ndarray, int]:
    """Self-attention pad mask [1, Sq, Sk]: rows i < L cannot see keys j >= L.

    ``L = S - round(pad_frac * S)`` with S = Sk. Rows i >= L (pad queries) stay
    fully open, so no key column is fully masked.
    """
    n_pad = int(round(pad_frac * Sk))
    L = Sk - n_pad
    m = np.zeros((1, Sq, Sk), dtype=np.float32)
    m[0, : min(L, Sq), L:] = -np.inf
    return m, L


def ca_keypad_mask(rng: np.random.Generator, B: int, Sq: int, Sk: int, lo: int, hi: int,
                   masked_rows: int) -> tuple[np.ndarray, list, list]:
    """Cross-attention key-pad mask [B, Sq, Sk] with a few fully masked rows per sample.

    ``L_b`` is uniform on the integers ``lo..hi`` inclusive; the fully masked rows
    are drawn without replacement, per sample, after all the lengths.
    """
    lens = [int(rng.integers(lo, hi + 1)) for _ in range(B)]
    rows = [sorted(int(r) for r in rng.choice(Sq, size=masked_rows, replace=False)) for _ in range(B)]
    m = np.zeros((B, Sq, Sk), dtype=np.float32)
    for b in range(B):
        m[b, :, lens[b]:] = -np.inf
        for r in rows[b]:
            m[b, r, :] = -np.inf
    return m, lens, rows


def random_bias_mask(rng: np.random.Generator, Bm: int, Sq: int, Sk: int, p_masked: float = 0.2,
                     bias_std: float = 1.0, full_rows: int = 1, full_cols: int = 1) -> np.ndarray:
    """A general additive mask: finite N(0, bias_std) biases, ``-inf`` holes, and
    (per batch entry) ``full_rows`` fully masked rows and ``full_cols`` fully masked columns."""
    bias = _normal(rng, (Bm, Sq, Sk), bias_std)
    holes = rng.random((Bm, Sq, Sk)) < p_masked
    bias[holes] = -np.inf
    for b in range(Bm):
        if full_rows:
            for r in rng.choice(Sq, size=min(full_rows, Sq), replace=False):
                bias[b, r, :] = -np.inf
        if full_cols:
            for c in rng.choice(Sk, size=min(full_cols, Sk), replace=False):
                bias[b, :, c] = -np.inf
    return bias


def block_mask(rng: np.random.Generator, Bm: int, Sq: int, Sk: int, block: int = 64,
               p: tuple = (0.3, 0.3, 0.2, 0.2)) -> np.ndarray:
    """A mask made of ``block`` x ``block`` blocks, each drawn as all -inf, all 0, a 0 / -inf
    pattern (half the entries hidden) or finite N(0, 1) biases with probabilities ``p``, so
    that every block class appears along long rows and columns."""
    m = np.zeros((Bm, Sq, Sk), dtype=np.float32)
    nrb, ncb = -(-Sq // block), -(-Sk // block)
    kinds = rng.choice(4, size=(Bm, nrb, ncb), p=np.asarray(p, dtype=np.float64))
    for b in range(Bm):
        for i in range(nrb):
            for j in range(ncb):
                r0, c0 = i * block, j * block
                blk = m[b, r0:r0 + block, c0:c0 + block]
                if kinds[b, i, j] == 0:
                    blk[...] = -np.inf
                elif kinds[b, i, j] == 2:
                    blk[rng.random(blk.shape) < 0.5] = -np.inf
                elif kinds[b, i, j] == 3:
                    blk[...] = _normal(rng, blk.shape)
    return m


def sink_logits(seed: int, Hq: int, std: float = 1.0) -> np.ndarray:
    """Seeded per-head attention-sink logits, float32 [Hq], N(0, std^2): drawn from their
    own generator stream (seed + 7919), so that adding sinks to a case changes none of its
    other inputs."""
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    return (std * rng.standard_normal(Hq)).astype(np.float32)


def alibi_slopes(H: int) -> np.ndarray:
    """The usual ALiBi slopes for H heads, 2^(-8 (h + 1) / H), float32 [H]."""
    return (2.0 ** (-8.0 * np.arange(1, H + 1) / H)).astype(np.float32)


def quantize_q8_0(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Store a [..., D] array the way a q8_0 K/V cache holds it (ggml's q8_0 block: 32
    consecutive values share one fp16 scale d = max|x| / 127, each value kept as the int8
    q = round(x / d), halves away from zero). Returns (qs int8 [..., D], d float16
    [..., D / 32]); the stored value is d * q. This prepares inputs: the cache arrives
    quantized, and the op and its checker both start from (qs, d)."""
    x = np.asarray(x, np.float32)
    D = x.shape[-1]
    if D % 32:
        raise ValueError("q8_0 blocks need D to be a multiple of 32")
    xb = x.reshape(*x.shape[:-1], D // 32, 32)
    d = np.abs(xb).max(axis=-1) / np.float32(127)
    inv = np.where(d > 0, np.float32(1) / np.where(d > 0, d, 1), 0).astype(np.float32)
    v = xb * inv[..., None]
    q = np.trunc(v + np.copysign(np.float32(0.5), v))
    qs = np.clip(q, -127, 127).astype(np.int8).reshape(x.shape)
    return qs, d.astype(np.float16)


def make_case(name: str, *, B: int, Hq: int, Hkv: int, Sq: int, Sk: int, D: int, dtype: str,
              seed: int, causal: bool = False, q_offset: Optional[int] = None, do_std: float = 1.0,
              mask: str = "none", mask_args: Optional[dict] = None, scale: Optional[float] = None) -> Case:
    """Draw one seeded case. ``mask`` is one of none | sa_pad | ca_keypad | random | blocks."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _store(_normal(rng, (B, Hq, Sq, D)), dtype)
    k = _store(_normal(rng, (B, Hkv, Sk, D)), dtype)
    v = _store(_normal(rng, (B, Hkv, Sk, D)), dtype)
    do = _store(_normal(rng, (B, Hq, Sq, D), do_std), dtype)
    mask_args = dict(mask_args or {})
    meta: dict = {"mask_kind": mask}
    m = None
    if mask == "sa_pad":
        m, L = sa_pad_mask(Sq, Sk, mask_args.get("pad_frac", 0.1))
        meta["valid_len"] = L
    elif mask == "ca_keypad":
        m, lens, rows = ca_keypad_mask(rng, B, Sq, Sk, mask_args.get("lo", 128), mask_args.get("hi", 512),
                                       mask_args.get("masked_rows", 2))
        meta["valid_lens"] = lens
        meta["masked_rows"] = rows
    elif mask == "random":
        m = random_bias_mask(rng, mask_args.get("Bm", B), Sq, Sk, mask_args.get("p_masked", 0.2),
                             mask_args.get("bias_std", 1.0), mask_args.get("full_rows", 1),
                             mask_args.get("full_cols", 1))
    elif mask == "blocks":
        m = block_mask(rng, mask_args.get("Bm", B), Sq, Sk)
    elif mask != "none":
        raise ValueError(f"unknown mask kind {mask!r}")
    if q_offset is None:
        q_offset = Sk - Sq if causal else 0
    if scale is None:
        scale = 1.0 / float(np.sqrt(D))
    return Case(name=name, B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D, dtype=dtype, scale=float(scale),
                causal=bool(causal), q_offset=int(q_offset), q=q, k=k, v=v, do=do, mask=m, seed=seed,
                meta=meta)
