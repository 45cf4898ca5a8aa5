"""CPU oracle for softmax attention with an LSE side output and its gradient.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package's smoke check and the
bench's ``cpu_baseline`` leg may import this module; the op never does. It is a
plain float64 C implementation (``fa_oracle.c``) that materialises every score
row, plus this thin ctypes wrapper. It shares no code with the HIP library.

Every function takes float64 arrays in contiguous ``[B, H, S, D]`` layout and an
optional additive mask ``[Bm, Sq, Sk]`` or ``[Bm, Hm, Sq, Sk]`` (``Bm`` 1 or B, ``Hm`` 1
or Hq: a score bias per head; ``-inf`` = masked).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
_LIB = os.path.join(_HERE, "libfa_oracle.so")


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math: sums keep their order)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-fPIC", "-shared",
                        "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm", "-lpthread"],
                       check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("Sq", ctypes.c_int32), ("Sk", ctypes.c_int32), ("D", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("mask_b", ctypes.c_int32),
                ("q_offset", ctypes.c_int64), ("scale", ctypes.c_double), ("sinks", ctypes.c_void_p),
                ("alibi", ctypes.c_void_p), ("mask_h", ctypes.c_int32), ("softcap", ctypes.c_double)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int64)
        pp = ctypes.POINTER(_Problem)
        _lib.ora_forward.argtypes = [pp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
        _lib.ora_backward.argtypes = [pp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
        _lib.ora_rows.argtypes = [pp, dp, dp, dp, dp, dp, ctypes.c_int64, ip, dp, dp, dp, dp, ctypes.c_int]
        _lib.ora_cols.argtypes = [pp, dp, dp, dp, dp, dp, ctypes.c_int64, ip, dp, dp, ctypes.c_int]
        _lib.ora_score_grad.argtypes = [pp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
        for f in (_lib.ora_forward, _lib.ora_backward, _lib.ora_rows, _lib.ora_cols, _lib.ora_score_grad):
            f.restype = ctypes.c_int
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _problem(q, k, mask, scale, causal, q_offset, sinks=None, alibi=None, softcap=None):
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, _ = k.shape
    if q_offset is None:
        q_offset = Sk - Sq if causal else 0
    mb = 0 if mask is None else int(mask.shape[0])
    mh = 0
    if mask is not None:
        if mask.ndim == 4:  # [Bm, Hm, Sq, Sk]: Hm = 1 (every head) or Hq (a bias per head)
            mh = int(mask.shape[1])
            if mh not in (1, Hq):
                raise ValueError("a 4-D mask must have 1 or Hq heads")
        if tuple(mask.shape[-2:]) != (Sq, Sk) or mask.ndim not in (3, 4):
            raise ValueError("mask must be [Bm, Sq, Sk] or [Bm, Hm, Sq, Sk]")
    if sinks is not None and sinks.shape != (Hq,):
        raise ValueError("sinks must be [Hq]")
    if alibi is not None and alibi.shape != (Hq,):
        raise ValueError("alibi must be [Hq]")
    return _Problem(B, Hq, Hkv, Sq, Sk, D, int(bool(causal)), mb, int(q_offset), float(scale),
                    None if sinks is None else sinks.ctypes.data, None if alibi is None else alibi.ctypes.data, mh,
                    float(softcap or 0.0))


def forward(q, k, v, mask=None, *, scale: float, causal: bool = False, q_offset: Optional[int] = None,
            threads: Optional[int] = None, sinks=None, alibi=None, softcap: Optional[float] = None):
    """Returns (O [B,Hq,Sq,D], LSE [B,Hq,Sq]) in float64. ``sinks``: optional [Hq] sink logits;
    ``alibi``: optional [Hq] ALiBi slopes; ``softcap``: optional logit softcap c > 0."""
    q, k, v, mask, sinks, alibi = _f64(q), _f64(k), _f64(v), _f64(mask), _f64(sinks), _f64(alibi)
    p = _problem(q, k, mask, scale, causal, q_offset, sinks, alibi, softcap)
    O = np.zeros(q.shape, np.float64)
    L = np.zeros(q.shape[:3], np.float64)
    rc = _load().ora_forward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(mask), _ptr(O), _ptr(L),
                             threads or default_threads())
    if rc:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    return O, L


def backward(q, k, v, do, mask=None, *, scale: float, causal: bool = False, q_offset: Optional[int] = None,
             threads: Optional[int] = None, sinks=None, alibi=None, softcap: Optional[float] = None) -> dict:
    """The full forward and backward. Returns a dict with O, LSE, Delta, dQ, dK, dV (float64), and
    dSink [Hq] when ``sinks`` ([Hq] sink logits) is given. ``alibi``: optional [Hq] ALiBi slopes;
    ``softcap``: optional logit softcap c > 0."""
    q, k, v, do, mask, sinks, alibi = _f64(q), _f64(k), _f64(v), _f64(do), _f64(mask), _f64(sinks), _f64(alibi)
    p = _problem(q, k, mask, scale, causal, q_offset, sinks, alibi, softcap)
    out = {"O": np.zeros(q.shape), "LSE": np.zeros(q.shape[:3]), "Delta": np.zeros(q.shape[:3]),
           "dQ": np.zeros(q.shape), "dK": np.zeros(k.shape), "dV": np.zeros(k.shape)}
    rc = _load().ora_backward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(mask), _ptr(do),
                              *(_ptr(out[n]) for n in ("O", "LSE", "Delta", "dQ", "dK", "dV")),
                              threads or default_threads())
    if rc:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    if sinks is not None:
        out["dSink"] = sink_grad(sinks, out["LSE"], out["Delta"])
    return out


def bias_grad(q, k, v, do, mask, *, scale: float, causal: bool = False, q_offset: Optional[int] = None,
              threads: Optional[int] = None, sinks=None, alibi=None, softcap: Optional[float] = None) -> np.ndarray:
    """Gradient of L = <O, dO> with respect to the additive mask, shaped like the mask: each
    score's dM = P (dP - Delta) (the mask is added after the cap, so no cap' factor; 0 where an
    entry is hidden), summed over the batch entries / heads the mask is broadcast over."""
    q, k, v, do, mask, sinks, alibi = _f64(q), _f64(k), _f64(v), _f64(do), _f64(mask), _f64(sinks), _f64(alibi)
    if mask is None:
        raise ValueError("bias_grad needs the mask it differentiates")
    p = _problem(q, k, mask, scale, causal, q_offset, sinks, alibi, softcap)
    B, Hq, Sq, _ = q.shape
    Sk = k.shape[2]
    dm = np.zeros((B, Hq, Sq, Sk), np.float64)
    rc = _load().ora_score_grad(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(mask), _ptr(do), _ptr(dm),
                                threads or default_threads())
    if rc:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    if mask.ndim == 3:  # shared by the heads
        dm = dm.sum(axis=1)
    elif mask.shape[1] == 1:
        dm = dm.sum(axis=1, keepdims=True)
    if mask.shape[0] == 1 and B > 1:  # shared by the batch
        dm = dm.sum(axis=0, keepdims=True)
    return dm


def sink_grad(sinks, lse, delta) -> np.ndarray:
    """Gradient of the loss with respect to each head's sink logit: the sink is one more softmax
    column with no value row, so its dS is P_sink (0 - Delta_i) with P_sink = exp(sink_h - LSE_i),
    summed over every row of the head (all batches): dSink_h = -sum_{b,i} exp(sink_h - LSE_bhi) Delta_bhi.
    A fully masked row without a sink has no sink term; with one, its O is 0 and so is its Delta."""
    sinks = np.asarray(sinks, np.float64)
    lse = np.asarray(lse, np.float64)
    delta = np.asarray(delta, np.float64)
    out = np.zeros(sinks.shape[0])
    for h in range(sinks.shape[0]):
        out[h] = -np.sum(np.exp(sinks[h] - lse[:, h, :]) * delta[:, h, :])
    return out


def rows(q, k, v, do, row_ids, mask=None, *, scale: float, causal: bool = False,
         q_offset: Optional[int] = None, threads: Optional[int] = None, sinks=None, alibi=None,
         softcap: Optional[float] = None) -> dict:
    """Selected rows, ids (b*Hq + h)*Sq + i. Returns O [n,D], LSE [n], Delta [n], dQ [n,D]."""
    q, k, v, do, mask, sinks, alibi = _f64(q), _f64(k), _f64(v), _f64(do), _f64(mask), _f64(sinks), _f64(alibi)
    p = _problem(q, k, mask, scale, causal, q_offset, sinks, alibi, softcap)
    ids = np.ascontiguousarray(row_ids, dtype=np.int64)
    n, D = ids.size, q.shape[3]
    out = {"O": np.zeros((n, D)), "LSE": np.zeros(n), "Delta": np.zeros(n), "dQ": np.zeros((n, D))}
    rc = _load().ora_rows(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(mask), _ptr(do), n,
                          ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                          *(_ptr(out[x]) for x in ("O", "LSE", "Delta", "dQ")), threads or default_threads())
    if rc:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    return out


def cols(q, k, v, do, col_ids, mask=None, *, scale: float, causal: bool = False,
         q_offset: Optional[int] = None, threads: Optional[int] = None, sinks=None, alibi=None,
         softcap: Optional[float] = None) -> dict:
    """Selected key columns, ids (b*Hkv + g)*Sk + j. Returns dK [n,D], dV [n,D]."""
    q, k, v, do, mask, sinks, alibi = _f64(q), _f64(k), _f64(v), _f64(do), _f64(mask), _f64(sinks), _f64(alibi)
    p = _problem(q, k, mask, scale, causal, q_offset, sinks, alibi, softcap)
    ids = np.ascontiguousarray(col_ids, dtype=np.int64)
    n, D = ids.size, q.shape[3]
    out = {"dK": np.zeros((n, D)), "dV": np.zeros((n, D))}
    rc = _load().ora_cols(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(mask), _ptr(do), n,
                          ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                          _ptr(out["dK"]), _ptr(out["dV"]), threads or default_threads())
    if rc:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    return out


def dequant_q8_0(qs, d) -> np.ndarray:
    """The values a q8_0 K/V window holds (llama.cpp pull request 57 trains such a quantised cache in
    place): blocks of 32 consecutive values along the head dimension share one fp16 scale, and value
    t of block b is d[b] * qs[32 b + t]. qs: int8 [..., D]; d: float16 [..., D / 32]; float64 out."""
    qs = np.asarray(qs)
    d = np.asarray(d)
    D = qs.shape[-1]
    out = np.empty(qs.shape, np.float64)
    for b in range(D // 32):
        out[..., 32 * b:32 * (b + 1)] = d[..., b:b + 1].astype(np.float64) * qs[..., 32 * b:32 * (b + 1)]
    return out


def structured_mask(B: int, Sq: int, Sk: int, *, key_len=None, q_len=None, window_left: int = -1,
                    window_right: int = -1, q_offset: int = 0, causal: bool = False) -> np.ndarray:
    """The dense additive mask [B, Sq, Sk] (0 / -inf) of a structured mask, entry by entry:
    (b, i, j) is hidden when j >= key_len[b], when i >= q_len[b] (the whole row, which is
    then fully masked), when window_left >= 0 and j < q_offset + i - window_left, when
    window_right >= 0 and j > q_offset + i + window_right, or (causal) when j > q_offset + i.

    This is the reading of the pages' DiT batch masks ("sa" = sliding window + padded key
    columns, "sa_pad" = padded key columns) with the window as a band of explicit width on
    each side of a row's position; the pages give no width. The result feeds forward() /
    backward() like any dense mask."""
    m = np.zeros((B, Sq, Sk), np.float64)
    i = np.arange(Sq)[:, None]
    j = np.arange(Sk)[None, :]
    pos = q_offset + i
    hidden = np.zeros((Sq, Sk), bool)
    if window_left >= 0:
        hidden |= j < pos - window_left
    if window_right >= 0:
        hidden |= j > pos + window_right
    if causal:
        hidden |= j > pos
    for b in range(B):
        h = hidden.copy()
        if key_len is not None:
            h |= j >= int(key_len[b])
        if q_len is not None:
            h |= np.broadcast_to(i >= int(q_len[b]), (Sq, Sk))
        m[b][h] = -np.inf
    return m
