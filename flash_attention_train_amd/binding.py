"""Python binding over the C ABI in ``include/fa_train.h`` (argument marshalling only).

PyTorch provides device memory and the stream; every step of the op runs in the
HIP kernels of ``libfa_train.so``. There is no CPU or PyTorch fallback: if the
library is missing or a call fails, an exception says so.

Tensors are ``[B, H, S, D]`` views with the last dimension contiguous (any batch,
head and sequence strides that are multiples of 16 bytes). LSE and Delta are
fp32 ``[B, Hq, S]`` with a contiguous last dimension.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa_train.so")

FA_F32, FA_BF16 = 0, 1
FA_KV_DTYPE, FA_KV_F16, FA_KV_Q8_0 = 0, 1, 2


class FaView(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
                ("stride_s", ctypes.c_int64)]


class FaAttnParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("Sq", ctypes.c_int32),
                ("Sk", ctypes.c_int32), ("D", ctypes.c_int32), ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("q_offset", ctypes.c_int64), ("scale", ctypes.c_float), ("mask", ctypes.c_void_p),
                ("mask_stride_b", ctypes.c_int64), ("mask_stride_q", ctypes.c_int64), ("mask_tiles", ctypes.c_void_p),
                ("fwd_variant", ctypes.c_int32), ("kv_split", ctypes.c_int32), ("q_split", ctypes.c_int32),
                ("fwd_split", ctypes.c_int32), ("key_len", ctypes.c_void_p), ("q_len", ctypes.c_void_p),
                ("window_left", ctypes.c_int32), ("window_right", ctypes.c_int32),
                ("bwd_dq_launch", ctypes.c_int32), ("sinks", ctypes.c_void_p), ("alibi", ctypes.c_void_p),
                ("q_split_tiles", ctypes.c_int32), ("mask_stride_h", ctypes.c_int64), ("softcap", ctypes.c_float),
                ("bwd_kv_walk", ctypes.c_int32), ("kv_format", ctypes.c_int32), ("k_scale", FaView),
                ("v_scale", FaView), ("dbias", ctypes.c_void_p), ("dbias_stride_b", ctypes.c_int64),
                ("dbias_stride_h", ctypes.c_int64), ("dbias_stride_q", ctypes.c_int64)]


class FaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed with status {status}: {detail}")
        self.status = status


_lib = None

# exported symbol -> (argtypes, restype)
_VP = ctypes.c_void_p
_PV = ctypes.POINTER(FaView)
_PP = ctypes.POINTER(FaAttnParams)
SIGNATURES = {
    "fa_train_fwd": ([_PP, _PV, _PV, _PV, _PV, _PV, _VP], ctypes.c_int),
    "fa_train_fwd_workspace_bytes": ([_PP], ctypes.c_size_t),
    "fa_train_fwd_ws": ([_PP, _PV, _PV, _PV, _PV, _PV, _VP, ctypes.c_size_t, _VP], ctypes.c_int),
    "fa_train_bwd_preprocess": ([_PP, _PV, _PV, _PV, _VP], ctypes.c_int),
    "fa_train_bwd_workspace_bytes": ([_PP], ctypes.c_size_t),
    "fa_train_bwd": ([_PP, _PV, _PV, _PV, _PV, _PV, _PV, _PV, _PV, _PV, _VP, ctypes.c_size_t, _VP], ctypes.c_int),
    "fa_train_bwd_chunked": ([_PP, _PV, _PV, _PV, _PV, _PV, _PV, _PV, _PV, _PV, _VP, ctypes.c_size_t, _VP],
                             ctypes.c_int),
    "fa_train_bwd_noalloc": ([_PP, _PV, _PV, _PV, _PV, _PV, _PV, _PV, _PV, _PV, _VP], ctypes.c_int),
    "fa_train_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "fa_train_last_error": ([], ctypes.c_char_p),
    "fa_train_version": ([], ctypes.c_int),
    "fa_train_mask_tiles_bytes": ([_PP], ctypes.c_size_t),
    "fa_train_mask_tiles": ([_PP, _VP, _VP], ctypes.c_int),
    "fa_train_bwd_sinks": ([_PP, _PV, _PV, _VP, _VP], ctypes.c_int),
    "fa_train_dequant_q8_0": ([ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _PV, _PV, _PV, _VP],
                              ctypes.c_int),
    "fa_train_convert_f16": ([ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _PV, _PV,
                              ctypes.c_int32, _VP], ctypes.c_int),
    "fa_train_probe_mfma": ([ctypes.c_int32, ctypes.c_int32, _VP, _VP, _VP, _VP], ctypes.c_int),
    "fa_train_probe_ds_read_tr16": ([ctypes.c_int32, _VP, _VP, _VP], ctypes.c_int),
}


def library_path() -> str:
    return LIB_PATH


def lib():
    """Load libfa_train.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m flash_attention_train_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (argt, rest) in SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes = argt
            f.restype = rest
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise FaError(fn, status, lib().fa_train_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def view4(t: torch.Tensor) -> FaView:
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B, H, S, D] tensor with a contiguous last dimension")
    return FaView(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def view3(t: torch.Tensor) -> FaView:
    if t.dim() != 3 or t.dtype != torch.float32:
        raise ValueError("expected an fp32 [B, H, S] tensor")
    return FaView(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _expect(name: str, t, *, dtype=None, shape=None) -> None:
    """Type, dtype and shape of one tensor argument. The C ABI takes bare pointers and
    cannot see a tensor's size, type or residency, so a short or mistyped tensor would
    reach the kernels as an out-of-bounds address: every entry point checks its
    arguments here, then their residency (`_resident`), before any launch."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _resident(device, **named) -> None:
    """Every given tensor (None skipped) is device memory on `device`."""
    for name, t in named.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor (it is on {t.device})")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, the other operands on {device}")


def _check_qkv(q, k, v, k_scale=None, v_scale=None) -> None:
    """q [B, Hq, Sq, D] in bf16 or fp32; k and v [B, Hkv, Sk, D] in q's dtype, or (bf16 q) a
    K/V window stored in place: fp16 values, or q8_0 int8 quants with fp16 scale planes
    k_scale / v_scale [B, Hkv, Sk, D / 32]."""
    _expect("q", q, dtype=(torch.bfloat16, torch.float32))
    if q.dim() != 4:
        raise ValueError("q must be [B, Hq, Sq, D]")
    stored = (torch.float16, torch.int8) if q.dtype == torch.bfloat16 else ()
    _expect("k", k, dtype=(q.dtype,) + stored)
    if k.dim() != 4 or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise ValueError(f"k has shape {tuple(k.shape)}, expected [B={q.shape[0]}, Hkv, Sk, D={q.shape[3]}]")
    _expect("v", v, dtype=k.dtype, shape=k.shape)
    if k.dtype == torch.int8:
        if k_scale is None or v_scale is None:
            raise ValueError("a q8_0 K/V window needs k_scale and v_scale")
        B, H, S, D = k.shape
        _expect("k_scale", k_scale, dtype=torch.float16, shape=(B, H, S, D // 32))
        _expect("v_scale", v_scale, dtype=torch.float16, shape=(B, H, S, D // 32))
    elif k_scale is not None or v_scale is not None:
        raise ValueError("k_scale / v_scale belong to an int8 (q8_0) K/V window")


def _check_rowstats(q, **named) -> None:
    """fp32 [B, Hq, Sq] row statistics (LSE, Delta) beside q."""
    for name, t in named.items():
        _expect(name, t, dtype=torch.float32, shape=q.shape[:3])


def _stream_handle(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def make_params(q: torch.Tensor, k: torch.Tensor, *, scale: Optional[float], causal: bool,
                q_offset: Optional[int], mask: Optional[torch.Tensor], fwd_variant: int = 0, kv_split: int = 0,
                q_split: int = 0, mask_tiles: Optional[torch.Tensor] = None, fwd_split: int = 0,
                key_len: Optional[torch.Tensor] = None, q_len: Optional[torch.Tensor] = None,
                window: tuple = (-1, -1), dq_launch: int = 0,
                sinks: Optional[torch.Tensor] = None, alibi: Optional[torch.Tensor] = None,
                q_split_tiles: int = 0, softcap: float = 0.0, kv_walk: int = 0,
                k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                dbias: Optional[torch.Tensor] = None) -> FaAttnParams:
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Sk, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError("q and k disagree on B or D")
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    if q_offset is None:
        q_offset = Sk - Sq if causal else 0
    p = FaAttnParams(B, Hq, Hkv, Sq, Sk, D, _dtype_code(q), int(bool(causal)), int(q_offset), float(scale),
                     None, 0, 0, None, int(fwd_variant), int(kv_split), int(q_split), int(fwd_split), None, None,
                     int(window[0]), int(window[1]), int(dq_launch))
    for name, t, n in (("key_len", key_len, B), ("q_len", q_len, B)):
        if t is not None:
            if t.dtype != torch.int32 or t.dim() != 1 or t.shape[0] != n or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous int32 [B] tensor on the device")
            setattr(p, name, t.data_ptr())
    p.q_split_tiles = int(q_split_tiles)
    p.softcap = float(softcap)
    p.bwd_kv_walk = int(kv_walk)
    p.kv_format = {torch.float16: FA_KV_F16, torch.int8: FA_KV_Q8_0}.get(k.dtype, FA_KV_DTYPE)
    if p.kv_format == FA_KV_Q8_0:
        if k_scale is None or v_scale is None:
            raise ValueError("a q8_0 K/V window needs k_scale and v_scale")
        p.k_scale = view4(k_scale)
        p.v_scale = view4(v_scale)
    for name, t in (("sinks", sinks), ("alibi", alibi)):
        if t is not None:
            if t.dtype != torch.float32 or t.shape != (Hq,) or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous fp32 [Hq] tensor on the device")
            setattr(p, name, t.data_ptr())
    if mask is not None:
        if mask.dtype != torch.float32 or mask.dim() not in (3, 4) or mask.stride(-1) != 1:
            raise ValueError("mask must be an fp32 [Bm, Sq, Sk] or [Bm, Hm, Sq, Sk] tensor with a contiguous last "
                             "dimension")
        if mask.dim() == 4 and mask.shape[1] not in (1, Hq):
            raise ValueError("a per-head mask must have 1 or Hq heads")
        if mask.shape[-2] != Sq or mask.shape[-1] != Sk or mask.shape[0] not in (1, B):
            raise ValueError("mask must be [1 or B, (1 or Hq,) Sq, Sk]")
        p.mask = mask.data_ptr()
        p.mask_stride_b = 0 if mask.shape[0] == 1 else mask.stride(0)
        p.mask_stride_q = mask.stride(-2)
        p.mask_stride_h = mask.stride(1) if mask.dim() == 4 and mask.shape[1] > 1 else 0
        if mask_tiles is not None:
            if mask_tiles.dtype != torch.uint8 or not mask_tiles.is_contiguous():
                raise ValueError("mask_tiles must be a contiguous uint8 tensor from mask_tile_map()")
            need = int(lib().fa_train_mask_tiles_bytes(ctypes.byref(p)))
            if mask_tiles.numel() < need:
                raise ValueError(f"mask_tiles holds {mask_tiles.numel()} bytes; this mask's map needs {need}")
            p.mask_tiles = mask_tiles.data_ptr()
    elif mask_tiles is not None:
        raise ValueError("mask_tiles given without a mask")
    if dbias is not None:  # the mask's gradient: the mask's shape and broadcast
        if mask is None:
            raise ValueError("dbias is the gradient of the mask: pass the mask")
        if dbias.dtype != torch.float32 or tuple(dbias.shape) != tuple(mask.shape) or dbias.stride(-1) != 1:
            raise ValueError("dbias must be an fp32 tensor of the mask's shape with a contiguous last dimension")
        p.dbias = dbias.data_ptr()
        p.dbias_stride_b = 0 if dbias.shape[0] == 1 else dbias.stride(0)
        p.dbias_stride_q = dbias.stride(-2)
        p.dbias_stride_h = dbias.stride(1) if dbias.dim() == 4 and dbias.shape[1] > 1 else 0
    return p


def mask_tile_map(mask: torch.Tensor, q: torch.Tensor, k: torch.Tensor, *, stream=None,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Classify every 64 x 64 block of an additive mask (0 dead, 1 open, 2 visibility bits,
    3 finite biases) and record its visibility bits, for reuse by fwd/bwd/bwd_chunked
    through their ``mask_tiles`` argument. The first ``mask_tile_count`` bytes are the classes.
    ``out`` (uint8, at least the map's size) is filled instead of a new tensor."""
    p = make_params(q, k, scale=None, causal=False, q_offset=0, mask=mask)
    _resident(q.device, q=q, k=k, mask=mask)
    n = int(lib().fa_train_mask_tiles_bytes(ctypes.byref(p)))
    if out is not None:
        if out.dtype != torch.uint8 or not out.is_contiguous() or out.numel() < n:
            raise ValueError(f"out must be a contiguous uint8 tensor of at least {n} bytes")
        _resident(q.device, out=out)
        tiles = out
    else:
        tiles = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    _check("fa_train_mask_tiles",
           lib().fa_train_mask_tiles(ctypes.byref(p), tiles.data_ptr(), _stream_handle(stream)))
    return tiles


def mask_tile_count(mask: torch.Tensor) -> int:
    """Number of 64 x 64 blocks (and class bytes) of a [Bm, Sq, Sk] mask."""
    Bm, Sq, Sk = mask.shape
    return Bm * ((Sq + 63) // 64) * ((Sk + 63) // 64)


def fwd_workspace_bytes(q, k, *, scale=None, causal=False, q_offset=None, mask=None, split=0, key_len=None,
                        q_len=None, window=(-1, -1), softcap=0.0, k_scale=None, v_scale=None) -> int:
    p = make_params(q, k, scale=scale, causal=causal, q_offset=q_offset, mask=mask, fwd_split=split,
                    key_len=key_len, q_len=q_len, window=window, softcap=softcap, k_scale=k_scale, v_scale=v_scale)
    return int(lib().fa_train_fwd_workspace_bytes(ctypes.byref(p)))


def fwd(q, k, v, *, mask=None, scale=None, causal=False, q_offset=None, out=None, lse=None, stream=None,
        variant=0, mask_tiles=None, workspace=None, split=0, key_len=None, q_len=None, window=(-1, -1),
        sinks=None, alibi=None, softcap=0.0, k_scale=None, v_scale=None):
    """Forward: returns (O, LSE). O has q's dtype and shape; LSE is fp32 [B, Hq, Sq].
    Runs fa_train_fwd_ws: a short grid may split the key walks (split = 0: the library's
    choice; 1: never), with `workspace` (allocated here when None and needed). ``sinks``:
    optional fp32 [Hq] attention-sink logits; ``alibi``: fp32 [Hq] slopes; ``softcap``: a
    logit softcap c > 0 (0 = none)."""
    _check_qkv(q, k, v, k_scale, v_scale)
    p = make_params(q, k, scale=scale, causal=causal, q_offset=q_offset, mask=mask, fwd_variant=variant,
                    mask_tiles=mask_tiles, fwd_split=split, key_len=key_len, q_len=q_len, window=window,
                    sinks=sinks, alibi=alibi, softcap=softcap, k_scale=k_scale, v_scale=v_scale)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _expect("out", out, dtype=q.dtype, shape=q.shape)
    _check_rowstats(q, lse=lse)
    _resident(q.device, q=q, k=k, v=v, k_scale=k_scale, v_scale=v_scale, out=out, lse=lse, workspace=workspace,
              mask=mask, mask_tiles=mask_tiles,
              key_len=key_len, q_len=q_len, sinks=sinks, alibi=alibi)
    need = int(lib().fa_train_fwd_workspace_bytes(ctypes.byref(p)))
    if need == ctypes.c_size_t(-1).value:
        need = 0  # invalid parameters: the call itself reports why
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("fa_train_fwd_ws", lib().fa_train_fwd_ws(ctypes.byref(p), view4(q), view4(k), view4(v), view4(out),
                                                    view3(lse), ws_ptr, ws_bytes, _stream_handle(stream)))
    return out, lse


def fwd_unsplit(q, k, v, *, mask=None, scale=None, causal=False, q_offset=None, out=None, lse=None, stream=None,
                variant=0, mask_tiles=None, key_len=None, q_len=None, window=(-1, -1), sinks=None, alibi=None,
                softcap=0.0, k_scale=None, v_scale=None):
    """Forward through fa_train_fwd, the entry point without a workspace: the same results as
    fwd() (O, LSE), but every query tile's key walk stays in one workgroup."""
    _check_qkv(q, k, v, k_scale, v_scale)
    p = make_params(q, k, scale=scale, causal=causal, q_offset=q_offset, mask=mask, fwd_variant=variant,
                    mask_tiles=mask_tiles, key_len=key_len, q_len=q_len, window=window, sinks=sinks, alibi=alibi,
                    softcap=softcap, k_scale=k_scale, v_scale=v_scale)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _expect("out", out, dtype=q.dtype, shape=q.shape)
    _check_rowstats(q, lse=lse)
    _resident(q.device, q=q, k=k, v=v, k_scale=k_scale, v_scale=v_scale, out=out, lse=lse, mask=mask,
              mask_tiles=mask_tiles, key_len=key_len,
              q_len=q_len, sinks=sinks, alibi=alibi)
    _check("fa_train_fwd", lib().fa_train_fwd(ctypes.byref(p), view4(q), view4(k), view4(v), view4(out), view3(lse),
                                              _stream_handle(stream)))
    return out, lse


def bwd_preprocess(o, dout, *, delta=None, stream=None):
    """Delta = rowsum(dO * O) in fp32, [B, Hq, Sq]."""
    _expect("o", o, dtype=(torch.bfloat16, torch.float32))
    if o.dim() != 4:
        raise ValueError("o must be [B, Hq, Sq, D]")
    _expect("dout", dout, dtype=o.dtype, shape=o.shape)
    B, Hq, Sq, D = o.shape
    if delta is None:
        delta = torch.empty((B, Hq, Sq), dtype=torch.float32, device=o.device)
    _check_rowstats(o, delta=delta)
    _resident(o.device, o=o, dout=dout, delta=delta)
    p = FaAttnParams(B, Hq, Hq, Sq, Sq, D, _dtype_code(o), 0, 0, 1.0, None, 0, 0, None, 0, 0, 0)
    _check("fa_train_bwd_preprocess",
           lib().fa_train_bwd_preprocess(ctypes.byref(p), view4(o), view4(dout), view3(delta),
                                         _stream_handle(stream)))
    return delta


def bwd_sinks(lse, delta, sinks, *, dsink=None, stream=None):
    """Gradient of the attention sinks, ADDED into ``dsink`` (fp32 [Hq]; a zeroed one is made when
    None): dsink[h] += -sum over the head's rows of exp(sinks[h] - LSE) * Delta."""
    _expect("lse", lse, dtype=torch.float32)
    if lse.dim() != 3:
        raise ValueError("lse must be [B, Hq, Sq]")
    _expect("delta", delta, dtype=torch.float32, shape=lse.shape)
    B, Hq, Sq = lse.shape
    if dsink is None:
        dsink = torch.zeros(Hq, dtype=torch.float32, device=lse.device)
    if sinks.dtype != torch.float32 or sinks.shape != (Hq,) or not sinks.is_contiguous():
        raise ValueError("sinks must be a contiguous fp32 [Hq] tensor on the device")
    _expect("dsink", dsink, dtype=torch.float32, shape=(Hq,))
    _resident(lse.device, lse=lse, delta=delta, sinks=sinks, dsink=dsink)
    p = FaAttnParams(B, Hq, Hq, Sq, Sq, 64, FA_BF16, 0, 0, 1.0)
    p.window_left = p.window_right = -1
    p.sinks = sinks.data_ptr()
    _check("fa_train_bwd_sinks", lib().fa_train_bwd_sinks(ctypes.byref(p), view3(lse), view3(delta),
                                                          dsink.data_ptr(), _stream_handle(stream)))
    return dsink


def dequant_q8_0(qs, d, *, out=None, stream=None):
    """bf16 values of a q8_0-stored K or V window: ``qs`` int8 [B, H, S, D], ``d`` fp16 [B, H, S, D / 32]
    (views with a contiguous last dimension). Writes ``out`` (bf16 [B, H, S, D], made when None)."""
    if qs.dtype != torch.int8 or d.dtype != torch.float16:
        raise TypeError("qs must be int8 and d float16")
    if qs.dim() != 4:
        raise ValueError("qs must be [B, H, S, D]")
    B, H, S, D = qs.shape
    if tuple(d.shape) != (B, H, S, D // 32):
        raise ValueError("d must be [B, H, S, D / 32]")
    if out is None:
        out = torch.empty(qs.shape, dtype=torch.bfloat16, device=qs.device)
    _expect("out", out, dtype=torch.bfloat16, shape=qs.shape)
    _resident(qs.device, qs=qs, d=d, out=out)
    _check("fa_train_dequant_q8_0", lib().fa_train_dequant_q8_0(B, H, S, D, view4(qs), view4(d), view4(out),
                                                                _stream_handle(stream)))
    return out


def convert_f16(src, *, out=None, dtype=None, stream=None):
    """Values of an f16-stored K or V window in a compute type: ``src`` float16 [B, H, S, D] (a view
    with a contiguous last dimension). Writes ``out`` (float32 or bfloat16 [B, H, S, D]; made in
    ``dtype``, default bfloat16, when None): exact into float32, nearest-even into bfloat16."""
    if src.dtype != torch.float16:
        raise TypeError("src must be float16")
    if out is None:
        out = torch.empty(src.shape, dtype=dtype or torch.bfloat16, device=src.device)
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be float32 or bfloat16")
    if src.dim() != 4:
        raise ValueError("src must be [B, H, S, D]")
    _expect("out", out, shape=src.shape)
    _resident(src.device, src=src, out=out)
    Bn, H, S, D = src.shape
    _check("fa_train_convert_f16", lib().fa_train_convert_f16(Bn, H, S, D, view4(src), view4(out),
                                                              FA_F32 if out.dtype == torch.float32 else FA_BF16,
                                                              _stream_handle(stream)))
    return out


def bwd_workspace_bytes(q, k, *, scale=None, causal=False, q_offset=None, mask=None, kv_split=0, q_split=0,
                        key_len=None, q_len=None, window=(-1, -1), q_split_tiles=0, softcap=0.0, k_scale=None,
                        v_scale=None, dq_launch=0) -> int:
    p = make_params(q, k, scale=scale, causal=causal, q_offset=q_offset, mask=mask, kv_split=kv_split,
                    q_split=q_split, key_len=key_len, q_len=q_len, window=window, q_split_tiles=q_split_tiles,
                    softcap=softcap, k_scale=k_scale, v_scale=v_scale, dq_launch=dq_launch)
    return int(lib().fa_train_bwd_workspace_bytes(ctypes.byref(p)))


def _workspace(p: FaAttnParams, device, workspace):
    need = int(lib().fa_train_bwd_workspace_bytes(ctypes.byref(p)))
    if need == ctypes.c_size_t(-1).value:
        need = 0  # invalid parameters: the call itself reports why
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    else:
        _resident(device, workspace=workspace)
    return workspace, workspace.numel() * workspace.element_size()


def bwd(q, k, v, dout, lse, delta, *, mask=None, scale=None, causal=False, q_offset=None, dq=None, dk=None,
        dv=None, workspace=None, stream=None, kv_split=0, q_split=0, mask_tiles=None, key_len=None, q_len=None,
        window=(-1, -1), dq_launch=0, alibi=None, q_split_tiles=0, softcap=0.0, kv_walk=0, k_scale=None, v_scale=None,
        dbias=None):
    """Backward: returns (dQ, dK, dV), each in q's dtype, overwritten. ``dbias``: optional fp32
    tensor of the mask's shape that receives the mask's gradient, added in (zero it first).
    ``dq_launch``: 0 automatic, 1 / 2 the dQ walk in the dK/dV launch / its own, 3 dQ from the dS
    the dK/dV walk stores (a larger workspace), 4 the dQ walk's own kernel on a second stream
    beside the dK/dV kernel."""
    _check_qkv(q, k, v, k_scale, v_scale)
    _expect("dout", dout, dtype=q.dtype, shape=q.shape)
    _check_rowstats(q, lse=lse, delta=delta)
    p = make_params(q, k, scale=scale, causal=causal, q_offset=q_offset, mask=mask, kv_split=kv_split,
                    q_split=q_split, mask_tiles=mask_tiles, key_len=key_len, q_len=q_len, window=window,
                    dq_launch=dq_launch, alibi=alibi, q_split_tiles=q_split_tiles, softcap=softcap, kv_walk=kv_walk,
                    k_scale=k_scale, v_scale=v_scale,
                    dbias=dbias)
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    # (dK / dV in the compute dtype also for a K/V window stored as fp16 or q8_0)
    dk = torch.empty(k.shape, dtype=q.dtype, device=q.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=q.dtype, device=q.device) if dv is None else dv
    _expect("dq", dq, dtype=q.dtype, shape=q.shape)
    _expect("dk", dk, dtype=q.dtype, shape=k.shape)
    _expect("dv", dv, dtype=q.dtype, shape=k.shape)
    _resident(q.device, q=q, k=k, v=v, k_scale=k_scale, v_scale=v_scale, dout=dout, lse=lse, delta=delta, dq=dq,
              dk=dk, dv=dv, mask=mask,
              mask_tiles=mask_tiles, key_len=key_len, q_len=q_len, alibi=alibi, dbias=dbias)
    ws, nbytes = _workspace(p, q.device, workspace)
    _check("fa_train_bwd", lib().fa_train_bwd(ctypes.byref(p), view4(q), view4(k), view4(v), view4(dout), view3(lse),
                                              view3(delta), view4(dq), view4(dk), view4(dv), ws.data_ptr(), nbytes,
                                              _stream_handle(stream)))
    return dq, dk, dv


def bwd_noalloc(q, k, v, dout, lse, delta, *, mask=None, scale=None, causal=False, q_offset=None, dq=None,
                dk=None, dv=None, stream=None, kv_split=0, q_split=0, mask_tiles=None, key_len=None, q_len=None,
                window=(-1, -1), dq_launch=0, alibi=None, q_split_tiles=0, softcap=0.0, kv_walk=0, k_scale=None,
                v_scale=None,
                dbias=None):
    """Backward through fa_train_bwd_noalloc: the results of bwd(), with the workspace taken from
    the library's static device scratch instead of an allocation (dQ, dK and dV are still the
    caller's; pass them to allocate nothing here either)."""
    _check_qkv(q, k, v, k_scale, v_scale)
    _expect("dout", dout, dtype=q.dtype, shape=q.shape)
    _check_rowstats(q, lse=lse, delta=delta)
    p = make_params(q, k, scale=scale, causal=causal, q_offset=q_offset, mask=mask, kv_split=kv_split,
                    q_split=q_split, mask_tiles=mask_tiles, key_len=key_len, q_len=q_len, window=window,
                    dq_launch=dq_launch, alibi=alibi, q_split_tiles=q_split_tiles, softcap=softcap, kv_walk=kv_walk,
                    k_scale=k_scale, v_scale=v_scale,
                    dbias=dbias)
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    # (dK / dV in the compute dtype also for a K/V window stored as fp16 or q8_0)
    dk = torch.empty(k.shape, dtype=q.dtype, device=q.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=q.dtype, device=q.device) if dv is None else dv
    _expect("dq", dq, dtype=q.dtype, shape=q.shape)
    _expect("dk", dk, dtype=q.dtype, shape=k.shape)
    _expect("dv", dv, dtype=q.dtype, shape=k.shape)
    _resident(q.device, q=q, k=k, v=v, k_scale=k_scale, v_scale=v_scale, dout=dout, lse=lse, delta=delta, dq=dq,
              dk=dk, dv=dv, mask=mask,
              mask_tiles=mask_tiles, key_len=key_len, q_len=q_len, alibi=alibi, dbias=dbias)
    _check("fa_train_bwd_noalloc",
           lib().fa_train_bwd_noalloc(ctypes.byref(p), view4(q), view4(k), view4(v), view4(dout), view3(lse),
                                      view3(delta), view4(dq), view4(dk), view4(dv), _stream_handle(stream)))
    return dq, dk, dv


NOALLOC_SCRATCH_BYTES = 64 << 20  # FA_TRAIN_NOALLOC_SCRATCH_BYTES


BWD_SPLIT_CANDIDATES = ((0, 0), (1, 1), (2, 1), (4, 1), (8, 1), (1, 2), (2, 2), (4, 2))


def tune_bwd_splits(q, k, v, dout, lse, delta, *, mask=None, scale=None, causal=False, q_offset=None,
                    mask_tiles=None, candidates=BWD_SPLIT_CANDIDATES, reps=5, rounds=3, stream=None, key_len=None,
                    q_len=None, window=(-1, -1)):
    """Times the backward on these inputs for each (kv_split, q_split) candidate ((0, 0):
    the library's own choice) and returns the fastest pair: `rounds` passes over the
    candidates, interleaved, each candidate keeping its best pass of `reps` calls. The
    library chooses with a cost model that sees the shape but not the mask's content (key
    padding makes many key tiles dead), so a caller that runs one shape many times can
    tune once and pass the result to bwd(). Outputs go to scratch buffers; every pass
    synchronizes."""
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    need = max(bwd_workspace_bytes(q, k, scale=scale, causal=causal, q_offset=q_offset, mask=mask, kv_split=kv,
                                   q_split=qs, key_len=key_len, q_len=q_len, window=window) for kv, qs in candidates)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    best = {}
    for _ in range(rounds):
        for kv, qs in candidates:
            def call():
                bwd(q, k, v, dout, lse, delta, mask=mask, scale=scale, causal=causal, q_offset=q_offset, dq=dq,
                    dk=dk, dv=dv, workspace=ws, stream=s, kv_split=kv, q_split=qs, mask_tiles=mask_tiles,
                    key_len=key_len, q_len=q_len, window=window)
            call()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for _ in range(reps):
                call()
            e1.record(s)
            e1.synchronize()
            ms = e0.elapsed_time(e1) / reps
            best[(kv, qs)] = min(ms, best.get((kv, qs), ms))
    return min(best, key=best.get)


def bwd_chunked(q, k, v, dout, lse, delta, dk_acc, dv_acc, *, mask=None, scale=None, causal=True, q_offset=None,
                dq=None, workspace=None, stream=None, kv_split=0, q_split=0, mask_tiles=None, key_len=None,
                q_len=None, window=(-1, -1), dq_launch=0, alibi=None, q_split_tiles=0, softcap=0.0, kv_walk=0,
                k_scale=None, v_scale=None,
                dbias=None):
    """Chunked backward: returns dQ for the chunk; ADDS dK/dV into the fp32 window
    accumulators ``dk_acc`` / ``dv_acc`` ([B, Hkv, >= Sk, D]) and, when given, the mask's
    gradient into ``dbias`` (the mask's shape, fp32)."""
    _check_qkv(q, k, v, k_scale, v_scale)
    _expect("dout", dout, dtype=q.dtype, shape=q.shape)
    _check_rowstats(q, lse=lse, delta=delta)
    p = make_params(q, k, scale=scale, causal=causal, q_offset=q_offset, mask=mask, kv_split=kv_split,
                    q_split=q_split, mask_tiles=mask_tiles, key_len=key_len,
                    q_len=q_len, window=window, dq_launch=dq_launch, alibi=alibi, q_split_tiles=q_split_tiles,
                    softcap=softcap, kv_walk=kv_walk, k_scale=k_scale, v_scale=v_scale, dbias=dbias)
    if dk_acc.dtype != torch.float32 or dv_acc.dtype != torch.float32:
        raise TypeError("the window accumulators must be float32")
    B, Hkv, Sk, D = k.shape
    for name, acc in (("dk_acc", dk_acc), ("dv_acc", dv_acc)):
        if acc.dim() != 4 or acc.shape[0] != B or acc.shape[1] != Hkv or acc.shape[2] < Sk or acc.shape[3] != D:
            raise ValueError(f"{name} has shape {tuple(acc.shape)}, expected [{B}, {Hkv}, >= {Sk}, {D}]")
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    _expect("dq", dq, dtype=q.dtype, shape=q.shape)
    _resident(q.device, q=q, k=k, v=v, k_scale=k_scale, v_scale=v_scale, dout=dout, lse=lse, delta=delta, dq=dq,
              dk_acc=dk_acc, dv_acc=dv_acc,
              mask=mask, mask_tiles=mask_tiles, key_len=key_len, q_len=q_len, alibi=alibi, dbias=dbias)
    ws, nbytes = _workspace(p, q.device, workspace)
    _check("fa_train_bwd_chunked",
           lib().fa_train_bwd_chunked(ctypes.byref(p), view4(q), view4(k), view4(v), view4(dout), view3(lse),
                                      view3(delta), view4(dq), view4(dk_acc), view4(dv_acc), ws.data_ptr(), nbytes,
                                      _stream_handle(stream)))
    return dq


def probe_mfma(kind: int, a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """Run the matrix-core layout probe; a, b: fp32 [waves, 64, k]; returns [waves, 64, regs]."""
    waves = a.shape[0]
    regs = 16 if kind in (0, 2) else 4
    c = torch.empty((waves, 64, regs), dtype=torch.float32, device=a.device)
    _check("fa_train_probe_mfma", lib().fa_train_probe_mfma(kind, waves, a.data_ptr(), b.data_ptr(), c.data_ptr(),
                                                            _stream_handle(None)))
    return c


def probe_ds_read_tr16(byte_addr: torch.Tensor) -> torch.Tensor:
    """Run the LDS transpose-read probe; byte_addr: int32 [waves, 64]; returns int32 [waves, 64, 4]."""
    waves = byte_addr.shape[0]
    out = torch.empty((waves, 64, 4), dtype=torch.int16, device=byte_addr.device)
    _check("fa_train_probe_ds_read_tr16", lib().fa_train_probe_ds_read_tr16(waves, byte_addr.data_ptr(),
                                                                            out.data_ptr(), _stream_handle(None)))
    return out.to(torch.int32) & 0xFFFF
