"""The workloads the op is checked and measured on.

Shapes follow the pages' two trainers: the DiT adapter trainer (self-attention
at a 1542-token crop with GQA, cross-attention over up to 512 encoder tokens with
key padding), a causal GQA language-model layer, and the long-window exact walk
of the llama.cpp pull request (a 32768-token cached K/V window walked in 512-token
query chunks, each chunk attending causally to every earlier window position).

Config ``k`` (1-based) draws its inputs with seed ``1000 + k``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .inputs import BF16, F32, Case, alibi_slopes, make_case, quantize_q8_0, sink_logits, stored


@dataclass(frozen=True)
class Workload:
    key: str
    title: str
    index: int
    # the bf16 backward's (kv_split, q_split, q_split_tiles) for this workload: the fastest
    # or within noise of the fastest on MI355X over kv in {1, 2, 4}, q in {1, 2, 3, 4} and
    # the number of split query tiles (timed interleaved, best of three rounds); None: the
    # library's cost model
    bwd_splits: tuple | None = None
    # the bf16 backward's dQ formation (bwd_dq_launch): 0 the library's choice, 3 dQ from the dS
    # the dK/dV walk stores, 4 the dQ walk's own kernel on a second stream beside the dK/dV
    # kernel, where that measured faster on MI355X
    bwd_dq_launch: int = 0


WORKLOADS = {
    "tiny": Workload("tiny", "tiny parity case, fp32, B=1 H=2 S=64 D=64", 1),
    "dit_sa": Workload("dit_sa", "DiT self-attention, B=1 Hq=16 Hkv=8 S=1542 D=128 bf16, pad mask", 2, (2, 2, 6)),
    "dit_ca": Workload("dit_ca", "DiT cross-attention, B=2 H=16 Sq=1542 Sk=512 D=128 bf16, key-pad mask", 3,
                       (2, 1, 0), 4),
    "lm_causal": Workload("lm_causal", "LM causal GQA, B=1 Hq=32 Hkv=8 S=4096 D=128 bf16", 4, (2, 1, 0), 3),
    "long_window": Workload("long_window",
                            "long-window chunked walk, W=32768, 64 chunks of 512, Hq=16 Hkv=4 D=128 bf16", 5),
    # the DiT self-attention masks given by their structure instead of a dense mask:
    # the pad as a key length, and a mixed-length batch under a sliding window
    "dit_sa_len": Workload("dit_sa_len", "DiT self-attention, B=1 Hq=16 Hkv=8 S=1542 D=128 bf16, "
                           "key length 1388 (the pad as a length)", 6, (2, 2, 6)),
    "dit_sa_band": Workload("dit_sa_band", "DiT self-attention, mixed-length batch B=2 Hq=16 Hkv=8 S=1542 D=128 "
                            "bf16, key lengths 1542 / 1101, window 256 keys each side", 7),
    # the LM layer with one attention-sink logit per query head (N(0, 1)); its step adds the
    # sinks' gradient pass
    "lm_sinks": Workload("lm_sinks", "LM causal GQA with attention sinks, B=1 Hq=32 Hkv=8 S=4096 D=128 bf16", 8,
                         (2, 1, 0), 3),
    # the LM layer with ALiBi (slopes 2^(-8 (h + 1) / Hq)) in place of positional rotations
    "lm_alibi": Workload("lm_alibi", "LM causal GQA with ALiBi, B=1 Hq=32 Hkv=8 S=4096 D=128 bf16", 10, (2, 1, 0), 3),
    # the long-window walk over a q8_0-stored K/V window (the pages train such a cache in
    # place): the same queries and K/V values, quantised to q8_0 blocks
    "long_window_q8": Workload("long_window_q8", "long-window chunked walk over a q8_0 K/V window, W=32768, "
                               "64 chunks of 512, Hq=16 Hkv=4 D=128", 9),
    # the same walk over an fp16-stored window: the K/V draws rounded once to fp16
    # the LM layer with a logit softcap of 50 (the pages give no value; the cost does not depend
    # on it): the bf16 MFMA forward and backward with their cap variants
    "lm_softcap": Workload("lm_softcap", "LM causal GQA with logit softcap 50, B=1 Hq=32 Hkv=8 S=4096 D=128 bf16",
                           12, None, 3),
    "long_window_f16": Workload("long_window_f16", "long-window chunked walk over an f16 K/V window, W=32768, "
                                "64 chunks of 512, Hq=16 Hkv=4 D=128", 11),
}

# the sliding window of the structured DiT workload: keys within this distance on each
# side of a row's position (the trainer's width is not given)
DIT_WINDOW = 256

LONG_WINDOW = 32768
LONG_CHUNK = 512


def seed_of(key: str) -> int:
    return 1000 + WORKLOADS[key].index


def make(key: str, **shrink) -> Case:
    """Build the seeded case for a workload. Keyword overrides (e.g. ``Hq=2``) shrink
    a workload for a fast test while keeping its structure and its seed."""
    s = seed_of(key)
    if key == "tiny":
        a = dict(B=1, Hq=2, Hkv=2, Sq=64, Sk=64, D=64, dtype=F32)
        a.update(shrink)
        return make_case(key, seed=s, **a)
    if key == "dit_sa":
        a = dict(B=1, Hq=16, Hkv=8, Sq=1542, Sk=1542, D=128, dtype=BF16)
        a.update(shrink)
        return make_case(key, seed=s, mask="sa_pad", **a)
    if key == "dit_ca":
        a = dict(B=2, Hq=16, Hkv=16, Sq=1542, Sk=512, D=128, dtype=BF16)
        lo_hi = {"lo": 128, "hi": 512, "masked_rows": 2}
        if "Sk" in shrink:  # keep the valid lengths inside the shrunk key count, below its end
            lo_hi["hi"] = max(1, (3 * shrink["Sk"]) // 4)
            lo_hi["lo"] = max(1, shrink["Sk"] // 4)
        a.update(shrink)
        return make_case(key, seed=s, mask="ca_keypad", mask_args=lo_hi, **a)
    if key in ("lm_causal", "lm_sinks", "lm_alibi", "lm_softcap"):
        a = dict(B=1, Hq=32, Hkv=8, Sq=4096, Sk=4096, D=128, dtype=BF16, do_std=0.1)
        a.update(shrink)
        c = make_case(key, seed=s, causal=True, q_offset=0, **a)
        if key == "lm_sinks":
            c.meta["sinks"] = sink_logits(s, c.Hq)
        if key == "lm_alibi":
            c.meta["alibi"] = alibi_slopes(c.Hq)
        if key == "lm_softcap":
            c.meta["softcap"] = 50.0
        return c
    if key in ("dit_sa_len", "dit_sa_band"):
        a = dict(B=1 if key == "dit_sa_len" else 2, Hq=16, Hkv=8, Sq=1542, Sk=1542, D=128, dtype=BF16)
        a.update(shrink)
        c = make_case(key, seed=s, **a)
        n_pad = int(round(0.1 * c.Sk))  # the self-attention pad of the DiT workload
        if key == "dit_sa_len":
            c.meta["structure"] = {"key_len": [c.Sk - n_pad] * c.B, "q_len": None, "window": (-1, -1)}
        else:
            lens = [c.Sk if b % 2 == 0 else max(1, (c.Sk * 5) // 7) for b in range(c.B)]
            w = min(DIT_WINDOW, c.Sk)
            c.meta["structure"] = {"key_len": lens, "q_len": None, "window": (w, w)}
        c.meta["mask_kind"] = "structured"
        return c
    if key in ("long_window", "long_window_q8", "long_window_f16"):
        W = shrink.pop("W", LONG_WINDOW)
        a = dict(B=1, Hq=16, Hkv=4, Sq=W, Sk=W, D=128, dtype=BF16)
        a.update(shrink)
        c = make_case(key, seed=s, causal=True, q_offset=0, **a)
        if key == "long_window_q8":  # the cache holds the K / V values as q8_0 blocks
            c.meta["q8"] = {"k": quantize_q8_0(c.f64("k")), "v": quantize_q8_0(c.f64("v"))}
        if key == "long_window_f16":
            # the cache holds the K / V draws (the same normals, kept in fp32) rounded to fp16;
            # the case's own K / V are those fp16 values in the compute dtype
            full = make_case(key, seed=s, causal=True, q_offset=0, **dict(a, dtype=F32))
            c.meta["f16"] = {n: full.f64(n).astype(np.float16) for n in ("k", "v")}
            c.k, c.v = (stored(c.meta["f16"][n].astype(np.float32), c.dtype) for n in ("k", "v"))
        return c
    raise KeyError(key)


def chunk_plan(W: int = LONG_WINDOW, chunk: int = LONG_CHUNK) -> list[tuple[int, int, int]]:
    """The exact walk's fixed plan: (row start p0, rows, keys visible) per chunk.

    Chunk c covers query rows [p0, p0 + chunk) with p0 = c * chunk and sees window
    keys [0, p0 + chunk); its causal offset is p0.
    """
    if W % chunk:
        raise ValueError("window must be a whole number of chunks")
    return [(c * chunk, chunk, (c + 1) * chunk) for c in range(W // chunk)]
