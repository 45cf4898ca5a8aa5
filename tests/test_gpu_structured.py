"""GPU parity of the structured masks (per-batch key and query lengths, a band of
keys around each row's position, alone or with the causal diagonal and a dense
mask) against the oracle, which takes their dense definition
(oracle.structured_mask): every output, element by element, with the exact-zero
checks for fully masked rows and dead key columns. The pages' DiT masks ("sa":
sliding window with padded key columns, "sa_pad": padded key columns) are the
workloads these stand for; their widths are not given, so the cases vary them."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from flash_attention_train_amd import binding
from flash_attention_train_amd.inputs import make_case
from parity_util import compare_full, host64, say, upload

pytestmark = pytest.mark.gpu


def _case(name, *, B, Hq, Hkv, Sq, Sk, D, seed, causal=False, q_offset=None, key_len=None, q_len=None,
          window=(-1, -1), mask="none", mask_args=None):
    c = make_case(name, B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D, dtype="bf16", seed=seed, causal=causal,
                  q_offset=q_offset, mask=mask, mask_args=mask_args)
    s = oracle.structured_mask(B, Sq, Sk, key_len=key_len, q_len=q_len, window_left=window[0],
                               window_right=window[1], q_offset=c.q_offset, causal=False)
    c.meta["structure"] = dict(key_len=key_len, q_len=q_len, window=window)
    c.meta["dense_mask"] = c.mask  # what the GPU gets as its dense mask (or None)
    # what the oracle gets: the structure as a dense mask, plus the dense mask if any
    full = s if c.mask is None else s + np.broadcast_to(c.mask.astype(np.float64), s.shape)
    c.mask = full.astype(np.float32)
    return c


CASES = {
    # padded key columns per batch entry, one entry with no keys at all (every row fully masked)
    "key_len_ragged": lambda: _case("key_len_ragged", B=3, Hq=4, Hkv=2, Sq=300, Sk=300, D=128, seed=81,
                                    key_len=[300, 173, 0]),
    # query and key lengths together, ragged, GQA
    "q_and_key_len": lambda: _case("q_and_key_len", B=2, Hq=4, Hkv=1, Sq=260, Sk=200, D=128, seed=82,
                                   key_len=[131, 200], q_len=[260, 97]),
    # a two-sided band (sliding window) with padded keys, D = 64
    "band_two_sided": lambda: _case("band_two_sided", B=2, Hq=2, Hkv=2, Sq=400, Sk=400, D=64, seed=83,
                                    key_len=[400, 317], window=(64, 64)),
    # causal with a left window (local causal attention), GQA 4
    "causal_window": lambda: _case("causal_window", B=1, Hq=4, Hkv=1, Sq=333, Sk=333, D=128, seed=84, causal=True,
                                   window=(100, -1)),
    # a chunk of queries at an offset into a longer key window, causal and windowed
    "chunk_window": lambda: _case("chunk_window", B=1, Hq=4, Hkv=2, Sq=100, Sk=356, D=128, seed=85, causal=True,
                                  q_offset=256, window=(128, -1)),
    # a band one key wide on each side, queries before the keys: leading rows see no key
    "narrow_band": lambda: _case("narrow_band", B=1, Hq=2, Hkv=1, Sq=150, Sk=130, D=64, seed=86,
                                 q_offset=-20, window=(1, 1)),
    # a right window only (keys up to 7 ahead of the position) with a query length
    "right_window_qlen": lambda: _case("right_window_qlen", B=2, Hq=2, Hkv=1, Sq=190, Sk=190, D=128, seed=87,
                                       window=(-1, 7), q_len=[190, 65]),
    # the structure on top of a dense random bias mask with fully masked rows and columns
    "with_dense_mask": lambda: _case("with_dense_mask", B=2, Hq=2, Hkv=1, Sq=130, Sk=170, D=128, seed=88,
                                     key_len=[120, 170], window=(80, 40), mask="random",
                                     mask_args={"Bm": 2, "full_rows": 3, "full_cols": 2}),
}


def _lens(c):
    st = c.meta["structure"]
    out = {}
    for n in ("key_len", "q_len"):
        out[n] = None if st[n] is None else torch.tensor(st[n], dtype=torch.int32, device="cuda")
    out["window"] = st["window"]
    return out


def run_structured(c, *, split=0, kv_split=0, q_split=0):
    t = upload(c)
    dm = c.meta["dense_mask"]
    mask = None if dm is None else torch.from_numpy(dm).to("cuda")
    s = _lens(c)
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=mask, scale=c.scale, causal=c.causal, q_offset=c.q_offset,
                         split=split, **s)
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=mask, scale=c.scale,
                             causal=c.causal, q_offset=c.q_offset, kv_split=kv_split, q_split=q_split, **s)
    torch.cuda.synchronize()
    return {"O": host64(o), "LSE": host64(lse), "Delta": host64(delta), "dQ": host64(dq), "dK": host64(dk),
            "dV": host64(dv)}


_REF = {}


def reference(name):
    if name not in _REF:
        c = CASES[name]()
        _REF[name] = (c, oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), c.mask.astype(np.float64),
                                         scale=c.scale, causal=c.causal, q_offset=c.q_offset))
    return _REF[name]


@pytest.mark.parametrize("name", list(CASES))
def test_structured_parity(name):
    c, ref = reference(name)
    say(f"case {name}: B={c.B} Hq={c.Hq} Hkv={c.Hkv} Sq={c.Sq} Sk={c.Sk} D={c.D} causal={c.causal} "
        f"q_offset={c.q_offset} {c.meta['structure']} dense={c.meta['dense_mask'] is not None}")
    compare_full(c, run_structured(c), ref)


@pytest.mark.parametrize("split", [2, 3])
@pytest.mark.parametrize("name", ["key_len_ragged", "causal_window", "chunk_window", "narrow_band"])
def test_structured_split_forward(name, split):
    """The split key walk shares the structured key range; its merge gives the same rows."""
    c, ref = reference(name)
    say(f"case {name}: split {split}")
    compare_full(c, run_structured(c, split=split), ref)


@pytest.mark.parametrize("kv_split,q_split", [(2, 1), (1, 3), (4, 2)])
@pytest.mark.parametrize("name", ["q_and_key_len", "band_two_sided", "chunk_window"])
def test_structured_backward_decompositions(name, kv_split, q_split):
    """Split dK/dV and dQ walks over the structured row and key ranges."""
    c, ref = reference(name)
    say(f"case {name}: kv_split {kv_split} q_split {q_split}")
    compare_full(c, run_structured(c, kv_split=kv_split, q_split=q_split), ref)


def test_structured_equals_dense_mask():
    """The same problem with the structure given as a dense 0 / -inf mask instead: both
    are the oracle's within the tolerance, and they agree with each other as closely."""
    c, ref = reference("band_two_sided")
    got_s = run_structured(c)
    t = upload(c)
    m = torch.from_numpy(c.mask).to("cuda")
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=m, scale=c.scale, causal=c.causal, q_offset=c.q_offset)
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=m, scale=c.scale, causal=c.causal,
                             q_offset=c.q_offset)
    torch.cuda.synchronize()
    got_d = {"O": host64(o), "LSE": host64(lse), "Delta": host64(delta), "dQ": host64(dq), "dK": host64(dk),
             "dV": host64(dv)}
    compare_full(c, got_d, ref)
    for n in got_s:
        den = np.abs(ref[n]).max()
        assert np.abs(got_s[n] - got_d[n]).max() <= 2e-2 * den, n


def test_structured_chunked_window():
    """The chunked walk (fp32 dK/dV accumulated over chunks) with a left window: eight
    64-row chunks over a 512-key window against the one-shot oracle."""
    W, C, wl = 512, 64, 96
    c = _case("chunked_window", B=1, Hq=4, Hkv=2, Sq=W, Sk=W, D=128, seed=89, causal=True, q_offset=0,
              window=(wl, -1))
    t = upload(c)
    dk_acc = torch.zeros((1, c.Hkv, W, c.D), dtype=torch.float32, device="cuda")
    dv_acc = torch.zeros_like(dk_acc)
    O = torch.empty_like(t["q"])
    LSE = torch.empty((1, c.Hq, W), dtype=torch.float32, device="cuda")
    Delta = torch.empty_like(LSE)
    dQ = torch.empty_like(t["q"])
    for p0 in range(0, W, C):
        sk = p0 + C
        q = t["q"][:, :, p0:p0 + C]
        do = t["do"][:, :, p0:p0 + C]
        kk, vv = t["k"][:, :, :sk], t["v"][:, :, :sk]
        o, lse = binding.fwd(q, kk, vv, scale=c.scale, causal=True, q_offset=p0, out=O[:, :, p0:p0 + C],
                             lse=LSE[:, :, p0:p0 + C], window=(wl, -1))
        delta = binding.bwd_preprocess(o, do, delta=Delta[:, :, p0:p0 + C])
        binding.bwd_chunked(q, kk, vv, do, lse, delta, dk_acc, dv_acc, scale=c.scale, causal=True, q_offset=p0,
                            dq=dQ[:, :, p0:p0 + C], window=(wl, -1))
    torch.cuda.synchronize()
    ref = oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), c.mask.astype(np.float64),
                          scale=c.scale, causal=True, q_offset=0)
    got = {"O": host64(O), "LSE": host64(LSE), "Delta": host64(Delta), "dQ": host64(dQ),
           "dK": dk_acc.cpu().numpy().astype(np.float64), "dV": dv_acc.cpu().numpy().astype(np.float64)}
    compare_full(c, got, ref)


def test_structured_lengths_are_read_on_the_device():
    """key_len / q_len are device arrays read by the kernels: changing them between two
    calls (no host sync of their values) changes the result to the new lengths'."""
    c, ref = reference("q_and_key_len")
    t = upload(c)
    kl = torch.tensor([200, 200], dtype=torch.int32, device="cuda")
    o1, _ = binding.fwd(t["q"], t["k"], t["v"], scale=c.scale, key_len=kl)
    kl.copy_(torch.tensor([131, 200], dtype=torch.int32))
    ql = torch.tensor([260, 97], dtype=torch.int32, device="cuda")
    o2, _ = binding.fwd(t["q"], t["k"], t["v"], scale=c.scale, key_len=kl, q_len=ql)
    torch.cuda.synchronize()
    g2 = host64(o2)
    assert np.abs(g2 - ref["O"]).max() <= 2e-2 * np.abs(ref["O"]).max()
    assert np.abs(host64(o1) - g2).max() > 0.1  # the first call did not see the later lengths
