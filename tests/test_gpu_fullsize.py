"""GPU parity at the workloads' full sizes, in the launch configuration the bench
times (automatic decomposition, mask tile maps for masked workloads):

* DiT self-attention and DiT cross-attention: every output against the whole oracle;
* LM causal: every output against the whole oracle;
* long-window chunked walk (64 chunks of 512 over a 32768-key window, fp32 dK/dV
  accumulators): a row of every chunk, key columns spread over the whole window (so
  that each sums the contributions of many chunks), and the column-sum identities
  sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i, which hold at any size;
* the LM layer with sinks, ALiBi or a softcap: sampled rows and key columns.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from flash_attention_train_amd import binding, configs
from parity_util import TOL, compare_full, host64, rel_err, run_gpu, say, upload, visibility

pytestmark = pytest.mark.gpu


def _mask64(c):
    return None if c.mask is None else c.mask.astype(np.float64)


def _splits(key):
    """The backward decomposition the bench uses for this workload (its table entry, else automatic)."""
    kv, qs, qt = configs.WORKLOADS[key].bwd_splits or (0, 0, 0)
    return dict(kv_split=kv, q_split=qs, q_split_tiles=qt)


def _run_with_tiles(c, t):
    tiles = binding.mask_tile_map(t["mask"], t["q"], t["k"]) if t["mask"] is not None else None
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal,
                         q_offset=c.q_offset, mask_tiles=tiles)
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=t["mask"], scale=c.scale,
                             causal=c.causal, q_offset=c.q_offset, mask_tiles=tiles, **_splits(c.name))
    torch.cuda.synchronize()
    return {"O": host64(o), "LSE": host64(lse), "Delta": host64(delta), "dQ": host64(dq), "dK": host64(dk),
            "dV": host64(dv)}


@pytest.mark.parametrize("key", ["dit_sa", "dit_ca"])
def test_dit_full_size_every_element(key):
    c = configs.make(key)
    say(f"{key}: full size B={c.B} Hq={c.Hq} Hkv={c.Hkv} Sq={c.Sq} Sk={c.Sk}; oracle running")
    got = _run_with_tiles(c, upload(c))
    ref = oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), _mask64(c), scale=c.scale,
                          causal=c.causal, q_offset=c.q_offset)
    compare_full(c, got, ref)
    if key == "dit_ca":  # the workload's own exact-zero claims (skill page, traps 8 and 9)
        full, dead = visibility(c)
        assert full.sum() == 2 * c.B and dead.any()


@pytest.mark.parametrize("key", ["dit_sa_len", "dit_sa_band"])
def test_structured_dit_full_size_every_element(key):
    """The structured DiT workloads as the bench runs them (lengths on the device, the
    window, the table's backward decomposition): every output against the oracle given
    the structure's dense mask."""
    c = configs.make(key)
    st = c.meta["structure"]
    say(f"{key}: full size B={c.B} Hq={c.Hq} Hkv={c.Hkv} S={c.Sq} {st}; oracle running")
    t = upload(c)
    kl = torch.tensor(st["key_len"], dtype=torch.int32, device="cuda")
    o, lse = binding.fwd(t["q"], t["k"], t["v"], scale=c.scale, key_len=kl, window=st["window"])
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, scale=c.scale, key_len=kl,
                             window=st["window"], **_splits(key))
    torch.cuda.synchronize()
    got = {"O": host64(o), "LSE": host64(lse), "Delta": host64(delta), "dQ": host64(dq), "dK": host64(dk),
           "dV": host64(dv)}
    m = oracle.structured_mask(c.B, c.Sq, c.Sk, key_len=st["key_len"], q_len=st["q_len"],
                               window_left=st["window"][0], window_right=st["window"][1], q_offset=c.q_offset)
    ref = oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), m, scale=c.scale, causal=c.causal,
                          q_offset=c.q_offset)
    c.mask = m.astype(np.float32)  # for the exact-zero checks of dead rows and columns
    compare_full(c, got, ref)


def _check_rows(c, got, ids, ref, tol):
    D = c.D
    full, _ = visibility(c)
    b = ids // (c.Hq * c.Sq)
    i = ids % c.Sq
    masked = full[b, i]
    for n in ("O", "dQ"):
        g = got[n].reshape(-1, D)[ids]
        assert np.all(g[masked] == 0)
        e = rel_err(g[~masked], ref[n][~masked])
        say(f"    rows {n}: {e:.2e}")
        assert e <= tol, n
    for n in ("LSE", "Delta"):
        g = got[n].reshape(-1)[ids]
        assert np.all(g[masked] == 0)
        e = rel_err(g[~masked], ref[n][~masked])
        say(f"    rows {n}: {e:.2e}")
        assert e <= tol, n


def _check_cols(c, got_dk, got_dv, ids, ref, tol):
    for n, g in (("dK", got_dk.reshape(-1, c.D)[ids]), ("dV", got_dv.reshape(-1, c.D)[ids])):
        assert np.abs(ref[n]).max() > 0
        e = rel_err(g, ref[n])
        say(f"    cols {n}: {e:.2e}")
        assert e <= tol, n


def test_lm_causal_full_size_every_element():
    """The LM layer (B=1, Hq=32, Hkv=8, S=4096, D=128, causal) as the bench runs it: every output
    against the whole oracle (about 0.5 TFLOP of float64 work on the host cores)."""
    c = configs.make("lm_causal")
    say(f"lm_causal: full size B={c.B} Hq={c.Hq} Hkv={c.Hkv} S={c.Sq}; GPU step")
    got = _run_with_tiles(c, upload(c))
    say("lm_causal: whole oracle running (tens of seconds)")
    ref = oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), None, scale=c.scale, causal=True,
                          q_offset=0)
    compare_full(c, got, ref)


def run_walk(c, t, W, C):
    """The exact walk on the GPU: per chunk fwd -> preprocess -> chunked bwd, dK/dV in fp32."""
    dk_acc = torch.zeros((1, c.Hkv, W, c.D), dtype=torch.float32, device="cuda")
    dv_acc = torch.zeros_like(dk_acc)
    O = torch.empty_like(t["q"])
    LSE = torch.empty((1, c.Hq, W), dtype=torch.float32, device="cuda")
    Delta = torch.empty_like(LSE)
    dQ = torch.empty_like(t["q"])
    for p0, n, sk in configs.chunk_plan(W, C):
        q, do = t["q"][:, :, p0:p0 + n], t["do"][:, :, p0:p0 + n]
        kk, vv = t["k"][:, :, :sk], t["v"][:, :, :sk]
        o, lse = binding.fwd(q, kk, vv, scale=c.scale, causal=True, q_offset=p0, out=O[:, :, p0:p0 + n],
                             lse=LSE[:, :, p0:p0 + n])
        delta = binding.bwd_preprocess(o, do, delta=Delta[:, :, p0:p0 + n])
        binding.bwd_chunked(q, kk, vv, do, lse, delta, dk_acc, dv_acc, scale=c.scale, causal=True, q_offset=p0,
                            dq=dQ[:, :, p0:p0 + n])
    torch.cuda.synchronize()
    return {"O": host64(O), "LSE": host64(LSE), "Delta": host64(Delta), "dQ": host64(dQ),
            "dK": dk_acc.cpu().numpy().astype(np.float64), "dV": dv_acc.cpu().numpy().astype(np.float64)}


def test_long_window_walk_full_size():
    """The 64-chunk walk over the 32768-key window against the one-shot oracle: a query row from every
    chunk in two heads plus random rows (O, LSE, Delta, dQ); key columns spread over the whole window
    in two KV heads, one in every 2048 keys, so that early columns hold fp32 sums over up to 64 chunks
    (dK, dV); and the column-sum identities over the whole window."""
    W, C = configs.LONG_WINDOW, configs.LONG_CHUNK
    c = configs.make("long_window")
    say(f"long_window: 64-chunk walk over W={W}; GPU walk")
    got = run_walk(c, upload(c), W, C)
    rng = np.random.default_rng(5)
    nchunk = W // C
    every_chunk = [h * W + C * k + int(rng.integers(C)) for h in (0, 13) for k in range(nchunk)]
    rows = np.unique(np.concatenate([
        [0, 511, 512, 32767, 5 * W + 16384], every_chunk,
        rng.choice(c.Hq * W, 96, replace=False)]).astype(np.int64))
    say(f"    oracle rows ({rows.size})")
    ref = oracle.rows(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), rows, scale=c.scale, causal=True,
                      q_offset=0)
    _check_rows(c, got, rows, ref, TOL[c.dtype])
    q64, k64, v64, do64 = c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do")
    for g in (0, 3):
        # column 0 (seen by every row of the group), one column in each 2048 keys, the last key
        js = np.unique(np.concatenate([[0, W - 1], 2048 * np.arange(W // 2048) + rng.integers(2048, size=W // 2048)]))
        cols = (g * W + js).astype(np.int64)
        say(f"    oracle key columns of KV head {g} ({cols.size}, from key {js.min()} to {js.max()}; "
            f"about a minute of host time)")
        refc = oracle.cols(q64, k64, v64, do64, cols, scale=c.scale, causal=True, q_offset=0)
        _check_cols(c, got["dK"], got["dV"], cols, refc, TOL[c.dtype])
    # identities over the whole window, per KV head and feature
    do = c.f64("do")
    G = c.Hq // c.Hkv
    sum_do = do[0].reshape(c.Hkv, G, W, c.D).sum(axis=(1, 2))
    dv_sum = got["dV"][0].sum(axis=1)
    e_v = np.abs(dv_sum - sum_do).max() / np.abs(do).sum(axis=(0, 2)).reshape(c.Hkv, G, c.D).sum(axis=1).max()
    dk_sum = got["dK"][0].sum(axis=1)
    e_k = np.abs(dk_sum).max() / np.abs(got["dK"][0]).sum(axis=1).max()
    say(f"    identities: sum dV vs sum dO {e_v:.2e}, |sum dK| / sum |dK| {e_k:.2e}")
    assert e_v <= TOL[c.dtype] and e_k <= TOL[c.dtype]


def test_lm_sinks_full_size_sampled():
    """The LM layer with attention sinks, as the bench runs it: sampled rows (O, LSE, Delta, dQ) and key
    columns (dK, dV) against the oracle with the same sinks, and the sinks' gradient against its
    definition summed on the host over every row's GPU LSE and Delta (a property at any size; the
    LSE and Delta themselves are pinned by the sampled rows)."""
    c = configs.make("lm_sinks")
    say("lm_sinks: full size, sampled rows and columns, sink gradient over all rows")
    t = upload(c)
    sinks = torch.from_numpy(c.meta["sinks"]).to("cuda")
    o, lse = binding.fwd(t["q"], t["k"], t["v"], scale=c.scale, causal=True, q_offset=0, sinks=sinks)
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, scale=c.scale, causal=True, q_offset=0)
    dsink = binding.bwd_sinks(lse, delta, sinks)
    torch.cuda.synchronize()
    got = {"O": host64(o), "LSE": host64(lse), "Delta": host64(delta), "dQ": host64(dq), "dK": host64(dk),
           "dV": host64(dv)}
    s64 = c.meta["sinks"].astype(np.float64)
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, 1, c.Sq - 1, 7 * c.Sq + 2], rng.choice(c.Hq * c.Sq, 80, replace=False)])
                     ).astype(np.int64)
    ref = oracle.rows(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), rows, scale=c.scale, causal=True,
                      q_offset=0, sinks=s64)
    _check_rows(c, got, rows, ref, TOL[c.dtype])
    cols = np.unique(np.concatenate([[0, c.Sk - 1], rng.choice(np.arange(c.Sk, 2 * c.Sk), 8, replace=False)])
                     ).astype(np.int64)
    refc = oracle.cols(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), cols, scale=c.scale, causal=True,
                       q_offset=0, sinks=s64)
    _check_cols(c, got["dK"], got["dV"], cols, refc, TOL[c.dtype])
    terms = np.exp(s64[None, :, None] - got["LSE"]) * got["Delta"]
    want = -terms.sum(axis=(0, 2))
    e = np.abs(dsink.cpu().numpy().astype(np.float64) - want).max() / np.abs(terms).sum(axis=(0, 2)).max()
    say(f"    dSink vs the host sum over all rows: {e:.2e}")
    assert e <= 1e-5


def test_lm_alibi_full_size_sampled():
    """The LM layer with ALiBi, as the bench runs it: sampled rows (O, LSE, Delta, dQ) and key columns
    (dK, dV) against the oracle with the same slopes."""
    c = configs.make("lm_alibi")
    say("lm_alibi: full size, sampled rows and columns")
    t = upload(c)
    al = torch.from_numpy(c.meta["alibi"]).to("cuda")
    o, lse = binding.fwd(t["q"], t["k"], t["v"], scale=c.scale, causal=True, q_offset=0, alibi=al)
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, scale=c.scale, causal=True, q_offset=0,
                             alibi=al, **_splits("lm_alibi"))
    torch.cuda.synchronize()
    got = {"O": host64(o), "LSE": host64(lse), "Delta": host64(delta), "dQ": host64(dq), "dK": host64(dk),
           "dV": host64(dv)}
    a64 = c.meta["alibi"].astype(np.float64)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 1, c.Sq - 1, 31 * c.Sq + 4000], rng.choice(c.Hq * c.Sq, 80, replace=False)])
                     ).astype(np.int64)
    ref = oracle.rows(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), rows, scale=c.scale, causal=True,
                      q_offset=0, alibi=a64)
    _check_rows(c, got, rows, ref, TOL[c.dtype])
    cols = np.unique(np.concatenate([[0, c.Sk - 1], rng.choice(np.arange(7 * c.Sk, 8 * c.Sk), 8, replace=False)])
                     ).astype(np.int64)
    refc = oracle.cols(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), cols, scale=c.scale, causal=True,
                       q_offset=0, alibi=a64)
    _check_cols(c, got["dK"], got["dV"], cols, refc, TOL[c.dtype])


def test_lm_softcap_full_size_sampled():
    """The LM layer with a logit softcap, as the bench runs it (the MFMA kernels' cap variants): sampled rows
    (O, LSE, Delta, dQ) and key columns (dK, dV) against the oracle with the same cap."""
    c = configs.make("lm_softcap")
    cap = c.meta["softcap"]
    say(f"lm_softcap: full size, softcap {cap}, sampled rows and columns")
    t = upload(c)
    o, lse = binding.fwd(t["q"], t["k"], t["v"], scale=c.scale, causal=True, q_offset=0, softcap=cap)
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, scale=c.scale, causal=True, q_offset=0,
                             softcap=cap)
    torch.cuda.synchronize()
    got = {"O": host64(o), "LSE": host64(lse), "Delta": host64(delta), "dQ": host64(dq), "dK": host64(dk),
           "dV": host64(dv)}
    rng = np.random.default_rng(8)
    rows = np.unique(np.concatenate([[0, 1, c.Sq - 1, 17 * c.Sq + 2049], rng.choice(c.Hq * c.Sq, 60, replace=False)])
                     ).astype(np.int64)
    ref = oracle.rows(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), rows, scale=c.scale, causal=True,
                      q_offset=0, softcap=cap)
    _check_rows(c, got, rows, ref, TOL[c.dtype])
    cols = np.unique(np.concatenate([[0, c.Sk - 1], rng.choice(np.arange(5 * c.Sk, 6 * c.Sk), 8, replace=False)])
                     ).astype(np.int64)
    refc = oracle.cols(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), cols, scale=c.scale, causal=True,
                       q_offset=0, softcap=cap)
    _check_cols(c, got["dK"], got["dV"], cols, refc, TOL[c.dtype])
