"""Pins of the CPU oracle to things other than itself (no GPU involved).

Each check is chosen so that a plausible slip in the oracle -- a dropped scale, a
wrong sign, a transposed operand, a wrong GQA head index, a mishandled mask --
fails at least one of them:

* a hand-worked example whose every value was derived on paper (golden file);
* central finite differences, in float64, of L = <O, dO> with respect to Q, K, V;
* PyTorch CPU float64 autograd through an explicitly materialised softmax;
* closed forms (one key, uniform scores, first causal row) and invariants;
* exact zeros for fully masked rows and fully masked key columns;
* GQA equal to the group sum over the head-expanded problem;
* the chunked walk equal to the one-shot problem.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

import oracle
from flash_attention_train_amd import configs
from flash_attention_train_amd.inputs import make_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _problem(seed, B=1, Hq=2, Hkv=1, Sq=6, Sk=7, D=4, mask="none", causal=False, q_offset=None,
             mask_args=None, scale=None):
    c = make_case("pin", B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D, dtype="f32", seed=seed, mask=mask,
                  causal=causal, q_offset=q_offset, mask_args=mask_args, scale=scale)
    return c


def _arrays(c):
    return c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), (None if c.mask is None else c.mask.astype(np.float64))


def _full(c):
    q, k, v, do, m = _arrays(c)
    return oracle.backward(q, k, v, do, m, scale=c.scale, causal=c.causal, q_offset=c.q_offset)


def _fully_masked_rows(c):
    """Boolean [B, Sq]: rows with no visible key (mask and causal)."""
    vis = np.ones((c.B, c.Sq, c.Sk), bool)
    if c.mask is not None:
        vis &= np.isfinite(c.mask) if c.mask.shape[0] == c.B else np.isfinite(c.mask[[0] * c.B])
    if c.causal:
        vis &= np.arange(c.Sk)[None, None, :] <= (c.q_offset + np.arange(c.Sq))[None, :, None]
    return ~vis.any(axis=2), vis


# ---------------------------------------------------------------------------
# golden: a worked example derived by hand
# ---------------------------------------------------------------------------
def test_golden_worked_example():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)

    def arr(x):
        return np.array([[(-np.inf if e == "-inf" else e) for e in row] for row in x], dtype=np.float64)

    q = arr(g["q"])[None, None]
    k = arr(g["k"])[None, None]
    v = arr(g["v"])[None, None]
    do = arr(g["do"])[None, None]
    m = arr(g["mask"])[None]
    r = oracle.backward(q, k, v, do, m, scale=g["scale"])
    for name, want in g["expect"].items():
        got = r[name][0, 0]
        np.testing.assert_allclose(got, np.array(want), rtol=1e-14, atol=1e-14, err_msg=name)
    # the fully masked row and column are exactly zero, not merely small
    assert np.all(r["O"][0, 0, 2] == 0) and r["LSE"][0, 0, 2] == 0 and np.all(r["dQ"][0, 0, 2] == 0)
    assert np.all(r["dK"][0, 0, 3] == 0) and np.all(r["dV"][0, 0, 3] == 0)


# ---------------------------------------------------------------------------
# finite differences of L = <O, dO>
# ---------------------------------------------------------------------------
FD_CASES = {
    "plain": dict(seed=11),
    "gqa2_sa_pad": dict(seed=12, Hq=4, Hkv=2, Sq=8, Sk=8, mask="sa_pad", mask_args={"pad_frac": 0.25}),
    "ca_keypad_rows": dict(seed=13, B=2, Hq=2, Hkv=2, Sq=7, Sk=6, mask="ca_keypad",
                           mask_args={"lo": 2, "hi": 6, "masked_rows": 1}),
    "causal_offset": dict(seed=14, Hq=2, Hkv=1, Sq=5, Sk=9, causal=True, q_offset=3),
    "gqa4_random_bias": dict(seed=15, Hq=4, Hkv=1, Sq=6, Sk=7, mask="random",
                             mask_args={"Bm": 1, "p_masked": 0.25, "full_rows": 1, "full_cols": 1}),
    "causal_gqa_batch": dict(seed=16, B=2, Hq=4, Hkv=2, Sq=6, Sk=6, causal=True, q_offset=0),
}


@pytest.mark.parametrize("name", list(FD_CASES))
def test_finite_differences(name):
    c = _problem(**FD_CASES[name])
    q, k, v, do, m = _arrays(c)
    r = oracle.backward(q, k, v, do, m, scale=c.scale, causal=c.causal, q_offset=c.q_offset)
    assert np.abs(r["dQ"]).max() > 0 and np.abs(r["dK"]).max() > 0 and np.abs(r["dV"]).max() > 0

    def loss(a):
        O, _ = oracle.forward(a["q"], a["k"], a["v"], m, scale=c.scale, causal=c.causal,
                              q_offset=c.q_offset, threads=1)
        return float(np.sum(O * do))

    h = 1e-6
    for name_t, t, grad in (("q", q, r["dQ"]), ("k", k, r["dK"]), ("v", v, r["dV"])):
        fd = np.zeros_like(t)
        for idx in np.ndindex(t.shape):
            tp = t.copy()
            tp[idx] += h
            tm = t.copy()
            tm[idx] -= h
            fd[idx] = (loss({"q": q, "k": k, "v": v, name_t: tp})
                       - loss({"q": q, "k": k, "v": v, name_t: tm})) / (2 * h)
        err = np.abs(fd - grad).max() / max(np.abs(grad).max(), 1e-30)
        assert err < 1e-7, (name, name_t, err)


# ---------------------------------------------------------------------------
# an independent library routine: torch CPU float64 autograd, materialised softmax
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(FD_CASES))
def test_torch_autograd_crosscheck(name):
    torch = pytest.importorskip("torch")
    c = _problem(**FD_CASES[name])
    q, k, v, do, m = _arrays(c)
    r = oracle.backward(q, k, v, do, m, scale=c.scale, causal=c.causal, q_offset=c.q_offset)
    full, vis = _fully_masked_rows(c)
    G = c.Hq // c.Hkv
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    ke = tk.repeat_interleave(G, dim=1)
    ve = tv.repeat_interleave(G, dim=1)
    bias = torch.zeros((c.B, 1, c.Sq, c.Sk), dtype=torch.float64)
    if m is not None:
        bias = bias + torch.tensor(m)[:, None] if m.shape[0] == c.B else bias + torch.tensor(m)[None]
    bias = bias.masked_fill(~torch.tensor(vis)[:, None], float("-inf"))
    # keep fully masked rows finite for the library (it would give NaN there); they are
    # excluded from the comparison and from the loss below
    bias = bias.masked_fill(torch.tensor(full)[:, None, :, None], 0.0)
    s = torch.matmul(tq, ke.transpose(-1, -2).contiguous()) * c.scale + bias
    p = torch.softmax(s, dim=-1)
    o = torch.matmul(p, ve)
    lse = torch.logsumexp(s, dim=-1)
    keep = torch.tensor(~full)[:, None, :, None].to(torch.float64)
    (o * torch.tensor(do) * keep).sum().backward()
    keep_np = ~full[:, None, :]
    np.testing.assert_allclose(r["O"][np.broadcast_to(keep_np, r["LSE"].shape)],
                               o.detach().numpy()[np.broadcast_to(keep_np, r["LSE"].shape)], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["LSE"][np.broadcast_to(keep_np, r["LSE"].shape)],
                               lse.detach().numpy()[np.broadcast_to(keep_np, r["LSE"].shape)], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["dQ"], tq.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(r["dK"], tk.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(r["dV"], tv.grad.numpy(), rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
def test_single_key_closed_form():
    c = _problem(21, Hq=2, Hkv=1, Sq=5, Sk=1, D=4)
    q, k, v, do, _ = _arrays(c)
    r = oracle.backward(q, k, v, do, scale=c.scale)
    np.testing.assert_allclose(r["O"], np.broadcast_to(v.repeat(2, axis=1), r["O"].shape), rtol=0, atol=1e-15)
    lse = c.scale * np.einsum("bhid,bjd->bhi", q, k[:, 0])
    np.testing.assert_allclose(r["LSE"], lse, rtol=1e-14, atol=1e-14)
    assert np.abs(r["dQ"]).max() < 1e-14 and np.abs(r["dK"]).max() < 1e-14
    np.testing.assert_allclose(r["dV"][0, 0, 0], do[0].sum(axis=(0, 1)), rtol=1e-13, atol=1e-13)


def test_uniform_scores_closed_form():
    c = _problem(22, B=2, Hq=2, Hkv=2, Sq=4, Sk=9, D=3, mask="ca_keypad",
                 mask_args={"lo": 3, "hi": 8, "masked_rows": 1})
    q, k, v, do, m = _arrays(c)
    q = np.zeros_like(q)
    O, L = oracle.forward(q, k, v, m, scale=c.scale)
    full, vis = _fully_masked_rows(c)
    for b in range(c.B):
        for h in range(c.Hq):
            for i in range(c.Sq):
                if full[b, i]:
                    assert np.all(O[b, h, i] == 0) and L[b, h, i] == 0
                    continue
                js = np.nonzero(vis[b, i])[0]
                np.testing.assert_allclose(O[b, h, i], v[b, h][js].mean(axis=0), rtol=1e-14, atol=1e-14)
                assert abs(L[b, h, i] - math.log(len(js))) < 1e-14


def test_first_causal_row_closed_form():
    c = _problem(23, Hq=2, Hkv=2, Sq=6, Sk=6, D=5, causal=True, q_offset=0)
    q, k, v, _, _ = _arrays(c)
    O, L = oracle.forward(q, k, v, scale=c.scale, causal=True, q_offset=0)
    for h in range(2):
        np.testing.assert_allclose(O[0, h, 0], v[0, h, 0], rtol=0, atol=1e-15)
        assert abs(L[0, h, 0] - c.scale * float(q[0, h, 0] @ k[0, h, 0])) < 1e-14


def test_rows_sum_to_one_via_constant_values():
    c = _problem(24, B=2, Hq=4, Hkv=2, Sq=7, Sk=8, mask="random", mask_args={"Bm": 2})
    q, k, v, _, m = _arrays(c)
    O, _ = oracle.forward(q, k, np.ones_like(v), m, scale=c.scale)
    full, _ = _fully_masked_rows(c)
    for b in range(c.B):
        for i in range(c.Sq):
            want = 0.0 if full[b, i] else 1.0
            assert np.abs(O[b, :, i] - want).max() < 1e-13


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
def test_gradient_sum_invariants():
    c = _problem(31, B=2, Hq=4, Hkv=2, Sq=9, Sk=11, mask="random", mask_args={"Bm": 2, "full_rows": 2})
    r = _full(c)
    full, _ = _fully_masked_rows(c)
    do = c.f64("do")
    assert np.abs(r["dK"].sum(axis=2)).max() < 1e-13 * max(1.0, np.abs(r["dK"]).max())
    G = c.Hq // c.Hkv
    for b in range(c.B):
        for g in range(c.Hkv):
            want = sum(do[b, h][~full[b]].sum(axis=0) for h in range(g * G, (g + 1) * G))
            np.testing.assert_allclose(r["dV"][b, g].sum(axis=0), want, rtol=1e-12, atol=1e-12)
    # Delta equals sum_j P_ij dP_ij, i.e. <dO_i, O_i>
    np.testing.assert_allclose(r["Delta"], np.einsum("bhid,bhid->bhi", do, r["O"]), rtol=1e-13, atol=1e-13)


def test_mask_row_shift_and_key_permutation_and_linearity():
    c = _problem(32, B=1, Hq=2, Hkv=1, Sq=5, Sk=8, mask="random", mask_args={"Bm": 1, "full_rows": 0})
    q, k, v, do, m = _arrays(c)
    base = oracle.backward(q, k, v, do, m, scale=c.scale)
    # a constant added to one row's unmasked mask entries shifts that row's LSE only
    m2 = m.copy()
    m2[0, 2][np.isfinite(m2[0, 2])] += 3.25
    O2, L2 = oracle.forward(q, k, v, m2, scale=c.scale)
    np.testing.assert_allclose(O2, base["O"], rtol=1e-13, atol=1e-13)
    dl = L2 - base["LSE"]
    assert np.abs(dl[0, :, 2] - 3.25).max() < 1e-12 and np.abs(np.delete(dl, 2, axis=2)).max() < 1e-13
    # permuting keys permutes dK/dV and leaves O/LSE/dQ alone
    perm = np.random.default_rng(0).permutation(c.Sk)
    r = oracle.backward(q, k[:, :, perm], v[:, :, perm], do, m[:, :, perm], scale=c.scale)
    for n in ("O", "LSE", "dQ"):
        np.testing.assert_allclose(r[n], base[n], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["dK"], base["dK"][:, :, perm], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["dV"], base["dV"][:, :, perm], rtol=1e-12, atol=1e-12)
    # O is linear in V
    O3, _ = oracle.forward(q, k, 2.0 * v + 1.5 * np.flip(v, axis=3), m, scale=c.scale)
    O4, _ = oracle.forward(q, k, np.flip(v, axis=3), m, scale=c.scale)
    np.testing.assert_allclose(O3, 2.0 * base["O"] + 1.5 * O4, rtol=1e-12, atol=1e-12)


def test_exact_zeros_fully_masked_rows_and_columns():
    c = configs.make("dit_ca", B=2, Hq=2, Hkv=2, Sq=40, Sk=24, D=8)
    r = _full(c)
    full, vis = _fully_masked_rows(c)
    assert full.any() and (~vis.any(axis=1)).any()
    for b in range(c.B):
        rows = np.nonzero(full[b])[0]
        assert np.all(r["O"][b][:, rows] == 0) and np.all(r["LSE"][b][:, rows] == 0)
        assert np.all(r["dQ"][b][:, rows] == 0)
        cols = np.nonzero(~vis[b].any(axis=0))[0]
        assert cols.size > 0
        assert np.all(r["dK"][b][:, cols] == 0) and np.all(r["dV"][b][:, cols] == 0)
    assert np.abs(r["dK"]).max() > 0 and np.abs(r["dV"]).max() > 0


def test_sa_pad_mask_has_no_fully_masked_key_column():
    c = configs.make("dit_sa", Hq=2, Hkv=1, Sq=50, Sk=50, D=8)
    _, vis = _fully_masked_rows(c)
    assert vis.any(axis=1).all()
    assert c.meta["valid_len"] == 45


# ---------------------------------------------------------------------------
# GQA and the chunked walk
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("G", [2, 4])
def test_gqa_equals_group_sum_of_expanded_heads(G):
    c = _problem(41 + G, B=2, Hq=2 * G, Hkv=2, Sq=6, Sk=9, mask="random", mask_args={"Bm": 1})
    q, k, v, do, m = _arrays(c)
    r = oracle.backward(q, k, v, do, m, scale=c.scale)
    ke, ve = k.repeat(G, axis=1), v.repeat(G, axis=1)
    e = oracle.backward(q, ke, ve, do, m, scale=c.scale)
    for n in ("O", "LSE", "dQ"):
        np.testing.assert_allclose(r[n], e[n], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(r["dK"], e["dK"].reshape(2, 2, G, 9, -1).sum(axis=2), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["dV"], e["dV"].reshape(2, 2, G, 9, -1).sum(axis=2), rtol=1e-12, atol=1e-13)


def test_chunked_walk_equals_one_shot():
    W, C = 96, 16
    c = configs.make("long_window", W=W, Hq=4, Hkv=2, D=8)
    q, k, v, do, _ = _arrays(c)
    one = oracle.backward(q, k, v, do, scale=c.scale, causal=True, q_offset=0)
    dk = np.zeros_like(one["dK"])
    dv = np.zeros_like(one["dV"])
    for p0, n, sk in configs.chunk_plan(W, C):
        r = oracle.backward(q[:, :, p0:p0 + n], k[:, :, :sk], v[:, :, :sk], do[:, :, p0:p0 + n],
                            scale=c.scale, causal=True, q_offset=p0)
        for name in ("O", "LSE", "Delta", "dQ"):
            np.testing.assert_allclose(r[name], one[name][:, :, p0:p0 + n], rtol=1e-12, atol=1e-13)
        dk[:, :, :sk] += r["dK"]
        dv[:, :, :sk] += r["dV"]
    scale_k = np.abs(one["dK"]).max()
    assert np.abs(dk - one["dK"]).max() <= 1e-12 * scale_k
    assert np.abs(dv - one["dV"]).max() <= 1e-12 * np.abs(one["dV"]).max()


# ---------------------------------------------------------------------------
# the sampled entry points agree with the whole-problem entry point
# ---------------------------------------------------------------------------
def test_sampled_rows_and_columns_match_full():
    c = _problem(51, B=2, Hq=4, Hkv=2, Sq=10, Sk=12, mask="random", mask_args={"Bm": 2}, causal=True, q_offset=2)
    q, k, v, do, m = _arrays(c)
    full = oracle.backward(q, k, v, do, m, scale=c.scale, causal=True, q_offset=2)
    rng = np.random.default_rng(3)
    rows = rng.choice(c.B * c.Hq * c.Sq, 17, replace=False)
    rr = oracle.rows(q, k, v, do, rows, m, scale=c.scale, causal=True, q_offset=2)
    for n in ("O", "dQ"):
        np.testing.assert_allclose(rr[n], full[n].reshape(-1, c.D)[rows], rtol=1e-14, atol=1e-14)
    for n in ("LSE", "Delta"):
        np.testing.assert_allclose(rr[n], full[n].reshape(-1)[rows], rtol=1e-14, atol=1e-14)
    cols = rng.choice(c.B * c.Hkv * c.Sk, 13, replace=False)
    cc = oracle.cols(q, k, v, do, cols, m, scale=c.scale, causal=True, q_offset=2)
    np.testing.assert_allclose(cc["dK"], full["dK"].reshape(-1, c.D)[cols], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(cc["dV"], full["dV"].reshape(-1, c.D)[cols], rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------
# structured masks (key length, query length, sliding window): pinned to reductions
# that do not use the structured definition (slicing, closed forms)
# ---------------------------------------------------------------------------
def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_structured_key_length_equals_sliced_keys():
    B, H, Sq, Sk, D = 2, 2, 7, 9, 8
    q, k, v, do = _rand((B, H, Sq, D), 1), _rand((B, H, Sk, D), 2), _rand((B, H, Sk, D), 3), _rand((B, H, Sq, D), 4)
    klen = [5, 9]
    m = oracle.structured_mask(B, Sq, Sk, key_len=klen)
    ref = oracle.backward(q, k, v, do, m, scale=0.3)
    for b in range(B):
        kb = klen[b]
        one = oracle.backward(q[b:b + 1], k[b:b + 1, :, :kb], v[b:b + 1, :, :kb], do[b:b + 1], scale=0.3)
        for n in ("O", "LSE", "dQ"):
            np.testing.assert_allclose(ref[n][b:b + 1], one[n], rtol=1e-12, atol=1e-12)
        for n in ("dK", "dV"):
            np.testing.assert_allclose(ref[n][b:b + 1, :, :kb], one[n], rtol=1e-12, atol=1e-12)
            assert np.all(ref[n][b, :, kb:] == 0)  # keys past the length get nothing


def test_structured_query_length_rows_are_fully_masked():
    B, H, Sq, Sk, D = 2, 2, 6, 5, 8
    q, k, v, do = _rand((B, H, Sq, D), 5), _rand((B, H, Sk, D), 6), _rand((B, H, Sk, D), 7), _rand((B, H, Sq, D), 8)
    qlen = [6, 2]
    ref = oracle.backward(q, k, v, do, oracle.structured_mask(B, Sq, Sk, q_len=qlen), scale=0.4)
    b = 1
    for n in ("O", "dQ"):
        assert np.all(ref[n][b, :, 2:] == 0)
    assert np.all(ref["LSE"][b, :, 2:] == 0)
    one = oracle.backward(q[b:b + 1, :, :2], k[b:b + 1], v[b:b + 1], do[b:b + 1, :, :2], scale=0.4)
    for n in ("dK", "dV"):  # the masked rows add nothing
        np.testing.assert_allclose(ref[n][b:b + 1], one[n], rtol=1e-12, atol=1e-12)


def test_structured_zero_width_window_closed_form():
    # each row sees only the key at its own position: O_i = V_i, LSE_i = s <q_i, k_i>
    B, H, S, D = 1, 2, 6, 8
    q, k, v = _rand((B, H, S, D), 9), _rand((B, H, S, D), 10), _rand((B, H, S, D), 11)
    m = oracle.structured_mask(B, S, S, window_left=0, window_right=0)
    O, L = oracle.forward(q, k, v, m, scale=0.5)
    np.testing.assert_allclose(O, v, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(L, 0.5 * np.einsum("bhsd,bhsd->bhs", q, k), rtol=1e-13, atol=1e-13)


def test_structured_causal_window_equals_per_row_slices():
    # a causal sliding window of w: row i sees keys max(0, i + off - w) .. i + off
    B, H, Sq, Sk, D, w, off = 1, 2, 5, 9, 8, 3, 4
    q, k, v = _rand((B, H, Sq, D), 12), _rand((B, H, Sk, D), 13), _rand((B, H, Sk, D), 14)
    m = oracle.structured_mask(B, Sq, Sk, window_left=w, q_offset=off, causal=True)
    O, L = oracle.forward(q, k, v, m, scale=0.25, causal=True, q_offset=off)
    for i in range(Sq):
        lo, hi = max(0, i + off - w), i + off + 1
        Oi, Li = oracle.forward(q[:, :, i:i + 1], k[:, :, lo:hi], v[:, :, lo:hi], scale=0.25)
        np.testing.assert_allclose(O[:, :, i], Oi[:, :, 0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(L[:, :, i], Li[:, :, 0], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# attention sinks (one more logit per head in the softmax denominator, no value row):
# pinned to the same problem with the sink written as an extra key, to finite
# differences of the loss in the sink logits, and to closed forms
# ---------------------------------------------------------------------------
def _sink_problem(seed, B=2, Hq=4, Hkv=2, Sq=6, Sk=7, D=5, causal=False, q_offset=None, mask=True):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal(s) for s in ((B, Hq, Sq, D), (B, Hkv, Sk, D), (B, Hkv, Sk, D), (B, Hq, Sq, D)))
    m = None
    if mask:  # key padding with one fully masked row per sample
        m = np.zeros((B, Sq, Sk))
        m[0, :, Sk - 2:] = -np.inf
        m[1, 2, :] = -np.inf
    sinks = rng.standard_normal(Hq) + 0.5
    return q, k, v, do, m, sinks


@pytest.mark.parametrize("causal", [False, True])
def test_sinks_equal_an_extra_key_per_head(causal):
    """A sink is the score of one more key whose value row is zero: per query head, append a key with
    k = 0 (its product is 0) and the mask entry sink_h in every row, run the plain oracle on that head
    alone, and every output must agree (dK/dV summed over the group's heads, on the real keys)."""
    q, k, v, do, m, sinks = _sink_problem(21, causal=causal)
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    G, sc = Hq // Hkv, 0.45
    off = Sk - Sq if causal else None
    ref = oracle.backward(q, k, v, do, m, scale=sc, causal=causal, q_offset=off, sinks=sinks)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(Hq):
        g = h // G
        ke = np.concatenate([k[:, g:g + 1], np.zeros((B, 1, 1, D))], axis=2)
        ve = np.concatenate([v[:, g:g + 1], np.zeros((B, 1, 1, D))], axis=2)
        me = np.zeros((B, Sq, Sk + 1)) if m is None else np.concatenate([m, np.zeros((B, Sq, 1))], axis=2)
        me[:, :, Sk] = sinks[h]
        if causal:  # the real keys keep their causal visibility; the sink column is always visible
            i, j = np.arange(Sq)[:, None], np.arange(Sk)[None, :]
            me[:, :, :Sk] = np.where(j > (Sk - Sq) + i, -np.inf, me[:, :, :Sk])
        one = oracle.backward(q[:, h:h + 1], ke, ve, do[:, h:h + 1], me, scale=sc)
        for n in ("O", "LSE", "Delta", "dQ"):
            np.testing.assert_allclose(ref[n][:, h:h + 1], one[n], rtol=1e-12, atol=1e-12, err_msg=n)
        dk[:, g] += one["dK"][:, 0, :Sk]
        dv[:, g] += one["dV"][:, 0, :Sk]
    np.testing.assert_allclose(ref["dK"], dk, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ref["dV"], dv, rtol=1e-12, atol=1e-12)


def test_sink_gradient_finite_differences():
    """dSink_h against central differences of L = <O, dO> in the sink logits (float64)."""
    q, k, v, do, m, sinks = _sink_problem(22, Sq=5, Sk=6, D=4)
    sc = 0.6
    ref = oracle.backward(q, k, v, do, m, scale=sc, sinks=sinks)
    assert np.abs(ref["dSink"]).min() > 1e-6

    def loss(s):
        O, _ = oracle.forward(q, k, v, m, scale=sc, sinks=s, threads=1)
        return float(np.sum(O * do))

    h = 1e-6
    for i in range(len(sinks)):
        sp, sm = sinks.copy(), sinks.copy()
        sp[i] += h
        sm[i] -= h
        fd = (loss(sp) - loss(sm)) / (2 * h)
        assert abs(fd - ref["dSink"][i]) <= 1e-7 * max(1.0, abs(ref["dSink"][i])), (i, fd, ref["dSink"][i])
    # dQ / dK / dV with sinks also match finite differences (the sink changes P through the LSE)
    for name_t, t, grad in (("q", q, ref["dQ"]), ("v", v, ref["dV"])):
        idx = tuple(np.unravel_index(np.argmax(np.abs(grad)), grad.shape))
        tp, tm = t.copy(), t.copy()
        tp[idx] += h
        tm[idx] -= h
        args_p = {"q": q, "k": k, "v": v, name_t: tp}
        args_m = {"q": q, "k": k, "v": v, name_t: tm}
        Op, _ = oracle.forward(args_p["q"], args_p["k"], args_p["v"], m, scale=sc, sinks=sinks, threads=1)
        Om, _ = oracle.forward(args_m["q"], args_m["k"], args_m["v"], m, scale=sc, sinks=sinks, threads=1)
        fd = (np.sum(Op * do) - np.sum(Om * do)) / (2 * h)
        assert abs(fd - grad[idx]) <= 1e-7 * abs(grad[idx]), (name_t, fd, grad[idx])


def test_sink_closed_forms():
    """One key and a sink: P = sigmoid(s - sink), O = P v, LSE = log(exp(s) + exp(sink)). A row with every
    key masked keeps only the sink: O = 0, LSE = sink exactly, and its dQ is 0. A sink of -inf is no sink."""
    rng = np.random.default_rng(23)
    q, k, v, do = (rng.standard_normal((1, 1, 3, 4)), rng.standard_normal((1, 1, 1, 4)),
                   rng.standard_normal((1, 1, 1, 4)), rng.standard_normal((1, 1, 3, 4)))
    sinks = np.array([0.7])
    m = np.zeros((1, 3, 1))
    m[0, 1, 0] = -np.inf
    r = oracle.backward(q, k, v, do, m, scale=0.5, sinks=sinks)
    for i in (0, 2):
        s = 0.5 * float(q[0, 0, i] @ k[0, 0, 0])
        p = 1.0 / (1.0 + math.exp(sinks[0] - s))
        np.testing.assert_allclose(r["O"][0, 0, i], p * v[0, 0, 0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(r["LSE"][0, 0, i], math.log(math.exp(s) + math.exp(sinks[0])), rtol=1e-14)
    assert np.all(r["O"][0, 0, 1] == 0) and r["LSE"][0, 0, 1] == sinks[0] and np.all(r["dQ"][0, 0, 1] == 0)
    q2, k2, v2, do2, m2, _ = _sink_problem(24)
    a = oracle.backward(q2, k2, v2, do2, m2, scale=0.3)
    b = oracle.backward(q2, k2, v2, do2, m2, scale=0.3, sinks=np.full(4, -np.inf))
    for n in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.array_equal(a[n], b[n]), n


# ---------------------------------------------------------------------------
# q8_0 K/V window: the stored values, pinned to a block worked by hand, and the
# seeded quantizer's round trip on values already on the q8_0 grid
# ---------------------------------------------------------------------------
def test_q8_0_dequant_golden_block():
    with open(os.path.join(GOLDEN, "q8_0_blocks.json")) as f:
        g = json.load(f)
    t = np.arange(32)
    qs = np.concatenate([t - 16, 31 - 2 * t]).astype(np.int8)[None, None, None]
    d = np.array(g["d"], np.float16)[None, None, None]
    x = oracle.dequant_q8_0(qs, d)
    assert x.shape == (1, 1, 1, 64)
    for i, want in g["expect"].items():
        assert x[0, 0, 0, int(i)] == want, (i, x[0, 0, 0, int(i)], want)


def test_q8_0_quantizer_round_trip_on_grid_values():
    """Values d * q with d a power of two and max |q| = 127 in every block survive quantize -> dequantize
    exactly; values off the grid come back within half a step plus the fp16 rounding of the scale
    (d / 2 + 127 |d - fp16(d)|, with |d - fp16(d)| <= 2^-11 d)."""
    from flash_attention_train_amd.inputs import quantize_q8_0
    rng = np.random.default_rng(31)
    q = rng.integers(-127, 128, size=(2, 3, 5, 128))
    q[..., ::32] = 127  # every block reaches the end of the range
    d = 2.0 ** rng.integers(-6, 2, size=(2, 3, 5, 4))
    x = (np.repeat(d, 32, axis=-1) * q).astype(np.float32)
    qs, dh = quantize_q8_0(x)
    np.testing.assert_array_equal(oracle.dequant_q8_0(qs, dh), x.astype(np.float64))
    y = rng.standard_normal((3, 4, 64)).astype(np.float32)
    qs, dh = quantize_q8_0(y)
    back = oracle.dequant_q8_0(qs, dh)
    step = np.repeat(dh.astype(np.float64), 32, axis=-1)
    assert np.all(np.abs(back - y) <= step * (0.5 + 127 * 2.0 ** -11) * (1 + 1e-3))


# ---------------------------------------------------------------------------
# ALiBi slopes (S_ij gets -a_h |j - (q_offset + i)|): pinned to torch CPU float64
# autograd with the bias written out, to finite differences, and to the geometric
# series the LSE becomes when every raw score is zero
# ---------------------------------------------------------------------------
ALIBI_CASES = {
    "causal_gqa": dict(B=2, Hq=4, Hkv=2, Sq=6, Sk=6, causal=True, q_offset=0),
    "causal_offset": dict(B=1, Hq=2, Hkv=1, Sq=4, Sk=9, causal=True, q_offset=5),
    "bidirectional_masked": dict(B=2, Hq=2, Hkv=2, Sq=5, Sk=7, causal=False, q_offset=0, mask=True),
}


def _alibi_problem(name, seed):
    a = dict(ALIBI_CASES[name])
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, Sq, Sk, D = a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"], 5
    q, k, v, do = (rng.standard_normal(s) for s in ((B, Hq, Sq, D), (B, Hkv, Sk, D), (B, Hkv, Sk, D), (B, Hq, Sq, D)))
    m = None
    if a.get("mask"):
        m = np.zeros((B, Sq, Sk))
        m[1, :, Sk - 2:] = -np.inf
        m[0, 3, :] = -np.inf
    slopes = 2.0 ** (-8.0 * np.arange(1, Hq + 1) / Hq)
    return q, k, v, do, m, slopes, a["causal"], a["q_offset"]


@pytest.mark.parametrize("name", list(ALIBI_CASES))
def test_alibi_torch_autograd_crosscheck(name):
    torch = pytest.importorskip("torch")
    q, k, v, do, m, slopes, causal, off = _alibi_problem(name, 51)
    sc = 0.4
    r = oracle.backward(q, k, v, do, m, scale=sc, causal=causal, q_offset=off, alibi=slopes)
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    pos = off + np.arange(Sq)
    bias = -slopes[None, :, None, None] * np.abs(np.arange(Sk)[None, None, None, :] - pos[None, None, :, None])
    bias = np.broadcast_to(bias, (B, Hq, Sq, Sk)).copy()
    if m is not None:
        bias = bias + m[:, None]
    if causal:
        bias = np.where(np.arange(Sk)[None, None, None, :] > pos[None, None, :, None], -np.inf, bias)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = sc * torch.matmul(tq, tk.repeat_interleave(G, dim=1).transpose(-1, -2).contiguous()) + torch.tensor(bias)
    full = np.isinf(bias).all(axis=3)  # fully masked rows: the library gives NaN there, the oracle 0
    s = torch.where(torch.tensor(full)[..., None], torch.zeros_like(s), s)  # (kept finite, then dropped)
    p = torch.softmax(s, dim=-1)
    p = torch.where(torch.tensor(full)[..., None], torch.zeros_like(p), p)
    o = torch.matmul(p, tv.repeat_interleave(G, dim=1))
    lse = torch.logsumexp(s, dim=-1)
    (o * torch.tensor(do)).sum().backward()
    np.testing.assert_allclose(r["O"], o.detach().numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["LSE"][~full], lse.detach().numpy()[~full], rtol=1e-10, atol=1e-12)
    for n, t in (("dQ", tq), ("dK", tk), ("dV", tv)):
        np.testing.assert_allclose(r[n], t.grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=n)


def test_alibi_finite_differences():
    q, k, v, do, m, slopes, causal, off = _alibi_problem("causal_offset", 52)
    sc = 0.7
    r = oracle.backward(q, k, v, do, m, scale=sc, causal=causal, q_offset=off, alibi=slopes)

    def loss(a):
        O, _ = oracle.forward(a["q"], a["k"], a["v"], m, scale=sc, causal=causal, q_offset=off, alibi=slopes,
                              threads=1)
        return float(np.sum(O * do))

    h = 1e-6
    for name_t, t, grad in (("q", q, r["dQ"]), ("k", k, r["dK"]), ("v", v, r["dV"])):
        fd = np.zeros_like(t)
        for idx in np.ndindex(t.shape):
            tp, tm = t.copy(), t.copy()
            tp[idx] += h
            tm[idx] -= h
            fd[idx] = (loss({"q": q, "k": k, "v": v, name_t: tp}) - loss({"q": q, "k": k, "v": v, name_t: tm})) / (2 * h)
        assert np.abs(fd - grad).max() / np.abs(grad).max() < 1e-7, name_t


def test_alibi_zero_scores_geometric_series():
    """Q = 0 under a causal mask: row i sees keys 0..i with scores -a (i - j), so
    LSE_i = ln sum_{t=0}^{i} exp(-a t) = ln((1 - exp(-a (i + 1))) / (1 - exp(-a)))."""
    rng = np.random.default_rng(53)
    S, D = 7, 4
    q = np.zeros((1, 2, S, D))
    k, v = rng.standard_normal((1, 2, S, D)), rng.standard_normal((1, 2, S, D))
    slopes = np.array([0.5, 0.125])
    O, L = oracle.forward(q, k, v, scale=1.0, causal=True, q_offset=0, alibi=slopes)
    for h, a in enumerate(slopes):
        i = np.arange(S)
        np.testing.assert_allclose(L[0, h], np.log((1 - np.exp(-a * (i + 1))) / (1 - np.exp(-a))), rtol=1e-14)
        w = np.exp(-a * (S - 1 - np.arange(S)))  # last row's weights
        np.testing.assert_allclose(O[0, h, S - 1], (w / w.sum()) @ v[0, h], rtol=1e-13)


# ---------------------------------------------------------------------------
# a score bias per head (mask [Bm, Hq, Sq, Sk]): pinned to the heads run one by one
# with their own 3-D masks, and to finite differences
# ---------------------------------------------------------------------------
def _head_bias_problem(seed):
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, Sq, Sk, D = 2, 4, 2, 5, 6, 4
    q, k, v, do = (rng.standard_normal(s) for s in ((B, Hq, Sq, D), (B, Hkv, Sk, D), (B, Hkv, Sk, D), (B, Hq, Sq, D)))
    m = 0.7 * rng.standard_normal((B, Hq, Sq, Sk))
    m[0, 1, :, 2] = -np.inf      # a key column hidden in one head only
    m[1, 3, 4, :] = -np.inf      # a row fully masked in one head only
    return q, k, v, do, m


def test_head_bias_equals_heads_one_by_one():
    q, k, v, do, m = _head_bias_problem(61)
    ref = oracle.backward(q, k, v, do, m, scale=0.5)
    G = q.shape[1] // k.shape[1]
    dk, dv = np.zeros_like(k), np.zeros_like(v)
    for h in range(q.shape[1]):
        g = h // G
        one = oracle.backward(q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1], do[:, h:h + 1], m[:, h], scale=0.5)
        for n in ("O", "LSE", "Delta", "dQ"):
            np.testing.assert_allclose(ref[n][:, h:h + 1], one[n], rtol=1e-13, atol=1e-14, err_msg=n)
        dk[:, g] += one["dK"][:, 0]
        dv[:, g] += one["dV"][:, 0]
    np.testing.assert_allclose(ref["dK"], dk, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ref["dV"], dv, rtol=1e-12, atol=1e-13)
    assert np.all(ref["O"][1, 3, 4] == 0) and ref["LSE"][1, 3, 4] == 0  # fully masked in that head only
    assert np.any(ref["O"][1, 2, 4] != 0)
    # a per-head mask whose heads are all equal is the shared 3-D mask
    same = np.repeat(m[:, :1], q.shape[1], axis=1)
    a = oracle.backward(q, k, v, do, same, scale=0.5)
    b = oracle.backward(q, k, v, do, m[:, 0], scale=0.5)
    for n in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.array_equal(a[n], b[n]), n


def test_head_bias_finite_differences():
    q, k, v, do, m = _head_bias_problem(62)
    r = oracle.backward(q, k, v, do, m, scale=0.6)

    def loss(a):
        O, _ = oracle.forward(a["q"], a["k"], a["v"], m, scale=0.6, threads=1)
        return float(np.sum(O * do))

    h = 1e-6
    for name_t, t, grad in (("q", q, r["dQ"]), ("k", k, r["dK"]), ("v", v, r["dV"])):
        fd = np.zeros_like(t)
        for idx in np.ndindex(t.shape):
            tp, tm = t.copy(), t.copy()
            tp[idx] += h
            tm[idx] -= h
            fd[idx] = (loss({"q": q, "k": k, "v": v, name_t: tp}) - loss({"q": q, "k": k, "v": v, name_t: tm})) / (2 * h)
        assert np.abs(fd - grad).max() / np.abs(grad).max() < 1e-7, name_t


# ---------------------------------------------------------------------------
# logit softcap, S = c tanh(scale <q, k> / c) + mask: pinned to torch autograd on the
# materialised scores, to finite differences, and to its two limits (no cap as c grows;
# as c -> 0 the products vanish and the softmax runs over the mask alone, which also
# pins that the mask is added after the cap)
# ---------------------------------------------------------------------------
def _softcap_problem(seed, causal, mask):
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, Sq, Sk, D = 2, 4, 2, 6, 7, 5
    q, k, v, do = (rng.standard_normal(s) for s in ((B, Hq, Sq, D), (B, Hkv, Sk, D), (B, Hkv, Sk, D), (B, Hq, Sq, D)))
    q *= 2.0  # products of a few units: well inside tanh's bend for c = 1.5
    m = None
    if mask:
        m = rng.standard_normal((B, Sq, Sk))  # finite biases, plus hidden entries
        m[1, :, Sk - 2:] = -np.inf
        m[0, 3, :] = -np.inf
    return q, k, v, do, m, causal, (Sk - Sq if causal else 0)


@pytest.mark.parametrize("causal,mask", [(False, False), (True, True)])
def test_softcap_torch_autograd_crosscheck(causal, mask):
    torch = pytest.importorskip("torch")
    q, k, v, do, m, causal, off = _softcap_problem(61, causal, mask)
    sc, cap = 0.6, 1.5
    r = oracle.backward(q, k, v, do, m, scale=sc, causal=causal, q_offset=off, softcap=cap)
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    bias = np.zeros((B, Hq, Sq, Sk))
    if m is not None:
        bias = bias + m[:, None]
    if causal:
        pos = off + np.arange(Sq)
        bias = np.where(np.arange(Sk)[None, None, None, :] > pos[None, None, :, None], -np.inf, bias)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    x = sc * torch.matmul(tq, tk.repeat_interleave(G, dim=1).transpose(-1, -2).contiguous())
    s = cap * torch.tanh(x / cap) + torch.tensor(bias)
    full = np.isinf(bias).all(axis=3)
    s = torch.where(torch.tensor(full)[..., None], torch.zeros_like(s), s)  # (kept finite, then dropped)
    p = torch.softmax(s, dim=-1)
    p = torch.where(torch.tensor(full)[..., None], torch.zeros_like(p), p)
    o = torch.matmul(p, tv.repeat_interleave(G, dim=1))
    lse = torch.logsumexp(s, dim=-1)
    (o * torch.tensor(do)).sum().backward()
    assert np.abs(x.detach().numpy()).max() > 2 * cap  # the cap is active
    np.testing.assert_allclose(r["O"], o.detach().numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["LSE"][~full], lse.detach().numpy()[~full], rtol=1e-10, atol=1e-12)
    for n, t in (("dQ", tq), ("dK", tk), ("dV", tv)):
        np.testing.assert_allclose(r[n], t.grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=n)


def test_softcap_finite_differences():
    q, k, v, do, m, causal, off = _softcap_problem(62, True, True)
    sc, cap = 0.6, 1.5
    r = oracle.backward(q, k, v, do, m, scale=sc, causal=causal, q_offset=off, softcap=cap)

    def loss(a):
        O, _ = oracle.forward(a["q"], a["k"], a["v"], m, scale=sc, causal=causal, q_offset=off, softcap=cap,
                              threads=1)
        return float(np.sum(O * do))

    h = 1e-6
    for name_t, t, grad in (("q", q, r["dQ"]), ("k", k, r["dK"]), ("v", v, r["dV"])):
        fd = np.zeros_like(t)
        for idx in np.ndindex(t.shape):
            tp, tm = t.copy(), t.copy()
            tp[idx] += h
            tm[idx] -= h
            fd[idx] = (loss({"q": q, "k": k, "v": v, name_t: tp}) - loss({"q": q, "k": k, "v": v, name_t: tm})) / (2 * h)
        assert np.abs(fd - grad).max() / np.abs(grad).max() < 1e-7, name_t


def test_softcap_limits():
    q, k, v, do, m, causal, off = _softcap_problem(63, True, True)
    sc = 0.6
    plain = oracle.backward(q, k, v, do, m, scale=sc, causal=causal, q_offset=off)
    wide = oracle.backward(q, k, v, do, m, scale=sc, causal=causal, q_offset=off, softcap=1e7)
    for n in ("O", "LSE", "Delta", "dQ", "dK", "dV"):
        np.testing.assert_allclose(wide[n], plain[n], rtol=1e-10, atol=1e-12, err_msg=n)
    # c -> 0: S_ij -> M_ij, P = softmax of the visible mask values, and the product's gradient
    # carries a factor c, so dQ and dK vanish with it
    c = 1e-9
    r = oracle.backward(q, k, v, do, m, scale=sc, causal=causal, q_offset=off, softcap=c)
    B, Hq, Sq, _ = q.shape
    Sk = k.shape[2]
    G = Hq // k.shape[1]
    for b in range(B):
        for h in range(Hq):
            for i in range(Sq):
                mv = m[b, i].copy()
                mv[np.arange(Sk) > off + i] = -np.inf
                if np.isinf(mv).all():
                    assert r["LSE"][b, h, i] == 0 and np.all(r["O"][b, h, i] == 0)
                    continue
                mx = mv[np.isfinite(mv)].max()
                w = np.where(np.isfinite(mv), np.exp(mv - mx), 0.0)
                np.testing.assert_allclose(r["LSE"][b, h, i], mx + np.log(w.sum()), rtol=0, atol=1e-8)
                np.testing.assert_allclose(r["O"][b, h, i], (w / w.sum()) @ v[b, h // G], rtol=0, atol=1e-8)
    assert np.abs(r["dQ"]).max() < 1e-7 and np.abs(r["dK"]).max() < 1e-7
    assert np.abs(r["dV"]).max() > 0.1
    with pytest.raises(ValueError):
        oracle.forward(q, k, v, scale=sc, softcap=-1.0)


# ---------------------------------------------------------------------------
# gradient of the additive mask (a learnable KQ bias): dM = P (dP - Delta) per entry,
# summed over the dimensions the mask is broadcast over
# ---------------------------------------------------------------------------
def _bias_problem(seed, B=2, Hq=4, Hkv=2, Sq=5, Sk=6, D=4, heads=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Sq, D))
    k = rng.standard_normal((B, Hkv, Sk, D))
    v = rng.standard_normal((B, Hkv, Sk, D))
    do = rng.standard_normal((B, Hq, Sq, D))
    m = 0.7 * rng.standard_normal((B, Hq, Sq, Sk) if heads else (1, Sq, Sk))
    if heads:
        m[0, 1, 2, 3] = -np.inf
        m[1, 3, 4, :] = -np.inf  # a fully masked row in one head
    else:
        m[0, 2, 3] = -np.inf
    return q, k, v, do, m


@pytest.mark.parametrize("heads,causal,cap", [(True, False, None), (False, False, None), (True, True, 2.5),
                                             (False, True, None)])
def test_bias_gradient_finite_differences(heads, causal, cap):
    """dM against central differences of L = <O, dO> in every finite mask entry (float64), with a
    per-head and a batch- and head-shared mask (whose gradient sums over both), causal masking,
    a logit softcap (the mask is added after the cap: no cap' factor) and ALiBi."""
    q, k, v, do, m = _bias_problem(31 + int(heads) + 2 * int(causal), heads=heads)
    sc = 0.45
    al = np.array([0.1, 0.2, 0.05, 0.3])
    g = oracle.bias_grad(q, k, v, do, m, scale=sc, causal=causal, alibi=al, softcap=cap)
    assert g.shape == m.shape
    assert np.all(g[~np.isfinite(m)] == 0)

    def loss(mm):
        O, _ = oracle.forward(q, k, v, mm, scale=sc, causal=causal, alibi=al, softcap=cap, threads=1)
        return float(np.sum(O * do))

    h = 1e-6
    fd = np.zeros_like(g)
    for idx in zip(*np.nonzero(np.isfinite(m))):
        mp, mn = m.copy(), m.copy()
        mp[idx] += h
        mn[idx] -= h
        fd[idx] = (loss(mp) - loss(mn)) / (2 * h)
    err = np.abs(fd - g).max() / np.abs(g).max()
    assert err < 1e-6, err


def test_bias_gradient_rows_sum_to_zero_and_match_dq():
    """Two closed forms of dM = P (dP - Delta) without a sink: every row of one head sums to 0
    (sum_j P_ij dP_ij = Delta_i and sum_j P_ij = 1), and for a per-head mask without a cap,
    dQ_i = scale sum_j dM_ij k_j, which the oracle's backward computes by a separate route."""
    q, k, v, do, m = _bias_problem(41, heads=True)
    sc = 0.6
    g = oracle.bias_grad(q, k, v, do, m, scale=sc)
    ref = oracle.backward(q, k, v, do, m, scale=sc)
    np.testing.assert_allclose(g.sum(axis=-1), 0.0, atol=1e-12)
    G = q.shape[1] // k.shape[1]
    dq = sc * np.einsum("bhij,bhjd->bhid", g, np.repeat(k, G, axis=1))
    np.testing.assert_allclose(dq, ref["dQ"], rtol=1e-10, atol=1e-12)
