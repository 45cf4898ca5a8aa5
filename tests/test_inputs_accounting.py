"""Host-side checks of the input generators, mask builders, the chunk plan and the
work accounting (no GPU)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from flash_attention_train_amd import accounting as A
from flash_attention_train_amd import configs
from flash_attention_train_amd.inputs import F32, bf16_bits_to_f32, f32_to_bf16_bits, make_case


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-6, 6, 100000),
                        np.array([0.0, -0.0, 1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 65504.0], np.float32)])
    mine = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    back = bf16_bits_to_f32(mine)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generators_are_deterministic_and_seeded():
    a = configs.make("dit_ca", B=2, Hq=2, Hkv=2, Sq=33, Sk=20, D=8)
    b = configs.make("dit_ca", B=2, Hq=2, Hkv=2, Sq=33, Sk=20, D=8)
    for n in ("q", "k", "v", "do", "mask"):
        assert np.array_equal(getattr(a, n), getattr(b, n))
    c = make_case("x", B=1, Hq=1, Hkv=1, Sq=4, Sk=4, D=8, dtype="bf16", seed=1)
    d = make_case("x", B=1, Hq=1, Hkv=1, Sq=4, Sk=4, D=8, dtype="bf16", seed=2)
    assert not np.array_equal(c.q, d.q)


def test_full_size_masks_follow_the_workload_description():
    sa = configs.make("dit_sa", Hq=2, Hkv=1, D=8)
    assert sa.mask.shape == (1, 1542, 1542) and sa.meta["valid_len"] == 1388
    fin = np.isfinite(sa.mask[0])
    assert fin[:1388, :1388].all() and not fin[:1388, 1388:].any() and fin[1388:].all()
    ca = configs.make("dit_ca", Hq=2, Hkv=2, D=8)
    assert ca.mask.shape == (2, 1542, 512)
    for b, (L, rows) in enumerate(zip(ca.meta["valid_lens"], ca.meta["masked_rows"])):
        assert 128 <= L <= 512 and len(rows) == 2
        fin = np.isfinite(ca.mask[b])
        assert not fin[rows].any()
        keep = np.setdiff1d(np.arange(1542), rows)
        assert fin[keep, :L].all() and not fin[:, L:].any()


def test_pair_counts_match_brute_force():
    for causal, q_offset in ((False, 0), (True, 0), (True, 5)):
        c = make_case("x", B=2, Hq=3, Hkv=1, Sq=9, Sk=14, D=4, dtype="f32", seed=7, mask="random",
                      mask_args={"Bm": 2}, causal=causal, q_offset=q_offset)
        n = 0
        for b in range(c.B):
            for i in range(c.Sq):
                for j in range(c.Sk):
                    if np.isfinite(c.mask[b, i, j]) and (not causal or j <= q_offset + i):
                        n += 1
        assert A.case_pairs(c) == n * c.Hq


def test_headline_pair_counts():
    assert A.unmasked_pairs(1, 16, 1542, 1542, False, 0, configs.make("dit_sa", Hq=1, Hkv=1, D=8).mask) == 34_624_192
    assert A.unmasked_pairs(1, 32, 4096, 4096, True, 0, None) == 268_500_992
    assert A.chunked_pairs(16, 32768, 512) == 8_590_196_736
    assert A.unmasked_pairs(1, 16, 32768, 32768, True, 0, None) == 8_590_196_736


def test_chunk_plan():
    plan = configs.chunk_plan()
    assert len(plan) == 64
    assert plan[0] == (0, 512, 512) and plan[-1] == (32256, 512, 32768)
    with pytest.raises(ValueError):
        configs.chunk_plan(1000, 512)


@pytest.mark.parametrize("seed", range(6))
def test_structured_pair_counts_brute_force(seed):
    """Closed-form visible-key counts of a structured mask against an entry-by-entry count
    of the definition on small random structures (lengths, windows, offsets, causal)."""
    rng = np.random.default_rng(seed)
    Sq, Sk = int(rng.integers(1, 40)), int(rng.integers(1, 40))
    causal = bool(rng.integers(0, 2))
    q_offset = int(rng.integers(-10, 20))
    wl, wr = (int(x) for x in rng.integers(-1, 12, size=2))
    kl, ql = int(rng.integers(0, Sk + 1)), int(rng.integers(0, Sq + 1))
    n = A.structured_counts(Sq, Sk, causal, q_offset, kl, ql, wl, wr)
    for i in range(Sq):
        pos = q_offset + i
        want = 0
        for j in range(Sk):
            ok = i < ql and j < kl and (wl < 0 or j >= pos - wl) and (wr < 0 or j <= pos + wr)
            ok = ok and (not causal or j <= pos)
            want += ok
        assert n[i] == want, (i, n[i], want)


@pytest.mark.parametrize("key", ["dit_sa_len", "dit_sa_band"])
def test_structured_workload_pairs_match_the_dense_definition(key):
    c = configs.make(key, Hq=1, Hkv=1, D=8)
    st = c.meta["structure"]
    m = oracle.structured_mask(c.B, c.Sq, c.Sk, key_len=st["key_len"], q_len=st["q_len"],
                               window_left=st["window"][0], window_right=st["window"][1], q_offset=c.q_offset)
    assert A.case_pairs(c) == int(np.isfinite(m).sum())


def test_every_workload_draws_deterministically_at_a_small_size():
    """Each entry of the workload table can be drawn at a small size, twice with the same values,
    and the bench's default workloads all come from the table."""
    import bench
    assert set(bench.DEFAULT_EXTRA) <= set(configs.WORKLOADS)
    small = {"long_window": dict(W=256, Hq=2, Hkv=1, D=64), "lm": dict(Sq=96, Sk=96, Hq=4, Hkv=2, D=64),
             "dit": dict(Hq=2, Hkv=1, D=64)}
    for key in configs.WORKLOADS:
        kw = small["long_window"] if key.startswith("long_window") else small["lm"] if key.startswith("lm") \
            else small["dit"]
        a, b = configs.make(key, **kw), configs.make(key, **kw)
        for n in ("q", "k", "v", "do"):
            assert np.array_equal(getattr(a, n), getattr(b, n)), (key, n)
        assert a.q.shape[1] == kw["Hq"] and a.k.shape[1] == kw["Hkv"], key


def test_f16_window_holds_the_draws_rounded_once():
    c = configs.make("long_window_f16", W=256, Hq=2, Hkv=1, D=64)
    full = configs.make("long_window_f16", W=256, Hq=2, Hkv=1, D=64, dtype=F32)
    for n in ("k", "v"):
        w = c.meta["f16"][n]
        assert w.dtype == np.float16
        x = full.f64(n)
        # nearest fp16: within half a unit in the last place of the value (normal range)
        ulp = np.spacing(np.abs(w).astype(np.float16)).astype(np.float64)
        assert np.all(np.abs(w.astype(np.float64) - x) <= 0.5 * ulp + 1e-30)
        # the case's own bf16 K / V are those fp16 values rounded to bf16
        np.testing.assert_array_equal(getattr(c, n), f32_to_bf16_bits(w.astype(np.float32)))
    assert configs.make("lm_softcap", Sq=64, Sk=64, Hq=2, Hkv=1, D=64).meta["softcap"] == 50.0
