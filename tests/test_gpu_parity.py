"""GPU parity at sizes the oracle finishes in seconds: every output of the HIP
path (O, LSE, Delta, dQ, dK, dV) against the oracle, element by element, on
shapes that span several tiles and end in a ragged tail; plus the degenerate and
structural cases (fully masked rows and columns, GQA, causal offsets, strided
views, broadcast masks, fp32 and bf16, D = 64 and 128)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from flash_attention_train_amd import binding, configs
from flash_attention_train_amd.inputs import make_case
from parity_util import TOL, compare_full, dev, host64, run_gpu, say, upload

pytestmark = pytest.mark.gpu


def oracle_full(c):
    m = None if c.mask is None else c.mask.astype(np.float64)
    return oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), m, scale=c.scale, causal=c.causal,
                           q_offset=c.q_offset)


CASES = {
    # the tiny fp32 workload, exactly as specified
    "tiny_f32": lambda: configs.make("tiny"),
    # workload structures at reduced head counts and ragged lengths
    "dit_sa_ragged": lambda: configs.make("dit_sa", Hq=4, Hkv=2, Sq=300, Sk=300),
    "dit_ca_ragged": lambda: configs.make("dit_ca", B=2, Hq=2, Hkv=2, Sq=300, Sk=160),
    "lm_causal_gqa4": lambda: configs.make("lm_causal", Hq=4, Hkv=1, Sq=333, Sk=333),
    "chunk_offset": lambda: make_case("chunk_offset", B=1, Hq=4, Hkv=2, Sq=100, Sk=356, D=128, dtype="bf16",
                                      seed=61, causal=True, q_offset=256),
    "random_bias_bcast": lambda: make_case("random_bias_bcast", B=2, Hq=2, Hkv=1, Sq=130, Sk=70, D=128,
                                           dtype="bf16", seed=62, mask="random",
                                           mask_args={"Bm": 1, "full_rows": 3, "full_cols": 2}),
    "d64_bf16": lambda: make_case("d64_bf16", B=2, Hq=4, Hkv=4, Sq=200, Sk=129, D=64, dtype="bf16", seed=63,
                                  mask="random", mask_args={"Bm": 2, "p_masked": 0.5}),
    "d128_f32_causal": lambda: make_case("d128_f32_causal", B=1, Hq=2, Hkv=1, Sq=150, Sk=150, D=128, dtype="f32",
                                         seed=64, causal=True),
    "f32_d64_gqa_mask": lambda: make_case("f32_d64_gqa_mask", B=2, Hq=4, Hkv=2, Sq=70, Sk=90, D=64, dtype="f32",
                                          seed=65, mask="ca_keypad", mask_args={"lo": 10, "hi": 60,
                                                                                "masked_rows": 2}),
    "single_query_single_key": lambda: make_case("one_one", B=1, Hq=2, Hkv=1, Sq=1, Sk=1, D=128, dtype="bf16",
                                                 seed=66),
    "causal_q_before_keys": lambda: make_case("causal_negative_offset", B=1, Hq=2, Hkv=2, Sq=80, Sk=40, D=64,
                                              dtype="f32", seed=67, causal=True),  # q_offset = -40
    # whole dK/dV units (no per-element masking) whose only row tile holds one row, or ends one
    # row into a second tile: the rows past the end must contribute nothing
    "one_query_many_keys": lambda: make_case("one_many", B=1, Hq=2, Hkv=1, Sq=1, Sk=300, D=128, dtype="bf16",
                                             seed=68),
    "row_tail_of_one": lambda: make_case("row_tail_one", B=2, Hq=2, Hkv=2, Sq=65, Sk=256, D=64, dtype="bf16",
                                         seed=69),
}


@pytest.mark.parametrize("name", list(CASES))
def test_parity_small(name):
    c = CASES[name]()
    say(f"case {name}: B={c.B} Hq={c.Hq} Hkv={c.Hkv} Sq={c.Sq} Sk={c.Sk} D={c.D} {c.dtype} causal={c.causal} "
        f"q_offset={c.q_offset} mask={c.meta['mask_kind']}")
    got = run_gpu(c)
    ref = oracle_full(c)
    compare_full(c, got, ref, zero_ok=("dQ", "dK") if c.Sk == 1 else ())


def test_deterministic_outputs():
    """With unsplit backward work every output is stored once by one workgroup: two runs
    agree bitwise on every output (split work also sums fixed fp32 slices in a fixed order)."""
    c = CASES["dit_ca_ragged"]()
    t = upload(c)

    def once():
        o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale)
        delta = binding.bwd_preprocess(o, t["do"])
        grads = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=t["mask"], scale=c.scale,
                            kv_split=1, q_split=1)
        torch.cuda.synchronize()
        return [host64(x) for x in (o, lse, delta, *grads)]

    for x, y, n in zip(once(), once(), ("O", "LSE", "Delta", "dQ", "dK", "dV")):
        assert np.array_equal(x, y), n


def test_pad_invariance_bitwise():
    """Changing K/V at pad keys leaves every real row's O and LSE bitwise unchanged
    (the pages' dirty-padding check, HOT-Step TRAINING.md, batching paragraph)."""
    c = configs.make("dit_sa", Hq=2, Hkv=1, Sq=200, Sk=200)
    L = c.meta["valid_len"]
    t = upload(c)
    o1, l1 = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale)
    k2, v2 = t["k"].clone(), t["v"].clone()
    k2[:, :, L:] = 7.0
    v2[:, :, L:] = -3.0
    o2, l2 = binding.fwd(t["q"], k2, v2, mask=t["mask"], scale=c.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :, :L], o2[:, :, :L]) and torch.equal(l1[:, :, :L], l2[:, :, :L])


def test_strided_views():
    """[B, S, H, D] memory order (permuted views) gives the same results as contiguous."""
    c = configs.make("dit_sa", Hq=4, Hkv=2, Sq=150, Sk=150)
    t = upload(c)

    def bshd(x):
        return x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)

    q, k, v, do = (bshd(t[n]) for n in ("q", "k", "v", "do"))
    assert q.stride(1) == c.D and not q.is_contiguous()
    o, lse = binding.fwd(q, k, v, mask=t["mask"], scale=c.scale, out=bshd(torch.empty_like(t["q"])))
    delta = binding.bwd_preprocess(o, do)
    dq, dk, dv = binding.bwd(q, k, v, do, lse, delta, mask=t["mask"], scale=c.scale,
                             dq=bshd(torch.empty_like(t["q"])), dk=bshd(torch.empty_like(t["k"])),
                             dv=bshd(torch.empty_like(t["v"])), kv_split=1, q_split=1)
    torch.cuda.synchronize()
    ref = run_gpu(c, t, kv_split=1, q_split=1)
    for n, x in (("O", o), ("LSE", lse), ("Delta", delta), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert np.array_equal(host64(x), ref[n]), n


def test_chunked_walk_small():
    """Eight 128-row chunks over a 1024-key window, dK/dV accumulated in fp32 on the
    device, against the one-shot oracle (the exact walk, llama.cpp PR 57)."""
    W, C = 1024, 128
    c = configs.make("long_window", W=W, Hq=4, Hkv=2)
    t = upload(c)
    dk_acc = torch.zeros((1, c.Hkv, W, c.D), dtype=torch.float32, device="cuda")
    dv_acc = torch.zeros_like(dk_acc)
    O = torch.empty_like(t["q"])
    LSE = torch.empty((1, c.Hq, W), dtype=torch.float32, device="cuda")
    Delta = torch.empty_like(LSE)
    dQ = torch.empty_like(t["q"])
    for p0, n, sk in configs.chunk_plan(W, C):
        q = t["q"][:, :, p0:p0 + n]
        do = t["do"][:, :, p0:p0 + n]
        kk, vv = t["k"][:, :, :sk], t["v"][:, :, :sk]
        o, lse = binding.fwd(q, kk, vv, scale=c.scale, causal=True, q_offset=p0, out=O[:, :, p0:p0 + n],
                             lse=LSE[:, :, p0:p0 + n])
        delta = binding.bwd_preprocess(o, do, delta=Delta[:, :, p0:p0 + n])
        binding.bwd_chunked(q, kk, vv, do, lse, delta, dk_acc, dv_acc, scale=c.scale, causal=True, q_offset=p0,
                            dq=dQ[:, :, p0:p0 + n])
    torch.cuda.synchronize()
    ref = oracle_full(c)
    got = {"O": host64(O), "LSE": host64(LSE), "Delta": host64(Delta), "dQ": host64(dQ),
           "dK": dk_acc.cpu().numpy().astype(np.float64), "dV": dv_acc.cpu().numpy().astype(np.float64)}
    compare_full(c, got, ref)
    # the accumulated gradient is a sum over chunks: the same walk in another order agrees
    dk2 = torch.zeros_like(dk_acc)
    dv2 = torch.zeros_like(dv_acc)
    for p0, n, sk in reversed(configs.chunk_plan(W, C)):
        binding.bwd_chunked(t["q"][:, :, p0:p0 + n], t["k"][:, :, :sk], t["v"][:, :, :sk], t["do"][:, :, p0:p0 + n],
                            LSE[:, :, p0:p0 + n], Delta[:, :, p0:p0 + n], dk2, dv2, scale=c.scale, causal=True,
                            q_offset=p0)
    torch.cuda.synchronize()
    assert np.abs(dk2.cpu().numpy() - dk_acc.cpu().numpy()).max() <= 1e-5 * np.abs(got["dK"]).max()


@pytest.mark.parametrize("config", [1, 2, 3])
@pytest.mark.parametrize("name", ["dit_sa_ragged", "dit_ca_ragged", "lm_causal_gqa4", "chunk_offset",
                                  "random_bias_bcast", "d64_bf16", "single_query_single_key"])
def test_forward_variants(name, config):
    """Every bf16 forward configuration (32 or 64 query rows per wave; keys split over two
    halves of the workgroup, merged at the end) against the oracle."""
    c = CASES[name]()
    t = upload(c)
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal,
                         q_offset=c.q_offset, variant=config, split=1)
    torch.cuda.synchronize()
    m = None if c.mask is None else c.mask.astype(np.float64)
    O, L = oracle.forward(c.f64("q"), c.f64("k"), c.f64("v"), m, scale=c.scale, causal=c.causal,
                          q_offset=c.q_offset)
    compare_full(c, {"O": host64(o), "LSE": host64(lse)}, {"O": O, "LSE": L}, names=("O", "LSE"))


@pytest.mark.parametrize("split", [2, 3, 7])
@pytest.mark.parametrize("name", ["dit_sa_ragged", "dit_ca_ragged", "lm_causal_gqa4", "chunk_offset",
                                  "random_bias_bcast", "d64_bf16", "single_query_single_key"])
def test_forward_splits(name, split):
    """The split-key forward (each query tile's key walk over `split` workgroups, partial rows merged)
    against the oracle, fully masked rows exact; splits that see no key contribute nothing."""
    c = CASES[name]()
    t = upload(c)
    ws = torch.empty(max(1, binding.fwd_workspace_bytes(t["q"], t["k"], scale=c.scale, causal=c.causal,
                                                        q_offset=c.q_offset, mask=t["mask"], split=split)),
                     dtype=torch.uint8, device="cuda")
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal,
                         q_offset=c.q_offset, workspace=ws, split=split)
    torch.cuda.synchronize()
    m = None if c.mask is None else c.mask.astype(np.float64)
    O, L = oracle.forward(c.f64("q"), c.f64("k"), c.f64("v"), m, scale=c.scale, causal=c.causal,
                          q_offset=c.q_offset)
    compare_full(c, {"O": host64(o), "LSE": host64(lse)}, {"O": O, "LSE": L}, names=("O", "LSE"))


@pytest.mark.parametrize("name", ["tiny_f32", "d128_f32_causal", "f32_d64_gqa_mask", "dit_sa_ragged", "dit_ca_ragged",
                                  "lm_causal_gqa4", "chunk_offset", "single_query_single_key"])
def test_forward_entry_without_workspace(name):
    """fa_train_fwd itself (the forward entry point that takes no workspace), bf16 and fp32, against
    the oracle; and the same bits as fa_train_fwd_ws with the split pinned to 1."""
    c = CASES[name]()
    say(f"case {name}: fa_train_fwd, B={c.B} Hq={c.Hq} Hkv={c.Hkv} Sq={c.Sq} Sk={c.Sk} D={c.D} {c.dtype}")
    t = upload(c)
    o, lse = binding.fwd_unsplit(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal,
                                 q_offset=c.q_offset)
    o1, lse1 = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal,
                           q_offset=c.q_offset, split=1)
    torch.cuda.synchronize()
    m = None if c.mask is None else c.mask.astype(np.float64)
    O, L = oracle.forward(c.f64("q"), c.f64("k"), c.f64("v"), m, scale=c.scale, causal=c.causal,
                          q_offset=c.q_offset)
    compare_full(c, {"O": host64(o), "LSE": host64(lse)}, {"O": O, "LSE": L}, names=("O", "LSE"))
    assert torch.equal(o, o1) and torch.equal(lse, lse1)


def test_forward_split_hint_ignored_for_fp32():
    """The fp32 forward is never split: a split hint through the workspace entry point needs no
    workspace and gives the unsplit results."""
    c = CASES["f32_d64_gqa_mask"]()
    t = upload(c)
    assert binding.fwd_workspace_bytes(t["q"], t["k"], scale=c.scale, mask=t["mask"], split=3) == 0
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, split=3)
    o1, lse1 = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, split=1)
    torch.cuda.synchronize()
    assert torch.equal(o, o1) and torch.equal(lse, lse1)


@pytest.mark.parametrize("dq_launch", [1, 2, 3, 4])
@pytest.mark.parametrize("kv_split,q_split", [(1, 1), (3, 1), (1, 2), (2, 5)])
@pytest.mark.parametrize("name", ["dit_sa_ragged", "lm_causal_gqa4", "random_bias_bcast", "d64_bf16"])
def test_backward_decompositions(name, kv_split, q_split, dq_launch):
    """Every split of the bf16 backward's work (direct stores, or fp32 partial slices summed by a reduce
    pass), with the dQ workgroups in the dK/dV launch (1), in a launch of their own (2), forming dQ
    from the dS the dK/dV walk stored (3), or in their own launch on a second stream beside the dK/dV
    launch (4), gives the oracle's gradients."""
    c = CASES[name]()
    t = upload(c)
    say(f"case {name}: kv_split {kv_split} q_split {q_split} dq_launch {dq_launch}")
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal,
                         q_offset=c.q_offset)
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=t["mask"], scale=c.scale,
                             causal=c.causal, q_offset=c.q_offset, kv_split=kv_split, q_split=q_split,
                             dq_launch=dq_launch)
    torch.cuda.synchronize()
    ref = oracle_full(c)
    compare_full(c, {"dQ": host64(dq), "dK": host64(dk), "dV": host64(dv)}, ref, names=("dQ", "dK", "dV"))


@pytest.mark.parametrize("kv_split,q_split", [(1, 1), (3, 2)])
@pytest.mark.parametrize("name", ["tiny_f32", "dit_sa_ragged", "dit_ca_ragged", "lm_causal_gqa4", "chunk_offset",
                                  "random_bias_bcast", "d64_bf16", "single_query_single_key", "causal_q_before_keys"])
def test_backward_role_split_walk(name, kv_split, q_split):
    """The dK/dV walk split by role (one wave S, P and dV, another dP, dS and dK per 32 keys, P passed
    through LDS in bf16; bwd_kv_walk = 2) gives the oracle's gradients, fully masked rows and dead key
    columns exactly zero; fp32 problems ignore the hint."""
    c = CASES[name]()
    t = upload(c)
    say(f"case {name}: role-split dK/dV walk, kv_split {kv_split} q_split {q_split}")
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal,
                         q_offset=c.q_offset)
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=t["mask"], scale=c.scale,
                             causal=c.causal, q_offset=c.q_offset, kv_split=kv_split, q_split=q_split, kv_walk=2)
    torch.cuda.synchronize()
    ref = oracle_full(c)
    compare_full(c, {"dQ": host64(dq), "dK": host64(dk), "dV": host64(dv)}, ref, names=("dQ", "dK", "dV"),
                 zero_ok=("dQ", "dK") if c.Sk == 1 else ())


def test_role_split_walk_chunked():
    """The role-split walk adding into the window accumulators over a 4-chunk walk equals the one-shot oracle."""
    W, C = 512, 128
    c = make_case("role_walk", B=1, Hq=4, Hkv=2, Sq=W, Sk=W, D=128, dtype="bf16", seed=71, causal=True)
    t = upload(c)
    dk_acc = torch.zeros((1, c.Hkv, W, c.D), dtype=torch.float32, device="cuda")
    dv_acc = torch.zeros_like(dk_acc)
    for p0, n, sk in configs.chunk_plan(W, C):
        q, do = t["q"][:, :, p0:p0 + n], t["do"][:, :, p0:p0 + n]
        kk, vv = t["k"][:, :, :sk], t["v"][:, :, :sk]
        o, lse = binding.fwd(q, kk, vv, scale=c.scale, causal=True, q_offset=p0)
        delta = binding.bwd_preprocess(o, do)
        binding.bwd_chunked(q, kk, vv, do, lse, delta, dk_acc, dv_acc, scale=c.scale, causal=True, q_offset=p0,
                            kv_walk=2)
    torch.cuda.synchronize()
    ref = oracle_full(c)
    compare_full(c, {"dK": dk_acc.cpu().numpy().astype(np.float64), "dV": dv_acc.cpu().numpy().astype(np.float64)},
                 ref, names=("dK", "dV"))


@pytest.mark.parametrize("q_split,q_split_tiles,dq_launch", [(2, 1, 1), (3, 2, 1), (4, 1, 2), (2, 99, 1), (2, 1, 3),
                                                             (3, 3, 3)])
@pytest.mark.parametrize("name", ["dit_sa_ragged", "lm_causal_gqa4", "random_bias_bcast", "d64_bf16"])
def test_backward_split_tail(name, q_split, q_split_tiles, dq_launch):
    """Only the first query tiles' dQ walks split (dispatched last), the others whole: the split tiles
    sum fp32 slices over their rows only, the whole ones store directly; the oracle's gradients either way."""
    c = CASES[name]()
    t = upload(c)
    say(f"case {name}: q_split {q_split} over the first {q_split_tiles} query tiles, dq_launch {dq_launch}")
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal,
                         q_offset=c.q_offset)
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=t["mask"], scale=c.scale,
                             causal=c.causal, q_offset=c.q_offset, kv_split=2, q_split=q_split,
                             q_split_tiles=q_split_tiles, dq_launch=dq_launch)
    torch.cuda.synchronize()
    compare_full(c, {"dQ": host64(dq), "dK": host64(dk), "dV": host64(dv)}, oracle_full(c), names=("dQ", "dK", "dV"))


@pytest.mark.parametrize("name", ["dit_sa_ragged", "lm_causal_gqa4"])
def test_dq_launch_is_bitwise_neutral(name):
    """The dQ walk in its own launch (two workgroups per compute unit) does the same arithmetic in the
    same order as in the shared launch: identical bits for a fixed split."""
    c = CASES[name]()
    t = upload(c)
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal,
                         q_offset=c.q_offset)
    delta = binding.bwd_preprocess(o, t["do"])
    out = [binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=t["mask"], scale=c.scale,
                       causal=c.causal, q_offset=c.q_offset, kv_split=2, q_split=1, dq_launch=m) for m in (1, 2)]
    torch.cuda.synchronize()
    for a, b in zip(*out):
        assert torch.equal(a, b)


def test_tuned_split_is_a_candidate_and_exact():
    """The split tuner returns one of its candidates, and the backward run with that split (and the mask
    tile map) gives the oracle's gradients."""
    c = CASES["dit_ca_ragged"]()
    t = upload(c)
    tiles = binding.mask_tile_map(t["mask"], t["q"], t["k"])
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal,
                         q_offset=c.q_offset, mask_tiles=tiles)
    delta = binding.bwd_preprocess(o, t["do"])
    kv, qs = binding.tune_bwd_splits(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=t["mask"], scale=c.scale,
                                     causal=c.causal, q_offset=c.q_offset, mask_tiles=tiles, reps=2)
    assert (kv, qs) in binding.BWD_SPLIT_CANDIDATES
    say(f"    tuned split kv {kv} q {qs}")
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=t["mask"], scale=c.scale,
                             causal=c.causal, q_offset=c.q_offset, kv_split=kv, q_split=qs, mask_tiles=tiles)
    torch.cuda.synchronize()
    compare_full(c, {"dQ": host64(dq), "dK": host64(dk), "dV": host64(dv)}, oracle_full(c), names=("dQ", "dK", "dV"))


@pytest.mark.parametrize("kv_split,q_split,dq_launch,q_split_tiles", [(1, 1, 0, 0), (2, 3, 0, 0), (2, 1, 2, 0),
                                                                      (2, 2, 0, 1)])
def test_chunked_decompositions(kv_split, q_split, dq_launch, q_split_tiles):
    """The chunked backward adds into the window accumulators the same way for any split."""
    W, C = 512, 128
    c = configs.make("long_window", W=W, Hq=4, Hkv=1)
    t = upload(c)
    dk_acc = torch.zeros((1, c.Hkv, W, c.D), dtype=torch.float32, device="cuda")
    dv_acc = torch.zeros_like(dk_acc)
    dQ = torch.empty_like(t["q"])
    for p0, n, sk in configs.chunk_plan(W, C):
        q, do = t["q"][:, :, p0:p0 + n], t["do"][:, :, p0:p0 + n]
        kk, vv = t["k"][:, :, :sk], t["v"][:, :, :sk]
        o, lse = binding.fwd(q, kk, vv, scale=c.scale, causal=True, q_offset=p0)
        delta = binding.bwd_preprocess(o, do)
        binding.bwd_chunked(q, kk, vv, do, lse, delta, dk_acc, dv_acc, scale=c.scale, causal=True, q_offset=p0,
                            dq=dQ[:, :, p0:p0 + n], kv_split=kv_split, q_split=q_split, dq_launch=dq_launch,
                            q_split_tiles=q_split_tiles)
    torch.cuda.synchronize()
    ref = oracle_full(c)
    got = {"dQ": host64(dQ), "dK": dk_acc.cpu().numpy().astype(np.float64),
           "dV": dv_acc.cpu().numpy().astype(np.float64)}
    compare_full(c, got, ref, names=("dQ", "dK", "dV"))


def numpy_tile_map(mask: np.ndarray) -> np.ndarray:
    Bm, Sq, Sk = mask.shape
    nr, nc = (Sq + 63) // 64, (Sk + 63) // 64
    out = np.zeros((Bm, nr, nc), np.uint8)
    for b in range(Bm):
        for r in range(nr):
            for c in range(nc):
                blk = mask[b, 64 * r:64 * r + 64, 64 * c:64 * c + 64]
                fin = np.isfinite(blk)
                if not fin.any():
                    out[b, r, c] = 0
                elif np.any(blk[fin] != 0):
                    out[b, r, c] = 3
                else:
                    out[b, r, c] = 1 if fin.all() else 2
    return out.reshape(-1)


TILE_CASES = {
    "dit_sa_ragged": lambda: configs.make("dit_sa", Hq=4, Hkv=2, Sq=300, Sk=300),
    "dit_ca_ragged": lambda: configs.make("dit_ca", B=2, Hq=2, Hkv=2, Sq=300, Sk=400),
    "random_blocks": lambda: _block_mask_case(),
    "causal_plus_pad": lambda: make_case("causal_pad", B=1, Hq=4, Hkv=1, Sq=260, Sk=260, D=128, dtype="bf16",
                                         seed=71, causal=True, mask="sa_pad", mask_args={"pad_frac": 0.2}),
}


def _block_mask_case():
    """Mask with whole dead blocks, whole open blocks, bias blocks and ragged edges."""
    c = make_case("random_blocks", B=2, Hq=2, Hkv=1, Sq=200, Sk=330, D=128, dtype="bf16", seed=72)
    rng = np.random.default_rng(73)
    m = np.zeros((2, 200, 330), np.float32)
    for b in range(2):
        for r in range(0, 200, 64):
            for cc in range(0, 330, 64):
                kind = rng.integers(0, 3)
                if kind == 0:
                    m[b, r:r + 64, cc:cc + 64] = -np.inf
                elif kind == 2:
                    m[b, r:r + 64, cc:cc + 64] = rng.standard_normal(m[b, r:r + 64, cc:cc + 64].shape)
    m[0, 5, :] = -np.inf  # a fully masked row
    c.mask = m
    c.meta["mask_kind"] = "blocks"
    return c


@pytest.mark.parametrize("name", list(TILE_CASES))
def test_mask_tile_map_and_skipping(name):
    """The mask block classification matches numpy, and fwd + bwd that use it (skipping
    dead blocks, not reading open ones) still match the oracle."""
    c = TILE_CASES[name]()
    t = upload(c)
    tiles = binding.mask_tile_map(t["mask"], t["q"], t["k"])
    torch.cuda.synchronize()
    nblk = binding.mask_tile_count(t["mask"])
    assert np.array_equal(tiles[:nblk].cpu().numpy(), numpy_tile_map(c.mask))
    # the visibility words: bit j of row word i / bit i of column word j = entry (i, j) finite
    Bm, Sq, Sk = c.mask.shape
    nr, nc = (Sq + 63) // 64, (Sk + 63) // 64
    off = (nblk + 255) // 256 * 256
    words = tiles[off:off + 2 * nblk * 64 * 8].cpu().numpy().view(np.uint64).reshape(2, Bm, nr, nc, 64)
    vis = np.zeros((Bm, nr * 64, nc * 64), bool)
    vis[:, :Sq, :Sk] = np.isfinite(c.mask)
    blocks = vis.reshape(Bm, nr, 64, nc, 64).transpose(0, 1, 3, 2, 4)  # [Bm, nr, nc, row, col]
    weights = (np.uint64(1) << np.arange(64, dtype=np.uint64))
    rows = (blocks.astype(np.uint64) * weights[None, None, None, None, :]).sum(axis=4, dtype=np.uint64)
    cols = (blocks.astype(np.uint64) * weights[None, None, None, :, None]).sum(axis=3, dtype=np.uint64)
    assert np.array_equal(words[0], rows) and np.array_equal(words[1], cols)
    # the key-split forward walks the live tiles in pairs; the split forward a share of them
    for variant, split in ((1, 1), (3, 1), (1, 3)):
        o3, lse3 = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal,
                               q_offset=c.q_offset, mask_tiles=tiles, variant=variant, split=split)
        torch.cuda.synchronize()
        ref = oracle_full(c)
        compare_full(c, {"O": host64(o3), "LSE": host64(lse3)}, ref, names=("O", "LSE"))
    o, lse = binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal,
                         q_offset=c.q_offset, mask_tiles=tiles)
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, mask=t["mask"], scale=c.scale,
                             causal=c.causal, q_offset=c.q_offset, mask_tiles=tiles)
    torch.cuda.synchronize()
    got = {"O": host64(o), "LSE": host64(lse), "Delta": host64(delta), "dQ": host64(dq), "dK": host64(dk),
           "dV": host64(dv)}
    compare_full(c, got, oracle_full(c))
