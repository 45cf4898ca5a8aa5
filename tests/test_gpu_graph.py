"""The whole step (mask tile map, forward, preprocess, backward) captured in a HIP graph
and replayed: every replay, with eager work and synchronizations between replays, must
reproduce the eager step's outputs bit for bit (split walks sum fixed fp32 slices in a
fixed order, so a fixed decomposition is reproducible), and the eager step itself matches
the oracle. This is the launch sequence the benchmark times, including a split tail of
dQ walks with its two reduce passes, dQ from stored dS, and the dQ kernel on the library's second
stream (forked from and joined back to the captured stream)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from flash_attention_train_amd import binding, configs
from flash_attention_train_amd.inputs import make_case
from parity_util import compare_full, host64, say, upload

pytestmark = pytest.mark.gpu


class Step:
    def __init__(self, c, t, fwd_split=0, bwd_splits=(1, 1, 0), dq_launch=0):
        self.c, self.t = c, t
        self.bwd_splits = bwd_splits
        self.dq_launch = dq_launch
        q = t["q"]
        self.fwd_split = fwd_split
        self.fws = torch.empty(max(256, binding.fwd_workspace_bytes(q, t["k"], scale=c.scale, causal=c.causal,
                                                                    q_offset=c.q_offset, mask=t["mask"],
                                                                    split=fwd_split)),
                               dtype=torch.uint8, device="cuda")
        self.o = torch.empty_like(q)
        self.lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        self.delta = torch.empty_like(self.lse)
        self.dq, self.dk, self.dv = torch.empty_like(q), torch.empty_like(t["k"]), torch.empty_like(t["v"])
        kv, qs, qt = bwd_splits
        self.ws = torch.empty(max(1 << 20, binding.bwd_workspace_bytes(q, t["k"], scale=c.scale, causal=c.causal,
                                                                       q_offset=c.q_offset, mask=t["mask"],
                                                                       kv_split=kv, q_split=qs, q_split_tiles=qt,
                                                                       dq_launch=dq_launch)),
                              dtype=torch.uint8, device="cuda")
        self.tiles = None if t["mask"] is None else binding.mask_tile_map(t["mask"], q, t["k"])

    def __call__(self):
        c, t = self.c, self.t
        if self.tiles is not None:
            binding.mask_tile_map(t["mask"], t["q"], t["k"], out=self.tiles)
        binding.fwd(t["q"], t["k"], t["v"], mask=t["mask"], scale=c.scale, causal=c.causal, q_offset=c.q_offset,
                    out=self.o, lse=self.lse, mask_tiles=self.tiles, workspace=self.fws, split=self.fwd_split)
        binding.bwd_preprocess(self.o, t["do"], delta=self.delta)
        binding.bwd(t["q"], t["k"], t["v"], t["do"], self.lse, self.delta, mask=t["mask"], scale=c.scale,
                    causal=c.causal, q_offset=c.q_offset, dq=self.dq, dk=self.dk, dv=self.dv, workspace=self.ws,
                    kv_split=self.bwd_splits[0], q_split=self.bwd_splits[1], q_split_tiles=self.bwd_splits[2],
                    mask_tiles=self.tiles, dq_launch=self.dq_launch)

    def outputs(self):
        return [x.clone() for x in (self.o, self.lse, self.delta, self.dq, self.dk, self.dv)]


@pytest.mark.parametrize("key,shrink,fwd_split,bwd_splits,dq_launch", [
    ("dit_sa", dict(Hq=4, Hkv=2, Sq=300, Sk=300), 0, (1, 1, 0), 0),
    ("dit_sa", dict(Hq=4, Hkv=2, Sq=300, Sk=300), 0, (2, 2, 1), 0),  # the split tail the bench runs
    ("dit_ca", dict(B=2, Hq=2, Hkv=2, Sq=300, Sk=160), 0, (1, 1, 0), 0),
    ("lm_causal", dict(Hq=4, Hkv=1, Sq=333, Sk=333), 0, (1, 1, 0), 0),
    ("chunk", None, 4, (1, 1, 0), 0),
    ("lm_causal", dict(Hq=4, Hkv=1, Sq=333, Sk=333), 0, (2, 1, 0), 3),  # dQ from stored dS
    ("dit_ca", dict(B=2, Hq=2, Hkv=2, Sq=300, Sk=160), 0, (2, 1, 0), 4),  # dQ kernel on the second stream
    ("dit_sa", dict(Hq=4, Hkv=2, Sq=300, Sk=300), 0, (2, 2, 1), 4)])
def test_graph_replays_match_eager(key, shrink, fwd_split, bwd_splits, dq_launch):
    if key == "chunk":  # a query chunk late in a causal window: the split-key forward and its merge
        c = make_case("graph_chunk", B=1, Hq=4, Hkv=2, Sq=200, Sk=1800, D=128, dtype="bf16", seed=71, causal=True,
                      q_offset=1600)
    else:
        c = configs.make(key, **shrink)
    say(f"{key}: graph capture of the whole step, B={c.B} Hq={c.Hq} Sq={c.Sq} Sk={c.Sk} fwd_split={fwd_split} "
        f"bwd_splits={bwd_splits} dq_launch={dq_launch}")
    step = Step(c, upload(c), fwd_split, bwd_splits, dq_launch)
    step()
    torch.cuda.synchronize()
    eager = step.outputs()
    got = dict(zip(("O", "LSE", "Delta", "dQ", "dK", "dV"), (host64(x) for x in eager)))
    m = None if c.mask is None else c.mask.astype(np.float64)
    ref = oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), m, scale=c.scale, causal=c.causal,
                          q_offset=c.q_offset)
    compare_full(c, got, ref)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    scratch = torch.zeros(1 << 16, device="cuda")
    for rep in range(4):
        for x in (step.o, step.lse, step.delta, step.dq, step.dk, step.dv):
            x.fill_(float("nan"))  # eager work between replays; every output must be rewritten
        scratch.add_(1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("O", "LSE", "Delta", "dQ", "dK", "dV"), eager, step.outputs()):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager step"
    say(f"    4 replays equal to the eager step")
