"""Dense masks over walks longer than 64 mask blocks, on the GPU against the oracle. Each
forward wave takes its blocks' classes along the keys 64 at a time, and each dK/dV wave
along the rows 64 at a time; a walk past 64 blocks loads the next run. The mask is drawn
block by block (hidden, open, 0 / -inf, finite biases), so every class appears along the
long axis, and the tile map lets the kernels skip, open or mask each block. Long key axis
(forward runs, split forward shares, dQ walks) and long query axis (dK/dV runs, the dQ
pass over stored dS), element by element."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from flash_attention_train_amd import binding
from flash_attention_train_amd.inputs import make_case
from parity_util import compare_full, host64, say, upload

pytestmark = pytest.mark.gpu

CASES = {
    # 71 key blocks: forward and dQ walks cross the 64-block run boundary
    "long_keys": dict(B=1, Hq=2, Hkv=1, Sq=200, Sk=4500, D=64, seed=611),
    # 71 row blocks: dK/dV walks cross it
    "long_rows": dict(B=1, Hq=2, Hkv=1, Sq=4500, Sk=200, D=64, seed=612),
}


@pytest.mark.parametrize("name,dq_launch", [("long_keys", 0), ("long_keys", 1), ("long_rows", 0), ("long_rows", 3)])
def test_long_mask_walks(name, dq_launch):
    c = make_case(f"long_mask_{name}", dtype="bf16", mask="blocks", **CASES[name])
    say(f"case {name}: B={c.B} Hq={c.Hq} Sq={c.Sq} Sk={c.Sk} D={c.D}, block mask, dq_launch={dq_launch}")
    t = upload(c)
    tiles = binding.mask_tile_map(t["mask"], t["q"], t["k"])
    kw = dict(mask=t["mask"], scale=c.scale, causal=c.causal, q_offset=c.q_offset, mask_tiles=tiles)
    o, lse = binding.fwd(t["q"], t["k"], t["v"], **kw)
    delta = binding.bwd_preprocess(o, t["do"])
    dq, dk, dv = binding.bwd(t["q"], t["k"], t["v"], t["do"], lse, delta, dq_launch=dq_launch, **kw)
    got = dict(zip(("O", "LSE", "Delta", "dQ", "dK", "dV"), (host64(x) for x in (o, lse, delta, dq, dk, dv))))
    ref = oracle.backward(c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), c.mask.astype(np.float64),
                          scale=c.scale, causal=c.causal, q_offset=c.q_offset)
    errs = compare_full(c, got, ref)
    say("  errors: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
