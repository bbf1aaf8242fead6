"""Parity of the fused attention join-agg (g = attention, aggregation = the
online-softmax triple) with the oracle's attention, through the C ABI.

Tolerance: Q, K, V are exact bf16 values and scores accumulate in fp32; the
probabilities enter the P V product rounded to bf16 (relative 2^-9 each),
and a bf16 output adds one more rounding, so the normwise error (max abs
difference over max abs value) stays under 8e-3.
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as O
from tensor_relational_einsum_amd import inputs as I
from tensor_relational_einsum_amd import jagg
from parity_util import normwise_err, padding_mask, to_np

pytestmark = pytest.mark.gpu

ATT_TOL = 8e-3


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    c = jagg.Context(0)
    yield c
    torch.cuda.synchronize()
    c.close()


def run_attention(ctx, spec, ext, blk, alpha, causal, out_dtype, seed=3):
    ins, out = spec.split("->")
    ins = ins.split(",")
    gens = I.streams(seed, 3)
    xs = [I.draw(g, [ext[c] for c in lt], "normal", "bf16") for g, lt in zip(gens, ins)]
    rels = [jagg.from_dense(ctx, x.to("cuda"), lt, blk) for x, lt in zip(xs, ins)]
    call = jagg.EinsumCall(ctx, spec, rels, blk, g="attention", agg="softmax", out_dtype=out_dtype, alpha=alpha,
                           causal=causal)
    call.out.data.fill_(5)
    call.run()
    torch.cuda.synchronize()
    got_rel = to_np(call.out.data)
    got = O.from_relation(got_rel, out, ext, blk)
    return xs, got, got_rel, out


CASES = [
    # spec, extents, blockings, causal, out dtype
    ("bhsd,bhtd,bhte->bhse", dict(b=2, h=3, s=256, t=256, d=128, e=128), dict(b=1, h=1, s=2, t=2, d=1, e=1), None,
     "f32"),
    ("bhsd,bhtd,bhte->bhse", dict(b=2, h=3, s=256, t=256, d=128, e=128), dict(b=1, h=1, s=2, t=2, d=1, e=1),
     ("s", "t"), "bf16"),
    ("bhsd,bhtd,bhte->bhse", dict(b=1, h=2, s=256, t=256, d=64, e=64), dict(b=1, h=2, s=2, t=4, d=1, e=1),
     None, "bf16"),
    # ragged: s = t = 200 in 2 blocks of 100 (partial tiles, padding rows)
    ("bhsd,bhtd,bhte->bhse", dict(b=1, h=3, s=200, t=200, d=128, e=128), dict(b=1, h=1, s=2, t=2, d=1, e=1),
     ("s", "t"), "f32"),
    ("bhsd,bhtd,bhte->bhse", dict(b=1, h=3, s=200, t=200, d=64, e=64), dict(b=1, h=1, s=2, t=2, d=1, e=1),
     None, "f32"),
    # several 128-row tiles per s block, causal
    ("hsd,htd,hte->hse", dict(h=2, s=512, t=512, d=128, e=128), dict(h=1, s=1, t=1, d=1, e=1), ("s", "t"), "f32"),
    # batch letters on both sides of s (the projection layout), q blocked
    ("bsqd,btqd,btqe->bsqe", dict(b=2, s=256, t=256, q=4, d=128, e=128), dict(b=1, s=2, t=2, q=2, d=1, e=1),
     ("s", "t"), "bf16"),
    # more keys than queries
    ("hsd,htd,hte->hse", dict(h=2, s=128, t=384, d=64, e=64), dict(h=1, s=1, t=3, d=1, e=1), None, "f32"),
    # grouped-query attention ("Every Kernel Is a Join", Example 3.10): 32 query
    # heads over 8 key-value heads, the kv heads in unit intervals; the query
    # group letter r appears in Q and the output only
    ("grsd,gtd,gte->grse", dict(g=8, r=4, s=512, t=512, d=128, e=128), dict(g=8, r=1, s=2, t=2, d=1, e=1),
     ("s", "t"), "bf16"),
    ("grsd,gtd,gte->grse", dict(g=2, r=3, s=200, t=200, d=64, e=64), dict(g=2, r=3, s=2, t=2, d=1, e=1), None,
     "f32"),
    # the projection layout with the group inside: s is the row letter, r a batch letter
    ("bsgrd,btgd,btge->bsgre", dict(b=2, s=256, t=256, g=2, r=4, d=128, e=128),
     dict(b=1, s=2, t=2, g=2, r=2, d=1, e=1), ("s", "t"), "bf16"),
]


@pytest.mark.parametrize("spec,ext,blk,causal,odt", CASES)
def test_attention_parity(ctx, spec, ext, blk, causal, odt):
    alpha = 1.0 / math.sqrt(ext["d"])
    xs, got, got_rel, out = run_attention(ctx, spec, ext, blk, alpha, causal, odt)
    want = O.round_to(O.attention_dense(spec, [to_np(x) for x in xs], ext, alpha=alpha, causal=causal), odt)
    err = normwise_err(got, want)
    print(f"normwise error {err:.3e}")
    assert err < ATT_TOL, f"normwise error {err:.3e}"
    pad = padding_mask(out, ext, blk)
    assert np.all(got_rel[pad] == 0.0), "output padding must be +0"


def test_attention_matches_relational_oracle(ctx):
    """The GPU walk and the oracle's join / triple-merge / recompose agree."""
    spec = "hsd,htd,hte->hse"
    ext = dict(h=2, s=192, t=192, d=64, e=64)
    blk = dict(h=1, s=3, t=3, d=1, e=1)
    xs, got, got_rel, out = run_attention(ctx, spec, ext, blk, 0.125, ("s", "t"), "f32", seed=9)
    rels = [O.to_relation(to_np(x), lt, ext, blk) for x, lt in zip(xs, ("hsd", "htd", "hte"))]
    want_rel, present = O.attention_relational(spec, rels, ext, blk, alpha=0.125, causal=("s", "t"))
    assert present.all()
    err = normwise_err(got_rel, O.round_to(want_rel, "f32"))
    assert err < ATT_TOL, f"normwise error {err:.3e}"


def test_attention_rejects_unsupported(ctx):
    ext = dict(h=2, s=64, t=64, d=96, e=96)
    blk = dict(h=1, s=1, t=1, d=1, e=1)
    gens = I.streams(1, 3)
    xs = [I.draw(g, [2, 64, 96], "normal", "bf16") for g in gens]
    rels = [jagg.from_dense(ctx, x.to("cuda"), lt, blk) for x, lt in zip(xs, ("hsd", "htd", "hte"))]
    with pytest.raises(jagg.JaggError):  # D = 96 is not a supported head size
        jagg.EinsumCall(ctx, "hsd,htd,hte->hse", rels, blk, g="attention", agg="softmax").run()
    with pytest.raises(jagg.JaggError):  # the triple aggregation pairs only with g = attention
        jagg.EinsumCall(ctx, "hsd,htd,hte->hse", rels, blk, g="mul", agg="softmax").run()
    ext = dict(g=2, r=2, s=64, t=64, d=64, e=64)
    blk = dict(g=1, r=1, s=1, t=1, d=1, e=1)
    xs = [I.draw(g, [ext[c] for c in lt], "normal", "bf16") for g, lt in zip(gens, ("grsd", "gtd", "gte"))]
    rels = [jagg.from_dense(ctx, x.to("cuda"), lt, blk) for x, lt in zip(xs, ("grsd", "gtd", "gte"))]
    with pytest.raises(jagg.JaggError):  # a causal pair whose first letter is a kv letter
        jagg.EinsumCall(ctx, "grsd,gtd,gte->grse", rels, blk, g="attention", agg="softmax", causal=("g", "t")).run()
