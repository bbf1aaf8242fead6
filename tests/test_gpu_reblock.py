"""Blocking reconciliation inside jagg_einsum, through the C ABI, against the
oracle.

"Every Kernel Is a Join" (Ding et al.), Sec. 4.3: executing a join-agg spec
includes repartitioning each input to the spec's own tiling, and Def. 3.7
joins tuples on equal intervals only.  So an input uploaded under a blocking
other than the call's `blockings` is re-blocked into the workspace before
the join.  Every case here uploads at least one input blocked differently,
fills the workspace with a non-zero byte and the output with a sentinel
first, and checks the whole output relation (padding +0 included) against
the oracle's dense evaluation on the original values: bit-exact for MAX,
the fp32 / bf16 normwise tolerances otherwise.
"""
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O
from tensor_relational_einsum_amd import inputs as I
from tensor_relational_einsum_amd import jagg
from parity_util import normwise_err, padding_mask, to_np

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5
BF16_OUT_TOL = 8e-3


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    old = os.environ.get("JAGG_TRACE")
    os.environ["JAGG_TRACE"] = "1"
    try:
        c = jagg.Context(0)
    finally:
        if old is None:
            del os.environ["JAGG_TRACE"]
        else:
            os.environ["JAGG_TRACE"] = old
    yield c
    torch.cuda.synchronize()
    c.close()


def run_reblock(ctx, capfd, spec, ext, call_blk, in_blks, g="mul", agg="sum", in_dtypes=None, out_dtype="f32",
                positive=(), seed=31, **kw):
    """Uploads input j under in_blks[j], runs the spec under call_blk; returns
    (gpu dense, oracle dense rounded, output relation values, padding mask)."""
    ins, out = spec.split("->")
    ins = ins.split(",")
    in_dtypes = in_dtypes or ["f32"] * len(ins)
    xs = []
    for j, (lt, gen, dt) in enumerate(zip(ins, I.streams(seed, len(ins)), in_dtypes)):
        x = I.draw(gen, [ext[c] for c in lt], "normal", dt)
        if j in positive:
            x = (x.float().abs() + 0.5).to(x.dtype)
        xs.append(x)
    rels = [jagg.from_dense(ctx, x.to("cuda"), lt, b) for x, lt, b in zip(xs, ins, in_blks)]
    call = jagg.EinsumCall(ctx, spec, rels, call_blk, g=g, agg=agg, out_dtype=out_dtype, **kw)
    call.workspace.fill_(0xAB)  # the re-blocked copies must overwrite every byte they use
    call.out.data.fill_(float("nan"))
    capfd.readouterr()
    call.run()
    torch.cuda.synchronize()
    trace = capfd.readouterr().err
    for j, b in enumerate(in_blks):
        differs = any(jagg.block_count(b.get(c, 1)) != jagg.block_count(call_blk.get(c, 1)) for c in ins[j])
        assert (f"{spec}: reblock input {j} into" in trace) == differs, trace
    got_rel = to_np(call.out.data)
    want = O.round_to(O.dense(spec, [to_np(x) for x in xs], ext, g=g, agg=agg, **kw), out_dtype)
    got = O.from_relation(got_rel, out, ext, call_blk)
    pad = padding_mask(out, ext, call_blk)
    return got, want, got_rel, pad


@pytest.mark.parametrize("idt,odt", [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16")])
def test_reblock_matmul_both_inputs(ctx, capfd, idt, odt):
    """'ij,jk->ik': A uploaded {i2, j3}, B {j5, k1}, the call asks {i4, j4, k2};
    ragged tails on every letter (j = 130 in 3, 4 and 5 blocks)."""
    ext = dict(i=200, j=130, k=70)
    got, want, got_rel, pad = run_reblock(ctx, capfd, "ij,jk->ik", ext, dict(i=4, j=4, k=2),
                                          [dict(i=2, j=3), dict(j=5, k=1)], in_dtypes=[idt, idt], out_dtype=odt)
    err = normwise_err(got, want)
    assert err < (F32_TOL if odt == "f32" else BF16_OUT_TOL), f"normwise error {err:.3e}"
    assert np.all(got_rel[pad] == 0.0), "output padding must be +0"


def test_reblock_one_input_batched_bf16(ctx, capfd):
    """A projection-shaped contraction where only the weight is blocked
    differently (h in 3 blocks against the call's 4, q in 1 against 2)."""
    ext = dict(b=2, s=96, h=384, q=4, d=64)
    blk = dict(b=1, s=2, h=4, q=2, d=1)
    got, want, got_rel, pad = run_reblock(ctx, capfd, "bsh,hqd->bsqd", ext, blk, [blk, dict(h=3, q=1, d=1)],
                                          in_dtypes=["bf16", "bf16"], out_dtype="bf16")
    assert normwise_err(got, want) < BF16_OUT_TOL
    assert np.all(got_rel[pad] == 0.0)


def test_reblock_rms_scale_map(ctx, capfd):
    """A three-input map: x {s5, h3} and the broadcast gamma {h2}, call
    {s3, h4}; the per-row sum of squares is already blocked as asked."""
    ext = dict(b=2, s=50, h=1000)
    blk = dict(b=1, s=3, h=4)
    got, want, got_rel, pad = run_reblock(ctx, capfd, "bsh,bs,h->bsh", ext, blk,
                                          [dict(b=1, s=5, h=3), dict(b=1, s=3), dict(h=2)], g="rms_scale",
                                          agg="none", in_dtypes=["f32", "f32", "bf16"], out_dtype="bf16",
                                          positive=(1,), beta=1.0 / 1000, eps=1e-6)
    assert normwise_err(got, want) < BF16_OUT_TOL
    assert np.all(got_rel[pad] == 0.0)


def test_reblock_max_reduce_bit_exact(ctx, capfd):
    """A row MAX whose input is uploaded {s2, t3} and reduced under {s3, t4}:
    bit-exact, since MAX is unique."""
    ext = dict(b=2, h=3, s=40, t=300)
    blk = dict(b=1, h=1, s=3, t=4)
    got, want, got_rel, pad = run_reblock(ctx, capfd, "bhst->bhs", ext, blk, [dict(b=1, h=1, s=2, t=3)],
                                          g="ident", agg="max")
    assert np.array_equal(got, want), "MAX must be bit-exact"
    assert np.all(got_rel[pad] == 0.0)


def test_reblock_sum_reduce_with_broadcast(ctx, capfd):
    """'bhst,bhs->bhs' (SUM of exp(S - m)) with S blocked {s4, t2} and m
    {s1} against the call's {s3, t4}: both inputs are re-blocked."""
    ext = dict(b=2, h=3, s=40, t=300)
    blk = dict(b=1, h=1, s=3, t=4)
    got, want, got_rel, pad = run_reblock(ctx, capfd, "bhst,bhs->bhs", ext, blk,
                                          [dict(b=1, h=1, s=4, t=2), dict(b=1, h=1, s=1)], g="exp_sub")
    assert normwise_err(got, want) < F32_TOL
    assert np.all(got_rel[pad] == 0.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_reblock_input_with_an_interval_letter(ctx, capfd, dtype):
    """A packed-sequence letter s (bounds 0, 100, 356, 512) in A and in the
    output, matching the call, while A's h is blocked 3 against the call's 4:
    the re-blocking copies the interval letter's padded blocks unchanged and
    re-tiles h."""
    S = [0, 100, 356, 512]
    ext = dict(s=512, h=130, f=96)
    blk = dict(s=S, h=4, f=2)
    got, want, got_rel, pad = run_reblock(ctx, capfd, "sh,hf->sf", ext, blk, [dict(s=S, h=3), dict(h=4, f=2)],
                                          in_dtypes=[dtype, dtype])
    assert normwise_err(got, want) < F32_TOL
    assert np.all(got_rel[pad] == 0.0), "output padding must be +0"
