"""The fused RMS-norm pair (jagg_plan_fuse): a sum-of-squares reduce over the
innermost letter and the RMS-scale map that reads it, run as one pass,
through the C ABI.

Against the oracle: ss = alpha_r * sum_r x^2 (oracle.dense of the reduce
spec on the original input, rounded to f32) and y = alpha_m * x *
rsqrt(ss * beta + eps) * gamma (oracle.dense of the map spec on the original
input, the oracle's own f32 ss and gamma, rounded to the output dtype);
bars 1e-5 normwise for f32, 8e-3 for one bf16 rounding; padding +0 in both
outputs.  Against the two plans run apart on the same buffers: the same
bars (only the order of the row sums differs).  Cases cover ragged rows, a
ragged last r-block, bf16 and f32 inputs and outputs, the longest row the
kernel holds (16 r-blocks of 256) and a single r-block; pairs of another
form are refused as unsupported.
"""
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O
from parity_util import normwise_err, padding_mask, to_np
from tensor_relational_einsum_amd import inputs as I
from tensor_relational_einsum_amd import jagg
from tensor_relational_einsum_amd.runner import ChainRunner

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


def make_pair(ctx, letters, ext, blk, xdt, gdt, odt, alpha_r=1.0, alpha_m=1.0, seed=91, red_agg="sum"):
    r, rows = letters[-1], letters[:-1]
    gens = I.streams(seed, 2)
    x = I.draw(gens[0], [ext[c] for c in letters], "normal", xdt)
    gam = I.draw(gens[1], [ext[r]], "normal", gdt, 0.02, 1.0)
    X = jagg.from_dense(ctx, x.to("cuda"), letters, blk)
    G = jagg.from_dense(ctx, gam.to("cuda"), r, blk)
    red = jagg.EinsumCall(ctx, f"{letters}->{rows}", [X], blk, g="square", agg=red_agg, out_dtype="f32",
                          alpha=alpha_r)
    mp = jagg.EinsumCall(ctx, f"{letters},{rows},{r}->{letters}", [X, red.out, G], blk, g="rms_scale", agg="none",
                         out_dtype=odt, alpha=alpha_m, beta=1.0 / ext[r], eps=1e-6)
    return x, gam, red, mp


CASES = [
    # letters, extents, blockings, x dtype, gamma dtype, out dtype, alpha_r, alpha_m
    # the block's form (4 r-blocks of 256), ragged rows (s: 34-row blocks, 100 valid)
    ("bsh", dict(b=2, s=100, h=1024), dict(b=1, s=3, h=4), "f32", "bf16", "bf16", 1.0, 1.0),
    # ragged r: 2045 = 3 x 512 + 509
    ("bsh", dict(b=1, s=64, h=2045), dict(b=1, s=2, h=4), "f32", "f32", "f32", 0.5, 1.5),
    # bf16 input, ragged r: 766 = 2 x 256 + 254
    ("sh", dict(s=130, h=766), dict(s=2, h=3), "bf16", "bf16", "f32", 1.0, 1.0),
    # the longest row the kernel holds: 16 r-blocks of 256
    ("bsh", dict(b=2, s=40, h=4096), dict(b=2, s=1, h=16), "f32", "bf16", "bf16", 1.0, 1.0),
    # a single r-block
    ("sh", dict(s=50, h=512), dict(s=1, h=1), "f32", "bf16", "bf16", 1.0, 1.0),
]


@pytest.mark.parametrize("letters,ext,blk,xdt,gdt,odt,ar,am", CASES)
def test_fused_norm_pair_parity(ctx, capfd, letters, ext, blk, xdt, gdt, odt, ar, am):
    r, rows = letters[-1], letters[:-1]
    x, gam, red, mp = make_pair(ctx, letters, ext, blk, xdt, gdt, odt, ar, am)
    print(f"[test] fused norm pair {letters} {ext} {blk} {xdt}->{odt}", flush=True)
    # the two plans apart, for the comparison below
    red.prepare()
    mp.prepare()
    red.out.data.fill_(3)
    mp.out.data.fill_(3)
    red.run_plan()
    mp.run_plan()
    torch.cuda.synchronize()
    ss_apart, y_apart = to_np(red.out.data), to_np(mp.out.data)
    fused = jagg.PlanFused(ctx, red, mp)
    red.out.data.fill_(3)
    mp.out.data.fill_(3)
    capfd.readouterr()
    fused.run()
    torch.cuda.synchronize()
    assert "rms norm pair in one pass" in capfd.readouterr().err
    ss_rel, y_rel = to_np(red.out.data), to_np(mp.out.data)
    assert np.all(ss_rel[padding_mask(rows, ext, blk)] == 0.0), "row-statistic padding must be +0"
    assert np.all(y_rel[padding_mask(letters, ext, blk)] == 0.0), "output padding must be +0"
    # oracle: each spec on the original inputs, ss rounded to f32 where stored
    xd, gd = to_np(x), to_np(gam)
    ss_want = O.round_to(O.dense(f"{letters}->{rows}", [xd], ext, g="square", agg="sum", alpha=ar), "f32")
    y_want = O.round_to(O.dense(f"{letters},{rows},{r}->{letters}", [xd, ss_want, gd], ext, g="rms_scale",
                                agg="none", alpha=am, beta=1.0 / ext[r], eps=1e-6), odt)
    ss_got = O.from_relation(ss_rel, rows, ext, blk)
    y_got = O.from_relation(y_rel, letters, ext, blk)
    tol = F32_TOL if odt == "f32" else BF16_OUT_TOL
    assert normwise_err(ss_got, ss_want) < F32_TOL
    assert normwise_err(y_got, y_want) < tol
    # the two plans run apart: the same values up to the order of the row sums
    assert normwise_err(ss_rel, ss_apart) < F32_TOL
    assert normwise_err(y_rel, y_apart) < tol


def test_fused_norm_pair_rejects_other_forms(ctx):
    blk = dict(b=1, s=2, h=4)
    # block extent of r not a multiple of 256 (1000 / 4 = 250)
    _, _, red, mp = make_pair(ctx, "bsh", dict(b=1, s=16, h=1000), blk, "f32", "bf16", "bf16")
    with pytest.raises(jagg.JaggError) as e:
        jagg.PlanFused(ctx, red, mp)
    assert e.value.status == -4
    # rows longer than 4096 elements (2 r-blocks of 4096)
    _, _, red, mp = make_pair(ctx, "bsh", dict(b=1, s=8, h=8192), dict(b=1, s=1, h=2), "f32", "bf16", "bf16")
    with pytest.raises(jagg.JaggError) as e:
        jagg.PlanFused(ctx, red, mp)
    assert e.value.status == -4
    # a MAX reduce is not a sum of squares
    _, _, red, mp = make_pair(ctx, "bsh", dict(b=1, s=16, h=1024), blk, "f32", "bf16", "bf16", red_agg="max")
    with pytest.raises(jagg.JaggError) as e:
        jagg.PlanFused(ctx, red, mp)
    assert e.value.status == -4
    # the pair in the wrong order
    _, _, red, mp = make_pair(ctx, "bsh", dict(b=1, s=16, h=1024), blk, "f32", "bf16", "bf16")
    with pytest.raises(jagg.JaggError) as e:
        jagg.PlanFused(ctx, mp, red)
    assert e.value.status == -4
    # a map over another relation than the one reduced
    x2, _, red2, _ = make_pair(ctx, "bsh", dict(b=1, s=16, h=1024), blk, "f32", "bf16", "bf16", seed=5)
    with pytest.raises(jagg.JaggError) as e:
        jagg.PlanFused(ctx, red2, mp)
    assert e.value.status == -4


def test_block_runs_both_norms_fused(ctx):
    w = I.llama_block(b=1, s=256, hid=512, heads=4, d=128, ffn=1376, s_blk=2, h_blk=2, q_blk=2, f_blk=4,
                      fused_attention=True, fused_epilogues=True)
    dense = I.generate(w)
    fused = ChainRunner(ctx, w, dense)
    apart = ChainRunner(ctx, w, dense, fuse_norms=False)
    assert [u[2] for u in fused.units if u[0] == "fused"] == [[0, 1], [7, 8]]
    assert not any(u[0] == "fused" for u in apart.units)
    for run in (fused, apart):
        run.run()
    torch.cuda.synchronize()
    # every relation of the block, at the block's end-to-end bar (the row sums'
    # last bits reach later relations through their bf16 roundings)
    for st in w.chain:
        a, b = to_np(fused.rel[st.out].data), to_np(apart.rel[st.out].data)
        assert normwise_err(a, b) < 2e-2, st.out


def test_fused_pair_in_a_group_and_refusal_of_a_reblocked_input(ctx):
    # a fused pair may be a member of a plan group beside an independent plan
    ext, blk = dict(b=1, s=64, h=1024), dict(b=1, s=2, h=4)
    x, gam, red, mp = make_pair(ctx, "bsh", ext, blk, "f32", "bf16", "bf16", seed=23)
    fused = jagg.PlanFused(ctx, red, mp)
    gens = I.streams(29, 2)
    a = I.draw(gens[0], [256, 512], "normal", "f32")
    b = I.draw(gens[1], [512, 192], "normal", "f32")
    cblk = dict(i=2, j=2, k=2)
    A = jagg.from_dense(ctx, a.to("cuda"), "ij", cblk)
    B = jagg.from_dense(ctx, b.to("cuda"), "jk", cblk)
    mm = jagg.EinsumCall(ctx, "ij,jk->ik", [A, B], cblk)
    group = jagg.PlanGroup(ctx, [fused, mm])
    red.out.data.fill_(3)
    mp.out.data.fill_(3)
    mm.out.data.fill_(3)
    group.run()
    torch.cuda.synchronize()
    xd, gd = to_np(x), to_np(gam)
    ss_want = O.round_to(O.dense("bsh->bs", [xd], ext, g="square", agg="sum"), "f32")
    y_want = O.round_to(O.dense("bsh,bs,h->bsh", [xd, ss_want, gd], ext, g="rms_scale", agg="none",
                                beta=1.0 / ext["h"], eps=1e-6), "bf16")
    assert normwise_err(O.from_relation(to_np(red.out.data), "bs", ext, blk), ss_want) < F32_TOL
    assert normwise_err(O.from_relation(to_np(mp.out.data), "bsh", ext, blk), y_want) < BF16_OUT_TOL
    mm_want = O.round_to(O.dense("ij,jk->ik", [to_np(a), to_np(b)], dict(i=256, j=512, k=192)), "f32")
    assert normwise_err(O.from_relation(to_np(mm.out.data), "ik", dict(i=256, j=512, k=192), cblk), mm_want) < F32_TOL
    # an input blocked otherwise than the spec asks is re-blocked by the plan:
    # the pair is refused as unsupported (the two plans still run apart)
    X = jagg.from_dense(ctx, x.to("cuda"), "bsh", dict(b=1, s=4, h=4))
    G = jagg.from_dense(ctx, gam.to("cuda"), "h", blk)
    red2 = jagg.EinsumCall(ctx, "bsh->bs", [X], blk, g="square", agg="sum", out_dtype="f32")
    mp2 = jagg.EinsumCall(ctx, "bsh,bs,h->bsh", [X, red2.out, G], blk, g="rms_scale", agg="none",
                          out_dtype="bf16", beta=1.0 / ext["h"], eps=1e-6)
    with pytest.raises(jagg.JaggError) as e:
        jagg.PlanFused(ctx, red2, mp2)
    assert e.value.status == -4
