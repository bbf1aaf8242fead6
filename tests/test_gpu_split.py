"""Split walks: a bf16 contraction whose 256 x 256 tiles fill the chip in few
or ragged waves runs its (joined tuple, K-step) walk in parts, each writing
fp32 partial sums, and a sum kernel adds the parts in order (JAGG_TRACE
names the split).  Against the oracle's dense definition on the same bf16
inputs: 1e-5 normwise for an f32 result, 8e-3 for one bf16 rounding;
output padding +0.  Cases: parts that start inside a joined tuple and cross
tuple boundaries, parts over one-step tuples, a ragged last K-tile, ragged M
and N, a batch letter, alpha != 1, and a contraction with enough tiles that
takes no split.
"""
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O
from parity_util import normwise_err, padding_mask, to_np
from tensor_relational_einsum_amd import inputs as I
from tensor_relational_einsum_amd import jagg

pytestmark = pytest.mark.gpu


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


CASES = [
    # spec, extents, blockings, out dtype, alpha, parts expected in the trace (None: no split)
    # 4 tiles, 256 steps in one tuple: 16 parts of 16 steps
    ("ij,jk->ik", dict(i=512, j=8192, k=512), dict(i=1, j=1, k=1), "bf16", 0.5, 16),
    # 3 tuples of 81 K-tiles (2568 = 80 x 32 + 8): 8 parts of about 30 steps
    # that start inside tuples and cross tuple boundaries
    ("ij,jk->ik", dict(i=512, j=7704, k=512), dict(i=1, j=3, k=1), "bf16", 1.0, 8),
    # 256 joined tuples of one K-step each: every part starts on a tuple
    ("ij,jk->ik", dict(i=512, j=8192, k=512), dict(i=1, j=256, k=1), "bf16", 1.0, 16),
    # ragged M and N, an f32 result
    ("ij,jk->ik", dict(i=300, j=4096, k=704), dict(i=1, j=1, k=1), "f32", 1.0, 8),
    # a batch letter
    ("bij,bjk->bik", dict(b=2, i=256, j=4096, k=256), dict(b=2, i=1, j=1, k=1), "bf16", 1.0, 8),
    # 256 tiles of 32 steps: one full wave, no split
    ("ij,jk->ik", dict(i=4096, j=1024, k=4096), dict(i=1, j=1, k=1), "bf16", 1.0, None),
]


@pytest.mark.parametrize("spec,ext,blk,odt,alpha,parts", CASES)
def test_split_walk_parity(ctx, capfd, spec, ext, blk, odt, alpha, parts):
    ins, out = spec.split("->")
    ins = ins.split(",")
    gens = I.streams(131, 2)
    xs = [I.draw(g, [ext[c] for c in lt], "normal", "bf16", 1.0 / np.sqrt(ext["j"]) if k else 1.0)
          for k, (g, lt) in enumerate(zip(gens, ins))]
    rels = [jagg.from_dense(ctx, x.to("cuda"), lt, blk) for x, lt in zip(xs, ins)]
    call = jagg.EinsumCall(ctx, spec, rels, blk, g="mul", agg="sum", out_dtype=odt, alpha=alpha)
    call.workspace.fill_(0xA5)
    call.out.data.fill_(float("nan"))
    print(f"[test] split walk {spec} {ext} {blk} -> {odt}", flush=True)
    capfd.readouterr()
    call.run()
    torch.cuda.synchronize()
    trace = capfd.readouterr().err
    if parts is None:
        assert "split walk" not in trace, trace
    else:
        assert f"walk in {parts} parts" in trace, trace
    got_rel = to_np(call.out.data)
    assert np.all(got_rel[padding_mask(out, ext, blk)] == 0.0), "output padding must be +0"
    want = O.round_to(O.dense(spec, [to_np(x) for x in xs], ext, g="mul", agg="sum", alpha=alpha), odt)
    got = O.from_relation(got_rel, out, ext, blk)
    tol = 1e-5 if odt == "f32" else 8e-3
    assert normwise_err(got, want) < tol


@pytest.fixture(scope="module")
def sctx():
    # capture needs a stream other than the null stream
    s = torch.cuda.Stream()
    old = os.environ.get("JAGG_TRACE")
    os.environ["JAGG_TRACE"] = "1"
    try:
        with torch.cuda.stream(s):
            c = jagg.Context(0, s)
    finally:
        if old is None:
            del os.environ["JAGG_TRACE"]
        else:
            os.environ["JAGG_TRACE"] = old
    with torch.cuda.stream(s):
        yield c
        torch.cuda.synchronize()
        c.close()


def test_split_walk_plan_and_graph_replays(sctx, capfd):
    # a prepared plan and replays of a captured graph give the eager result
    ctx = sctx
    spec, ext, blk = "ij,jk->ik", dict(i=512, j=7704, k=512), dict(i=1, j=3, k=1)
    gens = I.streams(7, 2)
    a = I.draw(gens[0], [512, 7704], "normal", "bf16")
    b = I.draw(gens[1], [7704, 512], "normal", "bf16", 1.0 / np.sqrt(7704))
    A = jagg.from_dense(ctx, a.to("cuda"), "ij", blk)
    B = jagg.from_dense(ctx, b.to("cuda"), "jk", blk)
    call = jagg.EinsumCall(ctx, spec, [A, B], blk, g="mul", agg="sum", out_dtype="bf16")
    capfd.readouterr()
    call.run()
    torch.cuda.synchronize()
    assert "walk in 8 parts" in capfd.readouterr().err
    eager = call.out.data.clone()
    call.prepare()
    call.out.data.fill_(float("nan"))
    call.run_plan()
    torch.cuda.synchronize()
    assert torch.equal(call.out.data, eager)
    g = jagg.capture(ctx, call.run_plan)
    for _ in range(3):
        call.out.data.fill_(float("nan"))
        torch.cuda.synchronize()
        g.launch()
        torch.cuda.synchronize()
        assert torch.equal(call.out.data, eager)
    g.close()


def test_split_walk_with_a_reblocked_input(ctx, capfd):
    # A arrives blocked (i 2, j 2) while the spec asks (i 1, j 3): the
    # re-blocked copy and the partial sums share the workspace
    ext, blk = dict(i=512, j=7704, k=512), dict(i=1, j=3, k=1)
    gens = I.streams(17, 2)
    a = I.draw(gens[0], [512, 7704], "normal", "bf16")
    b = I.draw(gens[1], [7704, 512], "normal", "bf16", 1.0 / np.sqrt(7704))
    A = jagg.from_dense(ctx, a.to("cuda"), "ij", dict(i=2, j=2))
    B = jagg.from_dense(ctx, b.to("cuda"), "jk", blk)
    call = jagg.EinsumCall(ctx, "ij,jk->ik", [A, B], blk, g="mul", agg="sum", out_dtype="f32")
    call.workspace.fill_(0x5A)
    capfd.readouterr()
    call.run()
    torch.cuda.synchronize()
    trace = capfd.readouterr().err
    assert "reblock input 0" in trace and "walk in 8 parts" in trace, trace
    want = O.dense("ij,jk->ik", [to_np(a), to_np(b)], ext, g="mul", agg="sum")
    got = O.from_relation(to_np(call.out.data), "ik", ext, blk)
    assert normwise_err(got, want) < 1e-5


def test_noalloc_runs_the_walk_whole(ctx, capfd):
    # the no-allocation entry point never splits; its result agrees with the
    # split call up to the order of the fp32 additions
    ext, blk = dict(i=512, j=7704, k=512), dict(i=1, j=3, k=1)
    gens = I.streams(19, 2)
    a = I.draw(gens[0], [512, 7704], "normal", "bf16")
    b = I.draw(gens[1], [7704, 512], "normal", "bf16", 1.0 / np.sqrt(7704))
    A = jagg.from_dense(ctx, a.to("cuda"), "ij", blk)
    B = jagg.from_dense(ctx, b.to("cuda"), "jk", blk)
    call = jagg.EinsumCall(ctx, "ij,jk->ik", [A, B], blk, g="mul", agg="sum", out_dtype="f32")
    capfd.readouterr()
    call.run()
    torch.cuda.synchronize()
    assert "walk in 8 parts" in capfd.readouterr().err
    split = to_np(call.out.data)
    whole = jagg.relation_like(ctx, "ik", ext, blk, "f32")
    capfd.readouterr()
    call.run_noalloc(whole)
    torch.cuda.synchronize()
    assert "split walk" not in capfd.readouterr().err
    assert normwise_err(to_np(whole.data), split) < 1e-5
