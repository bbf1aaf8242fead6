"""Contractions with a recompose map (g = mul_plus, swiglu), through the C
ABI, against the oracle's dense definitions (oracle_dense_recompose).

mul_plus: out = alpha * sum_r x0 x1 + x2, the addend laid out as the output;
on the general contraction kernel (small and ragged blocks) and on the
LDS-pipelined 256 x 256 kernel.  swiglu: out = alpha * silu(sum_r x0 x1) *
sum_r x0 x2, on the 256 x 128 LDS-pipelined kernel, with the weights
contiguous along the output letter or along the reduced one.  Bars: 1e-5
normwise for an fp32 result, 8e-3 for one bf16 rounding; output padding +0.
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


def run_recompose(ctx, capfd, spec, kind, ext, blk, dtypes, odt, alpha=1.0, seed=71, sigmas=(1.0, 0.05, 0.05),
                  sample=None):
    ins, out = spec.split("->")
    ins = ins.split(",")
    xs = [I.draw(g, [ext[c] for c in lt], "normal", dt, sg)
          for g, lt, dt, sg in zip(I.streams(seed, 3), ins, dtypes, sigmas)]
    rels = [jagg.from_dense(ctx, x.to("cuda"), lt, blk) for x, lt in zip(xs, ins)]
    call = jagg.EinsumCall(ctx, spec, rels, blk, g=kind, agg="sum", out_dtype=odt, alpha=alpha)
    call.out.data.fill_(float("nan"))
    capfd.readouterr()
    call.run()
    torch.cuda.synchronize()
    trace = capfd.readouterr().err
    got_rel = to_np(call.out.data)
    assert np.all(got_rel[padding_mask(out, ext, blk)] == 0.0), "output padding must be +0"
    got = O.from_relation(got_rel, out, ext, blk).reshape(-1)
    if sample is not None:
        rng = np.random.default_rng(seed)
        idx = np.concatenate([rng.integers(0, got.size, sample), [0, got.size - 1]])
        want = O.dense_recompose(spec, kind, [to_np(x) for x in xs], ext, alpha=alpha, sample=idx)
        got = got[idx]
    else:
        want = O.dense_recompose(spec, kind, [to_np(x) for x in xs], ext, alpha=alpha).reshape(-1)
    return got, O.round_to(want, odt), trace


MUL_PLUS_CASES = [
    # spec, extents, blockings, dtypes (x0, x1, addend), out dtype
    ("ij,jk,ik->ik", dict(i=200, j=130, k=70), dict(i=3, j=2, k=2), ["f32", "f32", "f32"], "f32"),
    ("ij,jk,ik->ik", dict(i=200, j=130, k=72), dict(i=3, j=2, k=2), ["bf16", "bf16", "bf16"], "f32"),
    ("bsqd,qdh,bsh->bsh", dict(b=2, s=96, q=4, d=64, h=256), dict(b=1, s=2, q=2, d=1, h=2),
     ["bf16", "bf16", "f32"], "f32"),
    ("bsqd,qdh,bsh->bsh", dict(b=2, s=96, q=4, d=64, h=256), dict(b=1, s=2, q=2, d=1, h=2),
     ["bf16", "bf16", "bf16"], "bf16"),
]


@pytest.mark.parametrize("spec,ext,blk,dts,odt", MUL_PLUS_CASES)
def test_mul_plus_general_kernel(ctx, capfd, spec, ext, blk, dts, odt):
    got, want, _ = run_recompose(ctx, capfd, spec, "mul_plus", ext, blk, dts, odt, alpha=0.5,
                                 sigmas=(1.0, 1.0, 1.0))
    tol = 1e-5 if odt == "f32" else 8e-3
    assert normwise_err(got, want) < tol


@pytest.mark.parametrize("adt,odt", [("f32", "f32"), ("bf16", "f32"), ("f32", "bf16")])
def test_mul_plus_lds_pipeline(ctx, capfd, adt, odt):
    """A residual add fused into a projection on the 256 x 256 pipeline."""
    ext = dict(b=2, s=4096, h=512, n=2048)
    blk = dict(b=1, s=16, h=2, n=4)
    got, want, trace = run_recompose(ctx, capfd, "bsh,hn,bsn->bsn", "mul_plus", ext, blk, ["bf16", "bf16", adt],
                                     odt, sample=3000, sigmas=(1.0, 0.05, 1.0))
    assert "lds pipeline, plus addend" in trace
    assert normwise_err(got, want) < (1e-5 if odt == "f32" else 8e-3)


@pytest.mark.parametrize("wl,nf,odt", [("hf", 1024, "bf16"), ("hf", 1024, "f32"), ("fh", 1000, "bf16")])
def test_swiglu_lds_pipeline(ctx, capfd, wl, nf, odt):
    """The gate and up projections and their product in one contraction;
    weights contiguous along f ('hf') or along the reduced h ('fh', with a
    ragged f block: 1000 = 2 blocks of 500, 4 column tiles, the last short)."""
    ext = dict(b=2, s=4096, h=512, f=nf)
    blk = dict(b=1, s=16, h=2, f=2)
    spec = f"bsh,{wl},{wl}->bsf"
    got, want, trace = run_recompose(ctx, capfd, spec, "swiglu", ext, blk, ["bf16", "bf16", "bf16"], odt,
                                     sample=3000)
    assert "256x128 lds pipeline, swiglu" in trace
    assert normwise_err(got, want) < (1e-5 if odt == "f32" else 8e-3)


# SwiGLU below one 256 x 128 tile and over ragged blocks: the pipeline
# bounds-checks rows and columns, so it takes any extents
SMALL_SWIGLU_CASES = [
    (dict(b=1, s=100, h=64, f=72), dict(b=1, s=1, h=1, f=1)),
    (dict(b=2, s=300, h=128, f=208), dict(b=1, s=2, h=2, f=2)),
]


@pytest.mark.parametrize("ext,blk", SMALL_SWIGLU_CASES)
def test_swiglu_small_and_ragged(ctx, capfd, ext, blk):
    got, want, trace = run_recompose(ctx, capfd, "bsh,hf,hf->bsf", "swiglu", ext, blk, ["bf16", "bf16", "bf16"],
                                     "bf16", alpha=0.75)
    assert "256x128 lds pipeline, swiglu" in trace
    assert normwise_err(got, want) < 8e-3


def test_recompose_rejects(ctx):
    blk = dict(i=1, j=1, k=1)
    rels = [jagg.Relation(ctx, lt, [64, 64], [1, 1], "f32", zeroed=True) for lt in ("ij", "jk", "jk")]
    with pytest.raises(jagg.JaggError, match="SWIGLU"):  # fp32 operands: no 256 x 128 bf16 pipeline
        jagg.EinsumCall(ctx, "ij,jk,jk->ik", rels, blk, g="swiglu", agg="sum").run()
    with pytest.raises(jagg.JaggError):  # the addend holds a reduced letter
        jagg.EinsumCall(ctx, "ij,jk,jk->ik", rels, blk, g="mul_plus", agg="sum").run()
    with pytest.raises(jagg.JaggError):  # a recompose map needs SUM
        jagg.EinsumCall(ctx, "ij,jk,jk->ik", rels, blk, g="swiglu", agg="max").run()


def test_grouped_swiglu_and_mul_plus(ctx, capfd):
    """Two independent SwiGLU contractions of one form share a launch and
    equal their solo runs bit for bit."""
    ext = dict(b=2, s=4096, h=512, f=1024)
    blk = dict(b=1, s=16, h=2, f=2)
    gens = I.streams(72, 5)
    x = I.draw(gens[0], [2, 4096, 512], "normal", "bf16")
    ws = [I.draw(g, [512, 1024], "normal", "bf16", 0.05) for g in gens[1:]]
    X = jagg.from_dense(ctx, x.to("cuda"), "bsh", blk)
    W = [jagg.from_dense(ctx, t.to("cuda"), "hf", blk) for t in ws]
    calls = [jagg.EinsumCall(ctx, "bsh,hf,hf->bsf", [X, W[0], W[1]], blk, g="swiglu", out_dtype="bf16"),
             jagg.EinsumCall(ctx, "bsh,hf,hf->bsf", [X, W[2], W[3]], blk, g="swiglu", out_dtype="bf16")]
    solo = []
    for c in calls:
        c.prepare().run_plan()
        solo.append(c.out.data.clone())
    group = jagg.PlanGroup(ctx, calls)
    for c in calls:
        c.out.data.fill_(float("nan"))
    capfd.readouterr()
    group.run()
    torch.cuda.synchronize()
    assert "group of 2" in capfd.readouterr().err
    for c, ref in zip(calls, solo):
        assert torch.equal(c.out.data, ref)
