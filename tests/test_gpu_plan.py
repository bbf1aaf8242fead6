"""Prepared specs (jagg_plan_create / jagg_plan_run), through the C ABI.

A plan does the host planning and the join once; each run launches the
block kernel (and any re-blocking) on the relations' current contents.  So
a planned chain must reproduce the unplanned one bit for bit, a plan must
follow new input values, and a plan whose input is blocked differently from
`blockings` re-blocks it on every run.  Values are checked against the
oracle at the usual bars (1e-5 fp32; 8e-3 for one bf16 rounding).
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tensor_relational_einsum_amd import inputs as I
from tensor_relational_einsum_amd import jagg
from tensor_relational_einsum_amd.runner import ChainRunner
from parity_util import normwise_err, padding_mask, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    c = jagg.Context(0)
    yield c
    torch.cuda.synchronize()
    c.close()


@pytest.mark.parametrize("fused", [True, False])
def test_planned_chain_equals_unplanned(ctx, fused):
    w = I.llama_block(b=1, s=256, hid=512, heads=4, d=128, ffn=1376, s_blk=2, h_blk=4, q_blk=2, f_blk=8,
                      fused_attention=fused)
    dense = I.generate(w)
    eager = ChainRunner(ctx, w, dense, planned=False)
    # the fused RMS-norm pair adds its row sums in another order; planning
    # alone must change nothing
    planned = ChainRunner(ctx, w, dense, planned=True, fuse_norms=False)
    for r in (eager, planned):
        for _ in range(2):
            r.run()
    torch.cuda.synchronize()
    for st in w.chain:
        assert torch.equal(planned.rel[st.out].data, eager.rel[st.out].data), f"{st.out} differs"


def test_plan_follows_new_input_values(ctx):
    ext = dict(i=300, j=200, k=170)
    blk = dict(i=3, j=2, k=2)
    gens = I.streams(61, 4)
    xs = [I.draw(gens[0], [300, 200], "normal", "f32"), I.draw(gens[1], [200, 170], "normal", "f32")]
    A = jagg.from_dense(ctx, xs[0].to("cuda"), "ij", blk)
    B = jagg.from_dense(ctx, xs[1].to("cuda"), "jk", blk)
    call = jagg.EinsumCall(ctx, "ij,jk->ik", [A, B], blk).prepare()
    for rep in range(2):
        if rep:
            xs[0] = I.draw(gens[2], [300, 200], "normal", "f32")
            A2 = jagg.from_dense(ctx, xs[0].to("cuda"), "ij", blk)
            A.data.copy_(A2.data)  # new values, same buffer
        call.out.data.fill_(float("nan"))
        call.run_plan()
        torch.cuda.synchronize()
        got_rel = to_np(call.out.data)
        got = O.from_relation(got_rel, "ik", ext, blk)
        want = O.round_to(O.dense("ij,jk->ik", [to_np(x) for x in xs], ext), "f32")
        assert normwise_err(got, want) < 1e-5, f"run {rep}"
        assert np.all(got_rel[padding_mask("ik", ext, blk)] == 0.0)


def test_plan_with_a_reblocked_input(ctx):
    ext = dict(b=2, s=96, h=384, q=4, d=64)
    blk = dict(b=1, s=2, h=4, q=2, d=1)
    gens = I.streams(62, 2)
    x = I.draw(gens[0], [2, 96, 384], "normal", "bf16")
    wq = I.draw(gens[1], [384, 4, 64], "normal", "bf16")
    X = jagg.from_dense(ctx, x.to("cuda"), "bsh", blk)
    W = jagg.from_dense(ctx, wq.to("cuda"), "hqd", dict(h=3, q=1, d=1))  # blocked otherwise
    call = jagg.EinsumCall(ctx, "bsh,hqd->bsqd", [X, W], blk, out_dtype="bf16").prepare()
    # the last bytes of the workspace lie in the re-blocked copy of W, which
    # every run writes again
    assert call.ws_bytes > 384 * 4 * 64 * 2
    call.plan_ws[call.ws_bytes - 256:call.ws_bytes].fill_(0xAB)
    for _ in range(2):
        call.out.data.fill_(float("nan"))
        call.run_plan()
    torch.cuda.synchronize()
    got = O.from_relation(to_np(call.out.data), "bsqd", ext, blk)
    want = O.round_to(O.dense("bsh,hqd->bsqd", [to_np(x), to_np(wq)], ext), "bf16")
    assert normwise_err(got, want) < 8e-3


def test_plan_errors(ctx):
    ext_a = jagg.Relation(ctx, "ij", [8, 8], [1, 1], "f32", zeroed=True)
    ext_b = jagg.Relation(ctx, "jk", [8, 8], [1, 1], "f32", zeroed=True)
    call = jagg.EinsumCall(ctx, "ij,jk->ik", [ext_a, ext_b], dict(i=1, j=1, k=1))
    h = jagg.ctypes.c_void_p()
    with pytest.raises(jagg.JaggError):  # no workspace
        ctx._check(jagg.lib().jagg_plan_create(ctx.handle, jagg.ctypes.byref(call.spec), call.in_arr, 2, call.blk,
                                               call.out.handle, None, 0, jagg.ctypes.byref(h)))
    with pytest.raises(jagg.JaggError):  # no plan
        ctx._check(jagg.lib().jagg_plan_run(ctx.handle, None))


@pytest.fixture(scope="module")
def trace_ctx():
    import os
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


@pytest.mark.parametrize("odt", ["bf16", "f32"])
def test_group_of_projections_shares_one_launch(trace_ctx, capfd, odt):
    """Three projections of one input (the Q, K, V form, 256 x 256 tiles)
    as a plan group: one grouped launch, results equal to the members run
    one by one, bit for bit, and to the oracle on sampled outputs."""
    ctx = trace_ctx
    ext = dict(b=2, s=4096, h=512, q=16, d=128)
    blk = dict(b=1, s=16, h=2, q=4, d=1)
    gens = I.streams(63, 4)
    x = I.draw(gens[0], [2, 4096, 512], "normal", "bf16")
    ws = [I.draw(g, [512, 16, 128], "normal", "bf16", 0.05) for g in gens[1:]]
    X = jagg.from_dense(ctx, x.to("cuda"), "bsh", blk)
    Ws = [jagg.from_dense(ctx, wt.to("cuda"), "hqd", blk) for wt in ws]
    calls = [jagg.EinsumCall(ctx, "bsh,hqd->bsqd", [X, W], blk, out_dtype=odt) for W in Ws]
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
    assert "group of 3: contract bf16 256x256 lds pipeline, one launch" in capfd.readouterr().err
    rng = np.random.default_rng(5)
    for c, ref, wt in zip(calls, solo, ws):
        assert torch.equal(c.out.data, ref), "grouped result differs from the member run alone"
        got = O.from_relation(to_np(c.out.data), "bsqd", ext, blk).reshape(-1)
        idx = np.concatenate([rng.integers(0, got.size, 400), [got.size - 1]])
        want = O.round_to(O.dense("bsh,hqd->bsqd", [to_np(x), to_np(wt)], ext, sample=idx), odt)
        assert normwise_err(got[idx], want) < (1e-5 if odt == "f32" else 8e-3)


def test_group_of_mixed_forms_runs_members_in_turn(ctx):
    """A contraction and a map in one group: no shared launch, same results."""
    ext = dict(i=200, j=130, k=70)
    blk = dict(i=2, j=2, k=2)
    gens = I.streams(64, 3)
    a, b, c = (I.draw(g, [ext[x] for x in lt], "normal", "f32") for g, lt in zip(gens, ("ij", "jk", "ij")))
    A, B, C = (jagg.from_dense(ctx, t.to("cuda"), lt, blk) for t, lt in zip((a, b, c), ("ij", "jk", "ij")))
    mm = jagg.EinsumCall(ctx, "ij,jk->ik", [A, B], blk)
    add = jagg.EinsumCall(ctx, "ij,ij->ij", [A, C], blk, g="add", agg="none")
    group = jagg.PlanGroup(ctx, [mm, add])
    mm.out.data.fill_(float("nan"))
    add.out.data.fill_(float("nan"))
    group.run()
    torch.cuda.synchronize()
    got = O.from_relation(to_np(mm.out.data), "ik", ext, blk)
    assert normwise_err(got, O.round_to(O.dense("ij,jk->ik", [to_np(a), to_np(b)], ext), "f32")) < 1e-5
    got = O.from_relation(to_np(add.out.data), "ij", ext, blk)
    want = O.round_to(O.dense("ij,ij->ij", [to_np(a), to_np(c)], ext, g="add", agg="none"), "f32")
    assert np.array_equal(got, want)


def test_group_rejects_dependent_members(ctx):
    blk = dict(i=1, j=1, k=1)
    A = jagg.Relation(ctx, "ij", [64, 64], [1, 1], "f32", zeroed=True)
    B = jagg.Relation(ctx, "jk", [64, 64], [1, 1], "f32", zeroed=True)
    first = jagg.EinsumCall(ctx, "ij,jk->ik", [A, B], blk)
    second = jagg.EinsumCall(ctx, "ij,jk->ik", [first.out, B], blk)  # reads what the first writes
    with pytest.raises(jagg.JaggError, match="writes what member"):
        jagg.PlanGroup(ctx, [first, second])
