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
    planned = ChainRunner(ctx, w, dense, planned=True)
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
