"""jagg_einsum_noalloc (the library's static device scratch as workspace)
against jagg_einsum (a caller-allocated workspace), through the C ABI.

Both run the same kernels on the same inputs, so their outputs must agree
bit for bit; each is also compared with the oracle's dense evaluation at the
spec's tolerance (1e-5 for fp32 results; MAX bit-exact).  Two calls in a row
share the scratch, the second with a smaller input; a call whose workspace
exceeds the scratch is refused before any launch.
"""
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
    c = jagg.Context(0)
    yield c
    torch.cuda.synchronize()
    c.close()


def make_call(ctx, spec, ext, call_blk, in_blks, g="mul", agg="sum", seed=51):
    ins, out = spec.split("->")
    ins = ins.split(",")
    xs = [I.draw(gen, [ext[c] for c in lt], "normal", "f32") for gen, lt in zip(I.streams(seed, len(ins)), ins)]
    rels = [jagg.from_dense(ctx, x.to("cuda"), lt, b) for x, lt, b in zip(xs, ins, in_blks)]
    call = jagg.EinsumCall(ctx, spec, rels, call_blk, g=g, agg=agg)
    want = O.round_to(O.dense(spec, [to_np(x) for x in xs], ext, g=g, agg=agg), "f32")
    return call, want, out


def check_against_workspace_call(ctx, call, want, out, ext, blk, agg):
    ref = call.run().data.clone()
    noalloc_out = jagg.relation_like(ctx, out, ext, blk, "f32")
    noalloc_out.data.fill_(float("nan"))
    call.run_noalloc(noalloc_out)
    torch.cuda.synchronize()
    assert torch.equal(noalloc_out.data, ref), "the scratch call differs from the workspace call"
    got_rel = to_np(noalloc_out.data)
    assert np.all(got_rel[padding_mask(out, ext, blk)] == 0.0), "output padding must be +0"
    got = O.from_relation(got_rel, out, ext, blk)
    if agg == "max":
        assert np.array_equal(got, want)
    else:
        assert normwise_err(got, want) < 1e-5


def test_noalloc_two_calls_in_a_row(ctx):
    # first call: A re-blocked in the scratch (3 MiB) besides the join list
    ext = dict(i=1024, j=768, k=520)
    blk = dict(i=4, j=4, k=2)
    call, want, out = make_call(ctx, "ij,jk->ik", ext, blk, [dict(i=2, j=3), dict(j=4, k=2)])
    assert call.ws_bytes > (1 << 20)
    check_against_workspace_call(ctx, call, want, out, ext, blk, "sum")
    # second call, smaller: a MAX reduce whose input is re-blocked
    ext2 = dict(b=2, h=3, s=40, t=300)
    blk2 = dict(b=1, h=1, s=3, t=4)
    call2, want2, out2 = make_call(ctx, "bhst->bhs", ext2, blk2, [dict(b=1, h=1, s=2, t=3)], g="ident", agg="max")
    assert call2.ws_bytes < call.ws_bytes
    check_against_workspace_call(ctx, call2, want2, out2, ext2, blk2, "max")
    # and the first spec again after the smaller one
    check_against_workspace_call(ctx, call, want, out, ext, blk, "sum")


def test_noalloc_refuses_a_workspace_beyond_the_scratch(ctx):
    """Re-blocking a 64 MiB input needs more than the 32 MiB scratch: the
    call is refused with JAGG_E_WORKSPACE and the output is not touched."""
    blk = dict(i=2, j=2, k=1)
    a = jagg.Relation(ctx, "ij", [4096, 4096], [1, 1], "f32", zeroed=True)
    b = jagg.Relation(ctx, "jk", [4096, 64], [2, 1], "f32", zeroed=True)
    call = jagg.EinsumCall(ctx, "ij,jk->ik", [a, b], blk)
    assert call.ws_bytes > jagg.NOALLOC_SCRATCH_BYTES
    call.out.data.fill_(5.0)
    with pytest.raises(jagg.JaggError, match="static scratch") as e:
        call.run_noalloc()
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert torch.all(call.out.data == 5.0)
