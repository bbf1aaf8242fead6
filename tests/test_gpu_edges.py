"""Edge cases of the join-agg executor through the C ABI, against the oracle.

Degenerate blockings (every block one element wide; one block per letter;
letters of extent one), the interval limits (32 intervals in one letter; one
interval), the element-count limit of a relation, and a large repartition
compared in full.  Bars as in the other parity tests: bit-exact for
repartition, the fp32 / bf16 normwise tolerances for contractions.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tensor_relational_einsum_amd import inputs as I
from tensor_relational_einsum_amd import jagg
from parity_util import bits, normwise_err, padding_mask, to_np

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    c = jagg.Context(0)
    yield c
    torch.cuda.synchronize()
    c.close()


def run_case(ctx, spec, ext, blk, g="mul", agg="sum", dtype="f32", seed=17):
    ins, out = spec.split("->")
    ins = ins.split(",")
    xs = [I.draw(gen, [ext[c] for c in lt], "normal", dtype) for gen, lt in zip(I.streams(seed, len(ins)), ins)]
    rels = [jagg.from_dense(ctx, x.to("cuda"), lt, blk) for x, lt in zip(xs, ins)]
    call = jagg.EinsumCall(ctx, spec, rels, blk, g=g, agg=agg, out_dtype="f32")
    call.out.data.fill_(3)
    call.run()
    torch.cuda.synchronize()
    got_rel = to_np(call.out.data)
    want = O.round_to(O.dense(spec, [to_np(x) for x in xs], ext, g=g, agg=agg), "f32")
    got = O.from_relation(got_rel, out, ext, blk)
    assert np.all(got_rel[padding_mask(out, ext, blk)] == 0.0)
    return got, want


@pytest.mark.parametrize("spec,ext,blk,g,agg", [
    # every block one element wide: k = n for every letter
    ("ij,jk->ik", dict(i=9, j=7, k=5), dict(i=9, j=7, k=5), "mul", "sum"),
    ("ij->i", dict(i=6, j=11), dict(i=6, j=11), "ident", "max"),
    ("ij,ij->ij", dict(i=5, j=13), dict(i=5, j=13), "add", "none"),
    # one block per letter
    ("ij,jk->ik", dict(i=300, j=257, k=129), dict(i=1, j=1, k=1), "mul", "sum"),
    # letters of extent one
    ("aij,ajk->aik", dict(a=1, i=1, j=1, k=1), dict(a=1, i=1, j=1, k=1), "mul", "sum"),
    ("bij,jk->bik", dict(b=3, i=1, j=64, k=1), dict(b=3, i=1, j=2, k=1), "mul", "sum"),
    ("ij->i", dict(i=1, j=1), dict(i=1, j=1), "square", "sum"),
])
def test_degenerate_blockings(ctx, spec, ext, blk, g, agg):
    got, want = run_case(ctx, spec, ext, blk, g=g, agg=agg)
    if agg == "max":
        assert np.array_equal(got, want)
    else:
        assert normwise_err(got, want) < F32_TOL


def test_interval_limits_in_a_contraction(ctx):
    """32 intervals (the limit) on the contracted letter, one interval on
    an output letter."""
    j_bounds = [0] + [6 * q + (q % 5) for q in range(1, 32)] + [200]
    assert len(j_bounds) == 33 and all(a < b for a, b in zip(j_bounds, j_bounds[1:]))
    ext = dict(i=70, j=200, k=40)
    blk = dict(i=[0, 70], j=j_bounds, k=2)
    got, want = run_case(ctx, "ij,jk->ik", ext, blk)
    assert normwise_err(got, want) < F32_TOL


def test_relation_element_limit(ctx):
    """A relation of 2^31 elements is refused before anything is touched;
    one just under the limit is accepted (metadata only)."""
    buf = torch.empty(16, dtype=torch.uint8, device="cuda")
    h = jagg.ctypes.c_void_p()
    L = jagg.lib()
    big = jagg._i64([1 << 16, 1 << 15])
    with pytest.raises(jagg.JaggError):
        ctx._check(L.jagg_relation_create(ctx.handle, b"ij", big, jagg._i32([1, 1]), jagg.DT["bf16"],
                                          jagg.ctypes.c_void_p(buf.data_ptr()), 1 << 40, jagg.ctypes.byref(h)))
    ok = jagg._i64([(1 << 16) - 1, 1 << 15])
    ctx._check(L.jagg_relation_create(ctx.handle, b"ij", ok, jagg._i32([1, 1]), jagg.DT["bf16"],
                                      jagg.ctypes.c_void_p(buf.data_ptr()), 1 << 40, jagg.ctypes.byref(h)))
    L.jagg_relation_destroy(h)


def test_large_repartition_in_full(ctx):
    """2^28 bf16 elements (512 MiB) re-blocked with a letter permutation and
    ragged blocks, every byte compared with the oracle."""
    shape, src_l, dst_l = (64, 1024, 4096), "abc", "cab"
    src_b, dst_b = dict(a=3, b=8, c=1), dict(a=1, b=5, c=7)
    ext = dict(zip(src_l, shape))
    x = I.draw(I.streams(23, 1)[0], shape, "normal", "bf16")
    src = jagg.from_dense(ctx, x.to("cuda"), src_l, src_b)
    dst = jagg.relation_like(ctx, dst_l, ext, dst_b, "bf16")
    dst.data.fill_(7)
    jagg.repartition(ctx, src, dst)
    torch.cuda.synchronize()
    want_src = O.to_relation(bits(x), src_l, ext, src_b)
    assert np.array_equal(bits(src.data), want_src)
    want = O.repartition(want_src, src_l, src_b, dst_l, dst_b, ext)
    assert np.array_equal(bits(dst.data), want)
