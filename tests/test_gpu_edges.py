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
    """A relation of 2^36 elements, or of 2^31 tuples, is refused before
    anything is touched; one just under the limits is accepted (metadata
    only: nothing reads the buffer)."""
    buf = torch.empty(16, dtype=torch.uint8, device="cuda")
    h = jagg.ctypes.c_void_p()
    L = jagg.lib()

    def create(ext, blk):
        ctx._check(L.jagg_relation_create(ctx.handle, b"ij", jagg._i64(ext), jagg._i32(blk), jagg.DT["bf16"],
                                          jagg.ctypes.c_void_p(buf.data_ptr()), 1 << 40, jagg.ctypes.byref(h)))
        L.jagg_relation_destroy(h)

    with pytest.raises(jagg.JaggError, match="2\\^36"):
        create([1 << 18, 1 << 18], [1, 1])
    with pytest.raises(jagg.JaggError, match="2\\^31"):
        create([1 << 16, 1 << 16], [1 << 16, 1 << 15])
    create([(1 << 18) - 1, 1 << 18], [1, 1])
    create([1 << 16, (1 << 15) - 1], [1 << 16, (1 << 15) - 1])  # 2^31 - 2^16 one-element tuples


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


# Causal outputs: a tuple whose t-block lies after its s-block has no joined
# tuple and is absent from the output relation.  Its slot must be left as it
# was (never written, never read), while every present tuple -- the masked
# elements t > s of the diagonal tuples and the padding included -- is exact.
CAUSAL_OUT_CASES = [
    # spec, g, agg, extents, blockings, in dtypes, out dtype, positive inputs
    ("bqsd,bqtd->bqst", "mul", "sum", dict(b=1, q=2, s=300, t=300, d=64), dict(b=1, q=1, s=3, t=3, d=1),
     ["bf16", "bf16"], "f32", ()),
    # the LDS-pipelined kernel (256 x 256 tiles) with the mask in its epilogue
    ("bhsd,bhtd->bhst", "mul", "sum", dict(b=2, h=4, s=1056, t=1056, d=128), dict(b=1, h=1, s=4, t=4, d=1),
     ["bf16", "bf16"], "f32", ()),
    ("qst,qs,qs->qst", "exp_sub_div", "none", dict(q=3, s=200, t=200), dict(q=1, s=4, t=4), ["f32", "f32", "f32"],
     "bf16", (2,)),
    ("qst,qs,qs->qst", "exp_sub_div", "none", dict(q=3, s=256, t=256), dict(q=1, s=4, t=4), ["f32", "f32", "f32"],
     "bf16", (2,)),
]


@pytest.mark.parametrize("spec,g,agg,ext,blk,idts,odt,pos", CAUSAL_OUT_CASES)
def test_causal_absent_tuples_are_never_written(ctx, spec, g, agg, ext, blk, idts, odt, pos):
    ins, out = spec.split("->")
    ins = ins.split(",")
    xs = []
    for j, (lt, gen, dt) in enumerate(zip(ins, I.streams(41, len(ins)), idts)):
        x = I.draw(gen, [ext[c] for c in lt], "normal", dt)
        if j in pos:
            x = (x.float().abs() + 0.5).to(x.dtype)
        xs.append(x)
    rels = [jagg.from_dense(ctx, x.to("cuda"), lt, blk) for x, lt in zip(xs, ins)]
    call = jagg.EinsumCall(ctx, spec, rels, blk, g=g, agg=agg, out_dtype=odt, causal=("s", "t"))
    # the binding clears a causal output once when it allocates it
    assert torch.count_nonzero(call.out.data).item() == 0
    call.out.data.fill_(float("nan"))
    call.run()
    torch.cuda.synchronize()
    got_rel = to_np(call.out.data)
    want = O.round_to(O.dense(spec, [to_np(x) for x in xs], ext, g=g, agg=agg, causal=("s", "t")), odt)
    want_rel = O.to_relation(want, out, ext, blk)
    # which tuples are present: t-block <= s-block
    kidx = np.indices([blk[c] for c in out]).reshape(len(out), -1)
    present = kidx[out.index("t")] <= kidx[out.index("s")]
    per = got_rel.size // present.size
    got_t, want_t = got_rel.reshape(present.size, per), want_rel.reshape(present.size, per)
    assert np.all(np.isnan(got_t[~present])), "an absent tuple's slot was written"
    assert not np.isnan(got_t[present]).any(), "a present tuple was left unwritten"
    pad = padding_mask(out, ext, blk).reshape(present.size, per)
    assert np.all(got_t[present][pad[present]] == 0.0), "padding of present tuples must be +0"
    # masked elements t > s inside the diagonal tuples are written as 0
    tmask = O.to_relation(np.triu(np.ones((ext["s"], ext["t"]), dtype=np.uint8), 1)[None].repeat(
        int(np.prod([ext[c] for c in out[:-2]])), 0).reshape([ext[c] for c in out]), out, ext, blk)
    tmask = tmask.reshape(present.size, per).astype(bool)
    assert np.all(got_t[present][tmask[present]] == 0.0), "elements with t > s must be +0"
    err = normwise_err(got_t[present], want_t[present])
    tol = F32_TOL if odt == "f32" else 8e-3
    assert err < tol, f"normwise error {err:.3e}"


def test_causal_output_densifies_with_zeros_above_the_diagonal(ctx):
    """With the binding's zeroed allocation, a densified causal score relation
    equals the oracle's dense result everywhere (t > s gives +0)."""
    spec, ext, blk = "qsd,qtd->qst", dict(q=2, s=200, t=200, d=64), dict(q=1, s=4, t=4, d=1)
    xs = [I.draw(gen, [2, 200, 64], "normal", "bf16") for gen in I.streams(43, 2)]
    rels = [jagg.from_dense(ctx, x.to("cuda"), lt, blk) for x, lt in zip(xs, ("qsd", "qtd"))]
    call = jagg.EinsumCall(ctx, spec, rels, blk, causal=("s", "t"))
    call.run()
    got = to_np(jagg.to_dense(ctx, call.out))
    want = O.round_to(O.dense(spec, [to_np(x) for x in xs], ext, causal=("s", "t")), "f32")
    assert np.all(got[:, np.triu_indices(200, 1)[0], np.triu_indices(200, 1)[1]] == 0.0)
    assert normwise_err(got, want) < F32_TOL


def test_attention_joined_tuple_limit(ctx):
    """The fused attention kernel keeps a key's joined K/V tuples in an LDS
    table of 512 entries: t blocked 520 ways is refused before any launch,
    512 ways runs."""
    def call(nt):
        ext = dict(s=64, t=8 * nt, d=64, e=64)
        blk = dict(s=1, t=nt, d=1, e=1)
        rels = [jagg.Relation(ctx, lt, [ext[c] for c in lt], [blk[c] for c in lt], "bf16", zeroed=True)
                for lt in ("sd", "td", "te")]
        return jagg.EinsumCall(ctx, "sd,td,te->se", rels, blk, g="attention", agg="softmax", alpha=0.125)
    with pytest.raises(jagg.JaggError, match="512"):
        call(520).run()
    c = call(512)
    c.run()
    torch.cuda.synchronize()
    # all-zero inputs: uniform probabilities over zero values
    assert torch.count_nonzero(c.out.data).item() == 0
