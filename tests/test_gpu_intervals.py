"""Interval-blocked relations on the GPU, through the C ABI, against the oracle.

"Every Kernel Is a Join" (Ding et al.): a key is an interval per index
(Def. 3.1), and an index may be split only at legal positions (Sec. 3.3,
Example 3.10: a packed sequence index at the ends of its sequences, query
heads along with their key-value heads).  A blocking value here is a list of
bounds; blocks pad to the longest interval.

Bit-exact: every byte of a repartition (padding included) against the
oracle's.  Floating point: the normwise error of parity_util under the same
tolerances as the uniform cases (1e-5 for fp32 results, 8e-3 for one bf16
rounding of an fp32-accumulated result).
"""
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O
from tensor_relational_einsum_amd import inputs as I
from tensor_relational_einsum_amd import jagg
from parity_util import bits, normwise_err, padding_mask, to_np

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5
BF16_OUT_TOL = 8e-3
PACKED = [0, 1024, 2560, 4096]  # three packed sequences ending at 1024, 2560, 4096


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


def upload(ctx, x, letters, blk):
    return jagg.from_dense(ctx, x.to("cuda"), letters, blk)


def check_relayout(ctx, shape, src_l, src_b, dst_l, dst_b, dtype, seed=0):
    ext = dict(zip(src_l, shape))
    x = I.draw(I.streams(seed, 1)[0], shape, "normal", dtype)
    src = upload(ctx, x, src_l, src_b)
    dst = jagg.relation_like(ctx, dst_l, ext, dst_b, dtype)
    dst.data.fill_(7)  # every byte must be rewritten, padding included
    jagg.repartition(ctx, src, dst)
    torch.cuda.synchronize()
    want_src = O.to_relation(bits(x), src_l, ext, src_b)
    assert np.array_equal(bits(src.data), want_src), "dense -> blocked relation differs"
    want = O.repartition(want_src, src_l, src_b, dst_l, dst_b, ext)
    got = bits(dst.data)
    assert got.shape == want.shape
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} elements differ, first at {bad[:5]}"
    back = jagg.relation_like(ctx, src_l, ext, src_b, dtype)
    jagg.repartition(ctx, dst, back)
    dense = jagg.to_dense(ctx, dst)
    torch.cuda.synchronize()
    assert np.array_equal(bits(back.data), want_src), "round trip differs"
    perm = [src_l.index(c) for c in dst_l]
    assert np.array_equal(bits(dense), bits(x).transpose(perm)), "download differs"


RELAYOUT_CASES = [
    # packed sequences <-> uniform blocks (16-byte vectors along d)
    ((4096, 128), "sd", dict(s=PACKED), "sd", dict(s=4), "bf16"),
    ((4096, 128), "sd", dict(s=4, d=2), "sd", dict(s=PACKED, d=[0, 32, 128]), "bf16"),
    ((8, 4096, 64), "bsd", dict(b=2, s=PACKED), "sbd", dict(s=PACKED, b=4), "bf16"),
    # ragged bounds that are no multiple of a vector: element-wise copies
    ((11, 6), "ij", dict(i=[0, 3, 4, 11], j=2), "ji", dict(i=[0, 5, 11], j=[0, 1, 6]), "f32"),
    ((7, 5, 6), "abc", dict(a=2, b=[0, 2, 5], c=3), "cab", dict(a=[0, 1, 7], b=1, c=[0, 4, 6]), "f32"),
    ((7, 5, 6), "abc", dict(a=2, b=[0, 2, 5], c=3), "cab", dict(a=[0, 1, 7], b=1, c=[0, 4, 6]), "bf16"),
    # query heads blocked as intervals derived from 8 key-value heads
    ((32, 256, 128), "hsd", dict(h=[4 * m for m in range(9)]), "hsd", dict(h=2, s=2), "bf16"),
    # long rows along the innermost letter: a wave streams each row
    ((2, 1000, 1024), "bsh", dict(s=[0, 100, 356, 1000]), "sbh", dict(s=3, b=2), "bf16"),
    ((300, 2048), "sh", dict(s=2, h=[0, 512, 2048]), "sh", dict(s=[0, 7, 300], h=[0, 1000, 2048]), "f32"),
    ((64, 1001), "ab", dict(b=[0, 500, 1001]), "ab", dict(a=2, b=1), "f32"),
    # one interval per letter, and 32 intervals (the limit)
    ((5, 9), "ab", dict(a=[0, 5], b=[0, 9]), "ba", dict(a=5, b=3), "f32"),
    ((64, 40), "ab", dict(a=list(range(0, 32)) + [64]), "ab", dict(a=3, b=[0, 8, 40]), "f32"),
]


@pytest.mark.parametrize("shape,src_l,src_b,dst_l,dst_b,dtype", RELAYOUT_CASES)
def test_interval_repartition_bit_exact(ctx, shape, src_l, src_b, dst_l, dst_b, dtype):
    check_relayout(ctx, shape, src_l, src_b, dst_l, dst_b, dtype)


def test_packed_sequence_relayout_uses_vectors(ctx, capfd):
    check_relayout(ctx, (4096, 256), "sd", dict(s=1), "sd", dict(s=PACKED), "bf16")
    lines = [ln for ln in capfd.readouterr().err.splitlines() if "relayout sd -> sd: intervals" in ln]
    assert lines and all("8-element vectors" in ln for ln in lines), lines


def test_packed_sequence_long_rows_use_row_form(ctx, capfd):
    check_relayout(ctx, (2, 4096, 1024), "bsh", dict(s=1), "bsh", dict(s=PACKED), "bf16")
    check_relayout(ctx, (2, 4096, 1024), "bsh", dict(s=PACKED), "bsh", dict(s=4), "bf16")
    lines = [ln for ln in capfd.readouterr().err.splitlines() if "relayout bsh -> bsh: intervals" in ln]
    assert lines and all("8-element vectors" in ln and ln.endswith(", rows") for ln in lines), lines


def test_gqa_interval_heads_equal_split_heads(ctx):
    """Example 3.10: query heads [4m, 4m+4) as an interval blocking of heads_q
    hold the same bytes as the query tensor viewed [kv, group, s, d] and blocked
    by key-value head."""
    x = I.draw(I.streams(3, 1)[0], (32, 64, 128), "normal", "bf16")
    a = upload(ctx, x, "hsd", dict(h=[4 * m for m in range(9)], s=2))
    b = upload(ctx, x.view(8, 4, 64, 128), "grsd", dict(g=8, s=2))
    torch.cuda.synchronize()
    assert np.array_equal(bits(a.data), bits(b.data))


def run_iv_spec(ctx, spec, ext, blk, g="mul", agg="sum", in_dtypes=None, out_dtype="f32", beta=0.0, eps=0.0,
                positive=(), seed=5):
    ins, out = spec.split("->")
    ins = ins.split(",")
    in_dtypes = in_dtypes or ["f32"] * len(ins)
    xs = []
    for j, (lt, gen, dt) in enumerate(zip(ins, I.streams(seed, len(ins)), in_dtypes)):
        x = I.draw(gen, [ext[c] for c in lt], "normal", dt)
        if j in positive:
            x = (x.float().abs() + 0.5).to(x.dtype)
        xs.append(x)
    rels = [upload(ctx, x, lt, blk) for x, lt in zip(xs, ins)]
    call = jagg.EinsumCall(ctx, spec, rels, blk, g=g, agg=agg, out_dtype=out_dtype, beta=beta, eps=eps)
    call.out.data.fill_(3)
    call.run()
    torch.cuda.synchronize()
    got_rel = to_np(call.out.data)
    xs64 = [to_np(x) for x in xs]
    want = O.round_to(O.dense(spec, xs64, ext, g=g, agg=agg, beta=beta, eps=eps), out_dtype)
    got = O.from_relation(got_rel, out, ext, blk)
    # the relational oracle over the same interval keys agrees with the dense one
    want_rel, present = O.relational(spec, [O.to_relation(x, lt, ext, blk) for x, lt in zip(xs64, ins)], ext, blk,
                                     g=g, agg=agg, beta=beta, eps=eps)
    assert present.all()
    pad = padding_mask(out, ext, blk)
    assert np.all(got_rel[pad] == 0.0), "padding of the output must be +0"
    return got, want, got_rel, want_rel, pad


IV_SPEC_CASES = [
    # spec, extents, blockings, g, agg, in dtypes, out dtype, positive inputs
    # packed-sequence projection: the GEMM runs on 1536-row padded blocks
    ("sh,ho->so", dict(s=4096, h=512, o=256), dict(s=PACKED, h=2), "mul", "sum", "bf16", "bf16", ()),
    ("sh,ho->so", dict(s=4096, h=256, o=384), dict(s=PACKED, o=[0, 128, 384]), "mul", "sum", "bf16", "f32", ()),
    # contraction over the interval letter (gradient of a weight over packed tokens)
    ("sh,so->ho", dict(s=600, h=96, o=64), dict(s=[0, 100, 356, 600], h=1, o=1), "mul", "sum", "f32", "f32", ()),
    ("bsh,hqd->bsqd", dict(b=2, s=300, h=128, q=4, d=64), dict(b=1, s=[0, 44, 300], h=2, q=2), "mul", "sum", "bf16",
     "f32", ()),
    # streaming reduces and maps
    ("bsh->bs", dict(b=2, s=777, h=256), dict(b=1, s=[0, 77, 700, 777], h=[0, 96, 256]), "square", "sum", "f32",
     "f32", ()),
    ("bsh->bs", dict(b=2, s=200, h=64), dict(s=[0, 50, 200], h=2), "ident", "max", "f32", "f32", ()),
    ("bsh,bsh->bsh", dict(b=2, s=300, h=64), dict(s=[0, 100, 300], h=[0, 16, 64]), "add", "none", "f32", "f32", ()),
    ("bsf,bsf->bsf", dict(b=1, s=260, f=96), dict(s=[0, 4, 260], f=3), "silu_mul", "none", "bf16", "bf16", ()),
    ("bsh,bs,h->bsh", dict(b=2, s=130, h=64), dict(s=[0, 30, 130], h=2), "rms_scale", "none", "f32", "f32", (1,)),
]


@pytest.mark.parametrize("spec,ext,blk,g,agg,idt,odt,positive", IV_SPEC_CASES)
def test_interval_einsum_parity(ctx, spec, ext, blk, g, agg, idt, odt, positive):
    n_in = len(spec.split("->")[0].split(","))
    kw = dict(beta=1.0 / ext.get("h", 1), eps=1e-5) if g == "rms_scale" else {}
    got, want, got_rel, want_rel, pad = run_iv_spec(ctx, spec, ext, blk, g=g, agg=agg, in_dtypes=[idt] * n_in,
                                                    out_dtype=odt, positive=positive, **kw)
    tol = F32_TOL if (odt == "f32" and idt == "f32") else (BF16_OUT_TOL if odt == "bf16" else 1e-4)
    if agg == "max":
        assert np.array_equal(got, want)
    else:
        err = normwise_err(got, want)
        assert err < tol, f"normwise error {err:.3g} over {tol:g}"
    # relation to relation, padding included
    err = normwise_err(got_rel, O.round_to(want_rel, odt))
    assert err < max(tol, 1e-5)


def test_gqa_scores_and_values_by_kv_head(ctx):
    """Example 3.10 on the split head index: g (key-value heads) blocked into
    its 8 unit intervals gives 8 specifications per key; scores and the
    value product run as contractions with the query group r in the rows."""
    ext = dict(g=8, r=4, s=128, t=128, d=64, e=64)
    blk = dict(g=8, s=2, t=2)
    got, want, *_ = run_iv_spec(ctx, "grsd,gtd->grst", ext, blk, in_dtypes=["bf16", "bf16"])
    assert normwise_err(got, want) < 1e-4
    got, want, *_ = run_iv_spec(ctx, "grst,gte->grse", ext, blk, in_dtypes=["bf16", "bf16"])
    assert normwise_err(got, want) < 1e-4


def make(ctx, letters, ext, blk, dtype="f32"):
    r = jagg.relation_like(ctx, letters, ext, blk, dtype)
    r.data.zero_()
    return r


@pytest.mark.parametrize("spec,g,agg,blk_a,blk_b", [
    ("st->s", "ident", "max", dict(s=2, t=[0, 3, 8]), None),            # MAX over an interval letter
    ("st,s->st", "exp_sub", "none", dict(s=[0, 3, 8], t=2), None),     # exp(0 - 0) != 0 in padding
    ("st,s->st", "add", "none", dict(s=2, t=[0, 3, 8]), None),         # t missing from the second input
    ("st,tu->su", "mul", "sum", dict(s=2, t=[0, 3, 8], u=1), dict(t=[0, 4, 8], u=1)),  # bounds differ
    ("st,tu->su", "mul", "sum", dict(s=2, t=[0, 3, 8], u=1), dict(t=2, u=1)),          # interval vs uniform
])
def test_interval_einsum_rejects(ctx, spec, g, agg, blk_a, blk_b):
    ext = dict(s=8, t=8, u=8)
    ins, out = spec.split("->")
    ins = ins.split(",")
    blks = [blk_a, blk_b or blk_a]
    rels = [make(ctx, lt, ext, b) for lt, b in zip(ins, blks)]
    with pytest.raises(jagg.JaggError):
        jagg.EinsumCall(ctx, spec, rels, blk_a, g=g, agg=agg).run()


def test_interval_rms_scale_needs_positive_eps(ctx):
    """A padded row of an interval letter computes 0 * rsqrt(0 * beta + eps):
    +0 for eps > 0 (checked with padding by test_interval_einsum_parity),
    NaN for eps = 0, so eps <= 0 is refused before any launch."""
    ext = dict(s=8, h=8)
    blk = dict(s=[0, 3, 8], h=2)
    rels = [make(ctx, lt, ext, blk) for lt in ("sh", "s", "h")]
    for eps in (0.0, -1e-6):
        with pytest.raises(jagg.JaggError, match="eps"):
            jagg.EinsumCall(ctx, "sh,s,h->sh", rels, blk, g="rms_scale", agg="none", beta=0.125, eps=eps).run()
    jagg.EinsumCall(ctx, "sh,s,h->sh", rels, blk, g="rms_scale", agg="none", beta=0.125, eps=1e-6).run()


def test_interval_relation_rejects_bad_bounds(ctx):
    for bnd in ([1, 4, 8], [0, 4, 7], [0, 4, 4, 8], [0, 5, 3, 8]):
        with pytest.raises(jagg.JaggError):
            jagg.Relation(ctx, "a", [8], [bnd], "f32")
    with pytest.raises(jagg.JaggError):  # 33 intervals
        jagg.Relation(ctx, "a", [64], [list(range(33)) + [64]], "f32")


# ----------------------------------------------------------- packed attention
# Example 3.10: attention never crosses a sequence end; with s and t blocked
# at the sequence ends and a segment pair (s, t), each query block joins the
# key block of its own sequence only, and the kernel masks each block by its
# own interval's length.

def run_packed_attention(ctx, spec, ext, blk, bounds, causal, odt, seed=11):
    ins, out = spec.split("->")
    ins = ins.split(",")
    xs = [I.draw(g, [ext[c] for c in lt], "normal", "bf16") for g, lt in zip(I.streams(seed, 3), ins)]
    rels = [upload(ctx, x, lt, blk) for x, lt in zip(xs, ins)]
    alpha = 1.0 / ext["d"] ** 0.5
    call = jagg.EinsumCall(ctx, spec, rels, blk, g="attention", agg="softmax", out_dtype=odt, alpha=alpha,
                           causal=causal, segment=("s", "t"))
    call.out.data.fill_(5)
    call.run()
    torch.cuda.synchronize()
    got_rel = to_np(call.out.data)
    xs64 = [to_np(x) for x in xs]
    want = O.round_to(O.attention_dense(spec, xs64, ext, alpha=alpha, causal=causal, segments=("s", "t", bounds)),
                      odt)
    got = O.from_relation(got_rel, out, ext, blk)
    pad = padding_mask(out, ext, blk)
    assert np.all(got_rel[pad] == 0.0), "padding rows of short sequences must be +0"
    return got, want, got_rel, xs64


PACKED_ATT = [
    # spec, extents, blockings (s and t alike), causal, out dtype
    ("bhsd,bhtd,bhte->bhse", dict(b=1, h=2, s=1000, t=1000, d=128, e=128), [0, 200, 456, 1000], ("s", "t"), "bf16"),
    ("bhsd,bhtd,bhte->bhse", dict(b=2, h=1, s=600, t=600, d=64, e=64), [0, 64, 300, 301, 600], None, "f32"),
    # grouped-query attention over packed sequences: both halves of Example 3.10
    ("grsd,gtd,gte->grse", dict(g=2, r=4, s=700, t=700, d=128, e=128), [0, 129, 700], ("s", "t"), "bf16"),
]


@pytest.mark.parametrize("spec,ext,bounds,causal,odt", PACKED_ATT)
def test_packed_sequence_attention(ctx, spec, ext, bounds, causal, odt):
    blk = {c: 1 for c in ext}
    blk.update(s=bounds, t=bounds)
    if spec.startswith("grsd"):
        blk["g"] = ext["g"]
    got, want, got_rel, xs64 = run_packed_attention(ctx, spec, ext, blk, bounds, causal, odt)
    err = normwise_err(got, want)
    assert err < BF16_OUT_TOL, f"normwise error {err:.3e}"


def test_packed_attention_matches_relational_oracle(ctx):
    """The GPU walk and the oracle's segment join / triple merge / recompose
    agree relation to relation, padding included (a small case: the
    relational oracle runs on one host thread)."""
    spec, bounds = "hsd,htd,hte->hse", [0, 44, 300]
    ext = dict(h=1, s=300, t=300, d=64, e=64)
    blk = dict(h=1, s=bounds, t=bounds)
    got, want, got_rel, xs64 = run_packed_attention(ctx, spec, ext, blk, bounds, ("s", "t"), "f32")
    assert normwise_err(got, want) < BF16_OUT_TOL
    rels = [O.to_relation(x, lt, ext, blk) for x, lt in zip(xs64, ("hsd", "htd", "hte"))]
    want_rel, present = O.attention_relational(spec, rels, ext, blk, alpha=1.0 / 8.0, causal=("s", "t"),
                                               segment=("s", "t"))
    assert present.all()
    assert normwise_err(got_rel, O.round_to(want_rel, "f32")) < BF16_OUT_TOL


def test_segment_pair_on_uniform_blocks_is_block_local(ctx):
    ext = dict(h=2, s=512, t=512, d=64, e=64)
    blk = dict(h=1, s=4, t=4)
    got, want, _, _ = run_packed_attention(ctx, "hsd,htd,hte->hse", ext, blk, [0, 128, 256, 384, 512], None, "f32")
    assert normwise_err(got, want) < BF16_OUT_TOL


def test_segment_pair_rejects(ctx):
    ext = dict(h=1, s=256, t=256, d=64, e=64)
    bnd = [0, 100, 256]
    mk = lambda lt, b: jagg.relation_like(ctx, lt, ext, b, "bf16")
    q, k, v = mk("hsd", dict(s=bnd)), mk("htd", dict(t=bnd)), mk("hte", dict(t=bnd))
    spec = "hsd,htd,hte->hse"
    with pytest.raises(jagg.JaggError):  # interval s and t without a segment pair
        jagg.EinsumCall(ctx, spec, [q, k, v], dict(s=bnd, t=bnd), g="attention", agg="softmax").run()
    k2, v2 = mk("htd", dict(t=[0, 128, 256])), mk("hte", dict(t=[0, 128, 256]))
    with pytest.raises(jagg.JaggError):  # s and t cut at different places
        jagg.EinsumCall(ctx, spec, [q, k2, v2], dict(s=bnd, t=[0, 128, 256]), g="attention", agg="softmax",
                        segment=("s", "t")).run()
    with pytest.raises(jagg.JaggError):  # a segment pair outside attention
        a, b = mk("st", dict(s=2, t=2)), mk("td", dict(t=2))
        jagg.EinsumCall(ctx, "st,td->sd", [a, b], dict(s=2, t=2), segment=("s", "t")).run()
