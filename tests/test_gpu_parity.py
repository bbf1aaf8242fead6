"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bit-exact: join lists, repartition (every byte of the destination, padding
included), MAX aggregation on identical inputs.  Floating point: the normwise
error e = max|y - yhat| / max|yhat| (tests/parity_util.py) under 1e-5 for
fp32 results and 2e-2 for bf16 chains (fp32 accumulation); a single spec
with a bf16 output is held to 8e-3 (one bf16 rounding, 2^-8 relative, plus
fp32 summation error).
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as O
from tensor_relational_einsum_amd import inputs as I
from tensor_relational_einsum_amd import jagg
from tensor_relational_einsum_amd.runner import ChainRunner
from parity_util import bits, normwise_err, oracle_bits, oracle_chain, padding_mask, rel_dense, to_np

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5
BF16_OUT_TOL = 8e-3
CHAIN_TOL = 2e-2


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    c = jagg.Context(0)
    yield c
    torch.cuda.synchronize()
    c.close()


def upload(ctx, x: torch.Tensor, letters, blk):
    return jagg.from_dense(ctx, x.to("cuda"), letters, blk)


# ----------------------------------------------------------------- repartition

def check_relayout(ctx, shape, src_l, src_b, dst_l, dst_b, dtype, seed=0):
    ext = dict(zip(src_l, shape))
    g = I.streams(seed, 1)[0]
    x = I.draw(g, shape, "normal", dtype)
    src = upload(ctx, x, src_l, src_b)
    dst = jagg.relation_like(ctx, dst_l, ext, dst_b, dtype)
    dst.data.fill_(7)  # every byte must be rewritten, padding included
    jagg.repartition(ctx, src, dst)
    torch.cuda.synchronize()
    xb = bits(x)
    want_src = O.to_relation(xb, src_l, ext, src_b)
    assert np.array_equal(bits(src.data), want_src), "dense -> blocked relation differs"
    want = O.repartition(want_src, src_l, src_b, dst_l, dst_b, ext)
    got = bits(dst.data)
    assert got.shape == want.shape
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} elements differ, first at {bad[:5]}"
    # round trip back to the source blocking is the identity
    back = jagg.relation_like(ctx, src_l, ext, src_b, dtype)
    jagg.repartition(ctx, dst, back)
    torch.cuda.synchronize()
    assert np.array_equal(bits(back.data), want_src)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape,src_l,src_b,dst_l,dst_b", [
    ((64, 96), "ij", dict(i=8, j=1), "ij", dict(i=1, j=8)),
    ((32, 64, 16, 16), "abcd", dict(a=4, b=8, c=1, d=1), "acbd", dict(a=1, b=1, c=4, d=2)),
    ((30, 100, 50, 70), "abcd", dict(a=1, b=1, c=1, d=1), "abcd", dict(a=4, b=7, c=3, d=6)),
    ((30, 100, 50, 70), "abcd", dict(a=4, b=7, c=3, d=6), "abcd", dict(a=3, b=5, c=2, d=4)),
    ((7, 10, 5, 10), "abcd", dict(a=2, b=3, c=2, d=4), "dcba", dict(a=3, b=2, c=1, d=2)),
    ((6, 8, 4, 5), "abcd", dict(a=2, b=4, c=1, d=1), "acbd", dict(a=1, b=1, c=2, d=5)),
    ((1000, 167), "ij", dict(i=3, j=6), "ji", dict(i=7, j=2)),
    ((96, 300, 64, 48), "abcd", dict(a=1, b=1, c=1, d=1), "abcd", dict(a=5, b=7, c=4, d=3)),
    ((4, 256, 8, 128), "bsqd", dict(b=1, s=4, q=4, d=1), "bqsd", dict(b=1, q=1, s=4, d=1)),
    ((3,), "a", dict(a=1), "a", dict(a=3)),
])
def test_repartition_cases(ctx, shape, src_l, src_b, dst_l, dst_b, dtype):
    check_relayout(ctx, shape, src_l, src_b, dst_l, dst_b, dtype)


def test_repartition_config_8192_square(ctx):
    w = I.repartition_2d()
    x = I.generate(w)["X"]
    st = w.chain[0]
    check_relayout(ctx, tuple(x.shape), "ij", dict(i=8, j=1), st.letters, st.blockings, "bf16", seed=w.seed)


def test_repartition_config_4d(ctx):
    w = I.repartition_4d()
    st = w.chain[0]
    check_relayout(ctx, (32, 128, 64, 64), "abcd", dict(a=4, b=8, c=1, d=1), st.letters, st.blockings, "bf16",
                   seed=w.seed)


# Digit permutations whose shared innermost run is short: the LDS-transposing
# relayout (source-order reads, destination-order writes through LDS).
LDS_RELAYOUT_CASES = [
    # the 4-D config: d runs of 64 B in the destination, b and c exchanged
    ((32, 128, 64, 64), "abcd", dict(a=4, b=8, c=1, d=1), "acbd", dict(a=1, b=1, c=4, d=2), "bf16"),
    # head-major relayout of a projection output (8 x 2048 tokens, 16 heads of 128)
    ((8, 2048, 16, 128), "bsqd", dict(b=1, s=16, q=4, d=1), "bqsd", dict(b=1, q=1, s=16, d=1), "bf16"),
    ((16, 64, 32, 32), "abcd", dict(a=2, b=4, c=1, d=1), "acbd", dict(a=1, b=1, c=2, d=1), "f32"),
    ((4, 32, 64, 8), "abcd", dict(a=1, b=2, c=1, d=1), "acbd", dict(a=1, b=1, c=2, d=1), "f32"),
]


@pytest.mark.parametrize("shape,src_l,src_b,dst_l,dst_b,dtype", LDS_RELAYOUT_CASES)
def test_repartition_lds_transpose(trace_ctx, capfd, shape, src_l, src_b, dst_l, dst_b, dtype):
    check_relayout(trace_ctx, shape, src_l, src_b, dst_l, dst_b, dtype)
    lines = [ln for ln in capfd.readouterr().err.splitlines() if f"relayout {src_l} -> {dst_l}:" in ln]
    print("\n".join(lines))
    assert lines and "lds transpose" in lines[0], "the forward relayout must take the LDS-transposing kernel"


# ----------------------------------------------------------------- join lists

JOIN_CASES = [
    ("ij,jk->ik", dict(i=256, j=512, k=256), dict(i=1, j=2, k=1), None),
    ("ij,jk->ik", dict(i=256, j=512, k=256), dict(i=2, j=2, k=1), None),
    ("ij,jk->ik", dict(i=256, j=256, k=256), dict(i=4, j=4, k=4), None),
    ("abcd,cde->abe", dict(a=96, b=300, c=64, d=48, e=1000), dict(a=5, b=7, c=4, d=3, e=6), None),
    ("bhsd,bhtd->bhst", dict(b=4, h=32, s=2048, t=2048, d=128), dict(b=1, h=1, s=16, t=16, d=1), None),
    ("bhst->bhs", dict(b=4, h=32, s=2048, t=2048), dict(b=1, h=1, s=16, t=16), None),
    ("bhst,bhs,bhs->bhst", dict(b=4, h=32, s=2048, t=2048), dict(b=1, h=1, s=16, t=16), None),
    ("bhst,bhtd->bhsd", dict(b=4, h=32, s=2048, t=2048, d=128), dict(b=1, h=1, s=16, t=16, d=1), None),
    ("bsh,hqd->bsqd", dict(b=4, s=2048, h=4096, q=32, d=128), dict(b=1, s=16, h=4, q=4, d=1), None),
    ("bqsd,bqtd->bqst", dict(b=4, q=32, s=2048, t=2048, d=128), dict(b=1, q=1, s=16, t=16, d=1), ("s", "t")),
    ("bqst->bqs", dict(b=4, q=32, s=2048, t=2048), dict(b=1, q=1, s=16, t=16), ("s", "t")),
    ("bqst,bqtd->bqsd", dict(b=4, q=32, s=2048, t=2048, d=128), dict(b=1, q=1, s=16, t=16, d=1), ("s", "t")),
    ("sd,td->st", dict(s=100, t=100, d=8), dict(s=7, t=7, d=2), ("s", "t")),
]


@pytest.mark.parametrize("spec,ext,blk,causal", JOIN_CASES)
def test_join_list_bit_exact(ctx, spec, ext, blk, causal):
    lst, cnt = jagg.join_list(ctx, spec, ext, blk, causal)
    torch.cuda.synchronize()
    lst, cnt = lst.cpu().numpy(), cnt.cpu().numpy()
    got = np.concatenate([lst[k, :cnt[k]] for k in range(lst.shape[0])]) if lst.size else lst.reshape(0, 1)
    want = O.join_list(spec, ext, blk, causal)
    assert got.shape == want.shape
    assert np.array_equal(got.astype(np.int64), want)
    for k in range(lst.shape[0]):  # unused slots are -1
        assert np.all(lst[k, cnt[k]:] == -1)


# ----------------------------------------------------------------- single specs

def run_spec_case(ctx, spec, ext, blk, g="mul", agg="sum", in_dtypes=None, out_dtype="f32", alpha=1.0, beta=0.0,
                  eps=0.0, causal=None, seed=1, positive=()):
    """Runs one spec on seeded inputs and returns (gpu dense, oracle dense,
    gpu out relation, output letters)."""
    ins, out = spec.split("->")
    ins = ins.split(",")
    in_dtypes = in_dtypes or ["f32"] * len(ins)
    gens = I.streams(seed, len(ins))
    xs = []
    for j, (lt, gen, dt) in enumerate(zip(ins, gens, in_dtypes)):
        if j in positive:
            x = I.draw(gen, [ext[c] for c in lt], "uniform", dt, 1.0)
            x = (x.float().abs() + 0.5).to(x.dtype)
        else:
            x = I.draw(gen, [ext[c] for c in lt], "normal", dt)
        xs.append(x)
    rels = [upload(ctx, x, lt, blk) for x, lt in zip(xs, ins)]
    call = jagg.EinsumCall(ctx, spec, rels, blk, g=g, agg=agg, out_dtype=out_dtype, alpha=alpha, beta=beta, eps=eps,
                           causal=causal)
    call.out.data.fill_(3)
    call.run()
    torch.cuda.synchronize()
    got_rel = to_np(call.out.data)
    want = O.dense(spec, [to_np(x) for x in xs], ext, g=g, agg=agg, alpha=alpha, beta=beta, eps=eps, causal=causal)
    want = O.round_to(want, out_dtype)
    got = O.from_relation(got_rel, out, ext, blk)
    pad = padding_mask(out, ext, blk)
    return got, want, got_rel, pad, call


CONTRACT_CASES = [
    # spec, extents, blockings, input dtypes, out dtype
    ("ij,jk->ik", dict(i=256, j=256, k=256), dict(i=4, j=4, k=4), "f32", "f32"),
    ("ij,jk->ik", dict(i=200, j=130, k=70), dict(i=3, j=2, k=2), "f32", "f32"),
    ("abcd,cde->abe", dict(a=13, b=31, c=16, d=12, e=100), dict(a=5, b=7, c=4, d=3, e=6), "f32", "f32"),
    ("ij,jk->ik", dict(i=256, j=256, k=256), dict(i=2, j=4, k=2), "bf16", "f32"),
    ("ij,kj->ik", dict(i=192, j=256, k=160), dict(i=2, j=2, k=1), "bf16", "f32"),
    ("ji,jk->ik", dict(i=192, j=128, k=160), dict(i=1, j=2, k=1), "bf16", "f32"),
    ("ji,kj->ik", dict(i=96, j=64, k=80), dict(i=1, j=2, k=1), "f32", "f32"),
    ("ij,jk->ki", dict(i=96, j=64, k=80), dict(i=2, j=2, k=1), "f32", "f32"),
    ("bhsd,bhtd->bhst", dict(b=2, h=3, s=256, t=256, d=128), dict(b=1, h=1, s=2, t=2, d=1), "bf16", "f32"),
    ("bhst,bhtd->bhsd", dict(b=2, h=3, s=256, t=256, d=128), dict(b=1, h=1, s=2, t=2, d=1), "bf16", "f32"),
    ("bsh,hqd->bsqd", dict(b=2, s=256, h=512, q=4, d=128), dict(b=1, s=2, h=4, q=2, d=1), "bf16", "bf16"),
    ("bsf,fh->bsh", dict(b=2, s=128, f=688, h=256), dict(b=1, s=1, f=8, h=2), "bf16", "f32"),
    # N = 167 per block: 128x64 tiles (three 64-wide column tiles, the last ragged)
    ("ij,jk->ik", dict(i=300, j=96, k=334), dict(i=2, j=3, k=2), "f32", "f32"),
    ("ij,kj->ik", dict(i=300, j=96, k=334), dict(i=2, j=3, k=2), "bf16", "bf16"),
    ("abcd,cde->abe", dict(a=20, b=43, c=16, d=32, e=334), dict(a=1, b=1, c=1, d=2, e=2), "f32", "f32"),
]


@pytest.mark.parametrize("spec,ext,blk,idt,odt", CONTRACT_CASES)
def test_contraction_parity(ctx, spec, ext, blk, idt, odt):
    n_in = len(spec.split("->")[0].split(","))
    got, want, got_rel, pad, _ = run_spec_case(ctx, spec, ext, blk, in_dtypes=[idt] * n_in, out_dtype=odt)
    tol = F32_TOL if odt == "f32" else BF16_OUT_TOL
    err = normwise_err(got, want)
    assert err < tol, f"normwise error {err:.3e}"
    assert np.all(got_rel[pad] == 0.0), "output padding must be +0"


# The LDS-pipelined 256x256 kernel: at least 256 such tiles, 16-byte vectors,
# bf16 operands.  Blocks of 264 rows (one full tile and a ragged 8-row tail),
# two joined tuples per output key of 104 K values each (three full K-steps of
# 32 and a tail of 8), every operand orientation.
LDS_PIPELINE_CASES = [
    # spec, extents, blockings, out dtype, causal
    ("ij,jk->ik", dict(i=2112, j=208, k=2112), dict(i=8, j=2, k=8), "f32", None),
    ("ij,kj->ik", dict(i=2112, j=208, k=2112), dict(i=8, j=2, k=8), "bf16", None),
    ("ji,jk->ik", dict(i=2112, j=208, k=2112), dict(i=8, j=2, k=8), "f32", None),
    ("ji,kj->ik", dict(i=2112, j=208, k=2112), dict(i=8, j=2, k=8), "f32", None),
    # one long K walk per key (K = 528: 16 full steps and a tail of 16)
    ("ij,jk->ik", dict(i=2112, j=528, k=2112), dict(i=8, j=1, k=8), "bf16", None),
    # every step of the walk is a joined tuple of its own (32-wide K blocks),
    # and a K tail inside every step (24-wide K blocks)
    ("ij,jk->ik", dict(i=2112, j=256, k=2112), dict(i=8, j=8, k=8), "bf16", None),
    ("ji,kj->ik", dict(i=2112, j=192, k=2112), dict(i=8, j=8, k=8), "f32", None),
    # causal pair in the output (mask applied in the epilogue)
    ("bhsd,bhtd->bhst", dict(b=2, h=4, s=1056, t=1056, d=128), dict(b=1, h=1, s=4, t=4, d=1), "f32", ("s", "t")),
]


@pytest.mark.parametrize("spec,ext,blk,odt,causal", LDS_PIPELINE_CASES)
def test_contraction_lds_pipeline(trace_ctx, capfd, spec, ext, blk, odt, causal):
    n_in = len(spec.split("->")[0].split(","))
    got, want, got_rel, pad, _ = run_spec_case(trace_ctx, spec, ext, blk, in_dtypes=["bf16"] * n_in, out_dtype=odt,
                                               causal=causal, alpha=0.5 if causal else 1.0)
    assert "lds pipeline" in capfd.readouterr().err, "the case must run the LDS-pipelined kernel"
    if causal is not None:
        # tuples above the block diagonal are absent from the output relation
        # and never written; compare the present ones
        s_, t_ = causal
        out = spec.split("->")[1]
        e = -(-ext[s_] // blk[s_])
        idx = np.indices(got.shape)
        mask = (idx[out.index(t_)] // e) <= (idx[out.index(s_)] // e)
        got, want = np.where(mask, got, 0.0), np.where(mask, want, 0.0)
        kidx = np.indices([blk[c] for c in out]).reshape(len(out), -1)
        present = kidx[out.index(t_)] <= kidx[out.index(s_)]
        pad = (pad.reshape(present.size, -1) & present[:, None]).reshape(-1)
    tol = F32_TOL if odt == "f32" else BF16_OUT_TOL
    err = normwise_err(got, want)
    assert err < tol, f"normwise error {err:.3e}"
    assert np.all(got_rel[pad] == 0.0), "output padding must be +0"


# score-shaped specs whose walk is one or two K-steps with an fp32 output:
# the one-stage kernel (two stages and the LDS epilogue for a bf16 output)
SHORT_WALK_CASES = [
    ("bhsd,bhtd->bhst", dict(b=2, h=3, s=256, t=256, d=128), dict(b=1, h=1, s=2, t=2, d=1), "f32", "one stage"),
    ("bhsd,bhtd->bhst", dict(b=1, h=2, s=200, t=328, d=128), dict(b=1, h=1, s=2, t=3, d=1), "f32", "one stage"),
    ("bhsd,bhtd->bhst", dict(b=1, h=2, s=200, t=328, d=64), dict(b=1, h=1, s=2, t=3, d=1), "f32", "one stage"),
    ("bhsd,bhtd->bhst", dict(b=2, h=3, s=256, t=256, d=128), dict(b=1, h=1, s=2, t=2, d=1), "bf16", "128x128"),
]


@pytest.mark.parametrize("spec,ext,blk,odt,kernel", SHORT_WALK_CASES)
def test_contraction_short_walk(trace_ctx, capfd, spec, ext, blk, odt, kernel):
    got, want, got_rel, pad, _ = run_spec_case(trace_ctx, spec, ext, blk, in_dtypes=["bf16", "bf16"], out_dtype=odt)
    err_lines = [ln for ln in capfd.readouterr().err.splitlines() if ": contract " in ln]
    assert err_lines and kernel in err_lines[-1], err_lines
    if kernel == "128x128":
        assert "one stage" not in err_lines[-1]
    tol = F32_TOL if odt == "f32" else BF16_OUT_TOL
    err = normwise_err(got, want)
    assert err < tol, f"normwise error {err:.3e}"
    assert np.all(got_rel[pad] == 0.0), "output padding must be +0"


EW_CASES = [
    # spec, g, agg, extents, blockings, in dtypes, out dtype, positive inputs, causal
    ("bhst->bhs", "ident", "max", dict(b=2, h=3, s=40, t=300), dict(b=1, h=1, s=3, t=4), ["f32"], "f32", (), None),
    ("bhst,bhs->bhs", "exp_sub", "sum", dict(b=2, h=3, s=40, t=300), dict(b=1, h=1, s=3, t=4), ["f32", "f32"], "f32",
     (), None),
    ("bhst,bhs,bhs->bhst", "exp_sub_div", "none", dict(b=2, h=3, s=40, t=300), dict(b=1, h=1, s=3, t=4),
     ["f32", "f32", "f32"], "bf16", (2,), None),
    ("bsh->bs", "square", "sum", dict(b=2, s=50, h=1000), dict(b=1, s=3, h=4), ["f32"], "f32", (), None),
    ("bsh,bs,h->bsh", "rms_scale", "none", dict(b=2, s=50, h=1000), dict(b=1, s=3, h=4), ["f32", "f32", "bf16"],
     "bf16", (1,), None),
    ("bsf,bsf->bsf", "silu_mul", "none", dict(b=2, s=50, f=688), dict(b=1, s=3, f=8), ["f32", "f32"], "bf16", (),
     None),
    ("bsh,bsh->bsh", "add", "none", dict(b=2, s=50, h=1000), dict(b=1, s=3, h=4), ["f32", "f32"], "f32", (), None),
    ("ijk->ik", "ident", "sum", dict(i=30, j=70, k=50), dict(i=2, j=3, k=2), ["f32"], "f32", (), None),
    ("ij,j->i", "mul", "sum", dict(i=300, j=1000), dict(i=3, j=4), ["f32", "f32"], "f32", (), None),
    ("qst->qs", "ident", "max", dict(q=3, s=200, t=200), dict(q=1, s=4, t=4), ["f32"], "f32", (), ("s", "t")),
    ("qst,qs->qs", "exp_sub", "sum", dict(q=3, s=200, t=200), dict(q=1, s=4, t=4), ["f32", "f32"], "f32", (),
     ("s", "t")),
    ("qst,qs,qs->qst", "exp_sub_div", "none", dict(q=3, s=200, t=200), dict(q=1, s=4, t=4), ["f32", "f32", "f32"],
     "bf16", (2,), ("s", "t")),
]


@pytest.mark.parametrize("spec,g,agg,ext,blk,idts,odt,pos,causal", EW_CASES)
def test_map_reduce_parity(ctx, spec, g, agg, ext, blk, idts, odt, pos, causal):
    kw = dict(beta=1.0 / ext.get("h", 1), eps=1e-6) if g == "rms_scale" else {}
    got, want, got_rel, pad, call = run_spec_case(ctx, spec, ext, blk, g=g, agg=agg, in_dtypes=idts, out_dtype=odt,
                                                  positive=pos, causal=causal, **kw)
    present = call.out.data  # noqa: F841
    if causal is not None and agg == "none":
        # tuples above the block diagonal are absent from the output relation
        s, t = causal
        out = spec.split("->")[1]
        e = -(-ext[s] // blk[s])
        mask = np.zeros(got.shape, dtype=bool)
        idx = np.indices(got.shape)
        mask = (idx[out.index(t)] // e) <= (idx[out.index(s)] // e)
        got = np.where(mask, got, 0.0)
        want = np.where(mask, want, 0.0)
    if agg == "max":
        assert np.array_equal(got, want), "MAX must be bit-exact"
    else:
        tol = F32_TOL if odt == "f32" else BF16_OUT_TOL
        err = normwise_err(got, want)
        assert err < tol, f"normwise error {err:.3e}"
    if causal is None:
        assert np.all(got_rel[pad] == 0.0), "output padding must be +0"


# Row-compatible, unpadded-row operands take the flat-stream kernels; each
# case names the path it must take (read back through JAGG_TRACE).
FLAT_CASES = [
    # spec, g, agg, extents, blockings, in dtypes, out dtype, positive inputs, causal, path
    ("bhst->bhs", "ident", "max", dict(b=2, h=3, s=48, t=256), dict(b=1, h=1, s=3, t=2), ["f32"], "f32", (), None,
     "flat reduce"),
    ("bhst->bhs", "ident", "max", dict(b=2, h=3, s=48, t=290), dict(b=1, h=1, s=3, t=4), ["f32"], "f32", (), None,
     "flat reduce"),
    ("bhst,bhs->bhs", "exp_sub", "sum", dict(b=2, h=3, s=48, t=256), dict(b=1, h=1, s=3, t=2), ["f32", "f32"], "f32",
     (), None, "flat reduce"),
    ("bhst->bhs", "ident", "sum", dict(b=2, h=3, s=48, t=256), dict(b=1, h=1, s=3, t=2), ["bf16"], "f32", (), None,
     "flat reduce"),
    ("bsh->bs", "square", "sum", dict(b=2, s=48, h=1000), dict(b=1, s=3, h=4), ["f32"], "bf16", (), None,
     "flat reduce"),
    ("ij,j->i", "mul", "sum", dict(i=256, j=1024), dict(i=2, j=4), ["f32", "bf16"], "f32", (), None, "flat reduce"),
    # a 1000-byte 'j' block is not 16-byte aligned: the general row reduce
    ("ij,j->i", "mul", "sum", dict(i=256, j=1000), dict(i=2, j=4), ["bf16", "f32"], "f32", (), None, "reduce rows"),
    ("ij,j->i", "mul", "sum", dict(i=256, j=1000), dict(i=2, j=5), ["bf16", "f32"], "f32", (), None, "flat reduce"),
    ("bhst,bhs,bhs->bhst", "exp_sub_div", "none", dict(b=2, h=3, s=48, t=300), dict(b=1, h=1, s=3, t=19),
     ["f32", "f32", "f32"], "bf16", (2,), None, "flat map"),
    ("bsh,bs,h->bsh", "rms_scale", "none", dict(b=2, s=48, h=1024), dict(b=1, s=3, h=4), ["f32", "f32", "bf16"],
     "bf16", (1,), None, "flat map"),
    ("bsf,bsf->bsf", "silu_mul", "none", dict(b=2, s=48, f=704), dict(b=1, s=3, f=8), ["bf16", "bf16"], "f32", (),
     None, "flat map"),
    ("bsh,bsh,bsh->bsh", "add", "none", dict(b=2, s=48, h=1000), dict(b=1, s=3, h=5), ["f32", "f32", "f32"], "f32",
     (), None, "flat map"),
    ("bsh,bs->bsh", "mul", "none", dict(b=3, s=40, h=64), dict(b=1, s=1, h=1), ["f32", "bf16"], "f32", (), None,
     "flat map"),
    ("qst->qs", "ident", "max", dict(q=3, s=256, t=256), dict(q=1, s=4, t=4), ["f32"], "f32", (), ("s", "t"),
     "flat reduce"),
    ("qst,qs->qs", "exp_sub", "sum", dict(q=3, s=256, t=256), dict(q=1, s=4, t=4), ["f32", "f32"], "f32", (),
     ("s", "t"), "flat reduce"),
    ("qst,qs,qs->qst", "exp_sub_div", "none", dict(q=3, s=256, t=256), dict(q=1, s=4, t=4), ["f32", "f32", "f32"],
     "bf16", (2,), ("s", "t"), "flat map"),
]


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


def check_ew_case(got, want, got_rel, pad, spec, ext, blk, agg, odt, causal):
    if causal is not None and agg == "none":
        # tuples above the block diagonal are absent from the output relation
        s, t = causal
        out = spec.split("->")[1]
        e = -(-ext[s] // blk[s])
        idx = np.indices(got.shape)
        mask = (idx[out.index(t)] // e) <= (idx[out.index(s)] // e)
        got = np.where(mask, got, 0.0)
        want = np.where(mask, want, 0.0)
    if agg == "max":
        assert np.array_equal(got, want), "MAX must be bit-exact"
    else:
        tol = F32_TOL if odt == "f32" else BF16_OUT_TOL
        err = normwise_err(got, want)
        assert err < tol, f"normwise error {err:.3e}"
    if causal is None:
        assert np.all(got_rel[pad] == 0.0), "output padding must be +0"


@pytest.mark.parametrize("spec,g,agg,ext,blk,idts,odt,pos,causal,path", FLAT_CASES)
def test_flat_stream_parity(trace_ctx, capfd, spec, g, agg, ext, blk, idts, odt, pos, causal, path):
    kw = dict(beta=1.0 / ext.get("h", 1), eps=1e-6) if g == "rms_scale" else {}
    capfd.readouterr()
    got, want, got_rel, pad, _ = run_spec_case(trace_ctx, spec, ext, blk, g=g, agg=agg, in_dtypes=idts,
                                               out_dtype=odt, positive=pos, causal=causal, **kw)
    err_text = capfd.readouterr().err
    assert f"{spec}: {path}," in err_text, f"expected the {path} kernel, trace says: {err_text.strip()}"
    check_ew_case(got, want, got_rel, pad, spec, ext, blk, agg, odt, causal)


def test_bf16_rounding_bit_exact(trace_ctx):
    """f32 -> bf16 through a map: round to nearest, ties to even, on values
    chosen to hit every case (ties both ways, subnormals, the overflow edge,
    signed zeros), compared bit for bit with the oracle's rounding."""
    specials = np.array([
        1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -(1.0 + 2.0 ** -8), 0.0, -0.0,
        2.0 ** -126, 2.0 ** -130, 2.0 ** -133, 3 * 2.0 ** -134, 2.0 ** -149, -(2.0 ** -140),
        3.3895313892515355e38, 3.3961775292304e38, 3.4028234663852886e38, -3.3961775292304e38,
        65504.0, 1.00390625, 1.01171875, 123456.789, -0.0078125,
    ], dtype=np.float64).astype(np.float32)
    g = I.streams(5, 1)[0]
    rest = I.draw(g, [4096 - specials.size], "normal", "f32").numpy()
    x = np.concatenate([specials, rest]).reshape(32, 128)
    xt = torch.from_numpy(x.copy())
    ext = dict(i=32, j=128)
    blk = dict(i=2, j=1)
    src = upload(trace_ctx, xt, "ij", blk)
    call = jagg.EinsumCall(trace_ctx, "ij->ij", [src], blk, g="ident", agg="none", out_dtype="bf16")
    call.run()
    torch.cuda.synchronize()
    got = bits(call.out.data)
    want = oracle_bits(O.to_relation(O.round_to(x.astype(np.float64), "bf16"), "ij", ext, blk), "bf16")
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} values round differently, first at {bad[:5]}"


# ----------------------------------------------------------------- chains

def test_attention_chain_small(ctx):
    w = I.attention_chain(b=1, h=2, s=256, d=64, nb=4)
    dense = I.generate(w)
    run = ChainRunner(ctx, w, dense)
    run.run()
    torch.cuda.synchronize()
    want = oracle_chain(w, dense)
    for name in ["S", "M", "L", "P", "O"]:
        got = rel_dense(run.rel[name], w.extents)
        err = normwise_err(got, want[name])
        tol = CHAIN_TOL if name in ("P", "O") else 1e-4
        assert err < tol, f"{name}: normwise error {err:.3e}"
    # MAX is exact on the GPU's own scores
    S = rel_dense(run.rel["S"], w.extents)
    M = rel_dense(run.rel["M"], w.extents)
    assert np.array_equal(M, S.max(axis=-1))
    P = rel_dense(run.rel["P"], w.extents)
    assert np.allclose(P.sum(-1), 1.0, atol=2e-2)


def test_matmul_config_256(ctx):
    w = I.matmul_256()
    dense = I.generate(w)
    run = ChainRunner(ctx, w, dense)
    run.run()
    torch.cuda.synchronize()
    want = oracle_chain(w, dense)
    got = rel_dense(run.rel["C"], w.extents)
    err = normwise_err(got, want["C"])
    assert err < F32_TOL, f"normwise error {err:.3e}"


def test_multi_index_config_sampled(ctx):
    """'abcd,cde->abe' at full size, checked on sampled outputs."""
    w = I.multi_index()
    dense = I.generate(w)
    run = ChainRunner(ctx, w, dense)
    run.run()
    torch.cuda.synchronize()
    st = w.chain[0]
    got = rel_dense(run.rel["C"], w.extents)
    rng = np.random.default_rng(0)
    idx = rng.integers(0, got.size, size=3000)
    # include the ragged tail corner
    idx = np.concatenate([idx, [got.size - 1]])
    want = O.round_to(O.dense(st.spec, [to_np(dense["A"]), to_np(dense["B"])], w.extents, sample=idx), "f32")
    err = normwise_err(got.reshape(-1)[idx], want)
    assert err < F32_TOL, f"normwise error {err:.3e}"
    blk = st.blockings
    pad = padding_mask("abe", w.extents, blk)
    assert np.all(to_np(run.rel["C"].data)[pad] == 0.0)


def test_attention_config_sampled_rows(ctx):
    """The full-size unfused attention chain; every stage checked on sampled
    (b, h, s) rows against the oracle fed the GPU's stored inputs, and the
    final output against the oracle chain on those rows."""
    w = I.attention_chain()
    dense = I.generate(w)
    run = ChainRunner(ctx, w, dense)
    run.run()
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    B, H, S, T, D = (w.extents[c] for c in "bhstd")
    rows = [(int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(S))) for _ in range(24)]
    rows.append((B - 1, H - 1, S - 1))
    Q, K, V = (to_np(dense[n]) for n in "QKV")
    Sg = to_np(jagg.to_dense(ctx, run.rel["S"]))
    Mg = to_np(jagg.to_dense(ctx, run.rel["M"]))
    Lg = to_np(jagg.to_dense(ctx, run.rel["L"]))
    Pg = to_np(jagg.to_dense(ctx, run.rel["P"]))
    Og = to_np(jagg.to_dense(ctx, run.rel["O"]))
    for b, h, s in rows:
        ext1 = dict(s=1, t=T, d=D)
        s_row = O.round_to(O.dense("sd,td->st", [Q[b, h, s:s + 1], K[b, h]], ext1), "f32")
        assert normwise_err(Sg[b, h, s], s_row[0]) < F32_TOL
        srow = Sg[b, h, s:s + 1]
        m = O.dense("st->s", [srow], dict(s=1, t=T), g="ident", agg="max")
        assert m[0] == Mg[b, h, s]
        l = O.round_to(O.dense("st,s->s", [srow, Mg[b, h, s:s + 1]], dict(s=1, t=T), g="exp_sub"), "f32")
        assert normwise_err(Lg[b, h, s:s + 1], l) < F32_TOL
        p = O.round_to(O.dense("st,s,s->st", [srow, Mg[b, h, s:s + 1], Lg[b, h, s:s + 1]], dict(s=1, t=T),
                               g="exp_sub_div", agg="none"), "bf16")
        assert normwise_err(Pg[b, h, s], p[0]) < BF16_OUT_TOL
        o = O.round_to(O.dense("st,td->sd", [Pg[b, h, s:s + 1], V[b, h]], dict(s=1, t=T, d=D)), "f32")
        assert normwise_err(Og[b, h, s], o[0]) < F32_TOL
        # the chain from the original inputs, with the same cast points
        sc = O.round_to(O.dense("sd,td->st", [Q[b, h, s:s + 1], K[b, h]], ext1), "f32")
        mc = O.dense("st->s", [sc], dict(s=1, t=T), g="ident", agg="max")
        lc = O.round_to(O.dense("st,s->s", [sc, mc], dict(s=1, t=T), g="exp_sub"), "f32")
        pc = O.round_to(O.dense("st,s,s->st", [sc, mc, lc], dict(s=1, t=T), g="exp_sub_div", agg="none"), "bf16")
        oc = O.dense("st,td->sd", [pc, V[b, h]], dict(s=1, t=T, d=D))
        assert normwise_err(Og[b, h, s], oc[0]) < CHAIN_TOL


def sampled_spec_check(ctx, run, w, n_samples=400, seed=2):
    """Every spec of a chain checked on sampled outputs against the oracle
    fed the GPU's own stored inputs; every relayout checked bit-exactly."""
    rng = np.random.default_rng(seed)
    dense_cache = {}

    def dense_of(name):
        if name not in dense_cache:
            dense_cache[name] = jagg.to_dense(ctx, run.rel[name]).to("cpu")
        return dense_cache[name]

    for st in w.chain:
        if isinstance(st, I.Relayout):
            src, dst = run.rel[st.src], run.rel[st.out]
            ext = dict(zip(src.letters, src.extents))
            want = O.repartition(bits(src.data), src.letters, src.blocking(), dst.letters, dst.blocking(), ext)
            assert np.array_equal(bits(dst.data), want), f"relayout {st.out}"
            continue
        out_l = st.spec.split("->")[1]
        got = dense_of(st.out)
        idx = rng.integers(0, got.numel(), size=n_samples)
        idx = np.concatenate([idx, [got.numel() - 1]])
        xs = [to_np(dense_of(n)) for n in st.ins]
        if st.g == "attention":
            want = O.attention_dense(st.spec, xs, w.extents, alpha=st.alpha, causal=st.causal, sample=idx)
        elif st.g in ("mul_plus", "swiglu"):
            want = O.dense_recompose(st.spec, st.g, xs, w.extents, alpha=st.alpha, sample=idx)
        else:
            want = O.dense(st.spec, xs, w.extents, g=st.g, agg=st.agg, alpha=st.alpha, beta=st.beta, eps=st.eps,
                           causal=st.causal, sample=idx)
        want = O.round_to(want, st.out_dtype)
        g = to_np(got).reshape(-1)[idx]
        if st.causal is not None and st.agg == "none" or (st.causal is not None and st.g == "mul" and
                                                          st.causal[1] in out_l):
            # elements in absent tuples (t-block after s-block) are not stored
            s, t = st.causal
            shp = [w.extents[c] for c in out_l]
            coords = np.unravel_index(idx, shp)
            e = -(-w.extents[s] // st.blockings[s])
            keep = coords[out_l.index(t)] // e <= coords[out_l.index(s)] // e
            g, want = g[keep], want[keep]
        if st.agg == "max":
            assert np.array_equal(g, want), f"{st.out}: MAX differs"
        else:
            # fused attention: probabilities enter P V rounded to bf16 (see test_gpu_attention)
            tol = F32_TOL if st.out_dtype == "f32" and st.g != "attention" else BF16_OUT_TOL
            err = normwise_err(g, want)
            assert err < tol, f"{st.out} ({st.spec}): normwise error {err:.3e}"


def test_llama_block_small(ctx):
    w = I.llama_block(b=1, s=256, hid=512, heads=4, d=128, ffn=1376, s_blk=4, h_blk=4, q_blk=2, f_blk=8)
    dense = I.generate(w)
    run = ChainRunner(ctx, w, dense)
    run.run()
    torch.cuda.synchronize()
    want = oracle_chain(w, dense)
    for name in ["ss1", "r1", "Qp", "Kp", "Vp", "S", "M", "L", "P", "Oh", "A", "x2", "r2", "G", "U", "H", "D", "y"]:
        got = rel_dense(run.rel[name], w.extents)
        ref = want[name]
        if name in ("S", "P"):
            mask = np.tril(np.ones((w.extents["s"], w.extents["t"]), dtype=bool))
            got, ref = got[..., mask], ref[..., mask]
        err = normwise_err(got, ref)
        assert err < CHAIN_TOL, f"{name}: normwise error {err:.3e}"
    sampled_spec_check(ctx, run, w, n_samples=200)


def test_llama_block_small_fused_attention(ctx):
    w = I.llama_block(b=1, s=256, hid=512, heads=4, d=128, ffn=1376, s_blk=2, h_blk=4, q_blk=2, f_blk=8,
                      fused_attention=True)
    dense = I.generate(w)
    run = ChainRunner(ctx, w, dense)
    run.run()
    torch.cuda.synchronize()
    want = oracle_chain(w, dense)
    for name in ["ss1", "r1", "Qp", "Kp", "Vp", "O", "A", "x2", "r2", "G", "U", "H", "D", "y"]:
        err = normwise_err(rel_dense(run.rel[name], w.extents), want[name])
        assert err < CHAIN_TOL, f"{name}: normwise error {err:.3e}"
    sampled_spec_check(ctx, run, w, n_samples=200)


@pytest.mark.parametrize("epi", [True, False])
def test_llama_block_config_sampled_fused_attention(ctx, epi):
    """The full LLaMA-7B-shaped block with fused attention (and, as bench.py
    times it, fused residual / SwiGLU recompose maps): every spec checked on
    sampled outputs."""
    w = I.llama_block(fused_attention=True, fused_epilogues=epi)
    dense = I.generate(w)
    run = ChainRunner(ctx, w, dense)
    run.run()
    torch.cuda.synchronize()
    sampled_spec_check(ctx, run, w, n_samples=300)


def test_llama_block_config_sampled(ctx):
    """The full LLaMA-7B-shaped block (4 x 2048 tokens), each spec checked on
    sampled outputs, each relayout bit-exactly."""
    w = I.llama_block()
    dense = I.generate(w)
    run = ChainRunner(ctx, w, dense)
    run.run()
    torch.cuda.synchronize()
    sampled_spec_check(ctx, run, w, n_samples=300)


def test_multi_index_and_attention_configs_per_spec(ctx):
    for w in (I.multi_index(), I.attention_chain(), I.attention_chain(fused=True)):
        dense = I.generate(w)
        run = ChainRunner(ctx, w, dense)
        run.run()
        torch.cuda.synchronize()
        sampled_spec_check(ctx, run, w, n_samples=300)
        del run
        torch.cuda.empty_cache()
