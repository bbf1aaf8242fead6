"""Pins for the CPU oracle: checks against things other than itself.

Each test ties the oracle to a library routine (numpy / torch in float64), a
worked example printed by the pages (fixtures under tests/golden/), a closed
form, or an invariant of the method -- chosen so that a dropped term, a wrong
sign or index, or a transposed operand fails one of them.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(rng, shape, lo=-1.0, hi=1.0):
    return rng.uniform(lo, hi, size=shape)


# --------------------------------------------------------------------------
# Dense form against library routines
# --------------------------------------------------------------------------

@pytest.mark.parametrize("spec,ext", [
    ("ij,jk->ik", dict(i=5, j=7, k=3)),
    ("ij,jk->ki", dict(i=5, j=7, k=3)),          # transposed output
    ("abcd,cde->abe", dict(a=3, b=4, c=2, d=5, e=6)),
    ("bhsd,bhtd->bhst", dict(b=2, h=3, s=4, t=5, d=6)),
    ("bhst,bhtd->bhsd", dict(b=2, h=3, s=4, t=5, d=6)),
    ("bsh,hqd->bsqd", dict(b=2, s=3, h=4, q=2, d=3)),
    ("ij,j->i", dict(i=6, j=9)),                  # matrix-vector
    ("ij,ij->ij", dict(i=4, j=5)),                # Hadamard (map)
    ("ijk->ik", dict(i=3, j=4, k=5)),             # middle-letter reduction
])
def test_mul_sum_matches_numpy_einsum(spec, ext):
    rng = np.random.default_rng(1)
    ins, out = spec.split("->")
    xs = [rnd(rng, [ext[c] for c in lt]) for lt in ins.split(",")]
    n_in = len(xs)
    if n_in == 1:
        got = O.dense(spec, xs, ext, g="ident", agg="sum")
    elif set(out) == set("".join(ins.split(","))):
        got = O.dense(spec, xs, ext, g="mul", agg="none")
    else:
        got = O.dense(spec, xs, ext, g="mul", agg="sum")
    want = np.einsum(spec, *xs)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_alpha_scales_result():
    rng = np.random.default_rng(2)
    ext = dict(i=4, j=6, k=5)
    a, b = rnd(rng, (4, 6)), rnd(rng, (6, 5))
    got = O.dense("ij,jk->ik", [a, b], ext, alpha=0.125)
    np.testing.assert_allclose(got, 0.125 * (a @ b), rtol=1e-12)


def test_max_matches_numpy_max():
    rng = np.random.default_rng(3)
    ext = dict(b=2, h=3, s=4, t=7)
    s = rnd(rng, (2, 3, 4, 7), -5, 5)
    got = O.dense("bhst->bhs", [s], ext, g="ident", agg="max")
    assert np.array_equal(got, s.max(axis=3))
    got2 = O.dense("bhst->bht", [s], ext, g="ident", agg="max")
    assert np.array_equal(got2, s.max(axis=2))


def softmax_chain(S, ext, causal=None, spec_letters="bhst"):
    b, h, s, t = spec_letters
    m = O.dense(f"{b}{h}{s}{t}->{b}{h}{s}", [S], ext, g="ident", agg="max", causal=causal)
    l = O.dense(f"{b}{h}{s}{t},{b}{h}{s}->{b}{h}{s}", [S, m], ext, g="exp_sub", agg="sum", causal=causal)
    p = O.dense(f"{b}{h}{s}{t},{b}{h}{s},{b}{h}{s}->{b}{h}{s}{t}", [S, m, l], ext, g="exp_sub_div", agg="none",
                causal=causal)
    return m, l, p


def test_softmax_chain_matches_torch_softmax():
    rng = np.random.default_rng(4)
    ext = dict(b=2, h=2, s=5, t=9)
    S = rnd(rng, (2, 2, 5, 9), -8, 8)
    m, l, p = softmax_chain(S, ext)
    St = torch.from_numpy(S)
    np.testing.assert_allclose(p, torch.softmax(St, dim=-1).numpy(), rtol=1e-13, atol=1e-15)
    # l = sum exp(S - m) = exp(logsumexp(S) - m)
    np.testing.assert_allclose(l, np.exp(torch.logsumexp(St, dim=-1).numpy() - m), rtol=1e-13)
    assert np.allclose(p.sum(-1), 1.0, atol=1e-13)


def test_causal_softmax_matches_masked_torch_softmax():
    rng = np.random.default_rng(5)
    ext = dict(b=1, h=2, s=6, t=6)
    S = rnd(rng, (1, 2, 6, 6), -4, 4)
    m, l, p = softmax_chain(S, ext, causal=("s", "t"))
    mask = np.tril(np.ones((6, 6), dtype=bool))
    St = torch.from_numpy(np.where(mask, S, -np.inf))
    want = torch.softmax(St, dim=-1).numpy()
    np.testing.assert_allclose(p, want, rtol=1e-13, atol=1e-15)
    assert np.all(p[..., ~mask] == 0.0)


def test_causal_contraction_is_masked_matmul():
    rng = np.random.default_rng(6)
    ext = dict(b=1, q=2, s=5, t=5, d=3)
    p = rnd(rng, (1, 2, 5, 5))
    v = rnd(rng, (1, 2, 5, 3))
    got = O.dense("bqst,bqtd->bqsd", [p, v], ext, causal=("s", "t"))
    want = np.einsum("bqst,bqtd->bqsd", p * np.tril(np.ones((5, 5))), v)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_rmsnorm_matches_torch_rms_norm():
    rng = np.random.default_rng(7)
    B, S, H = 2, 3, 16
    ext = dict(b=B, s=S, h=H)
    x = rng.standard_normal((B, S, H))
    gam = 1 + 0.02 * rng.standard_normal(H)
    ss = O.dense("bsh->bs", [x], ext, g="square", agg="sum")
    r = O.dense("bsh,bs,h->bsh", [x, ss, gam], ext, g="rms_scale", agg="none", beta=1.0 / H, eps=1e-6)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (H,), weight=torch.from_numpy(gam), eps=1e-6)
    np.testing.assert_allclose(r, want.numpy(), rtol=1e-12)
    np.testing.assert_allclose(ss, (x * x).sum(-1), rtol=1e-13)


def test_silu_mul_matches_torch_silu():
    rng = np.random.default_rng(8)
    ext = dict(b=2, s=3, f=7)
    g, u = rng.standard_normal((2, 3, 7)) * 3, rng.standard_normal((2, 3, 7))
    got = O.dense("bsf,bsf->bsf", [g, u], ext, g="silu_mul", agg="none")
    want = torch.nn.functional.silu(torch.from_numpy(g)).numpy() * u
    np.testing.assert_allclose(got, want, rtol=1e-13)


def test_add_and_broadcast_mul():
    rng = np.random.default_rng(9)
    ext = dict(b=2, s=3, h=4)
    x, y, gam = rng.standard_normal((2, 3, 4)), rng.standard_normal((2, 3, 4)), rng.standard_normal(4)
    np.testing.assert_allclose(O.dense("bsh,bsh->bsh", [x, y], ext, g="add", agg="none"), x + y, rtol=1e-15)
    np.testing.assert_allclose(O.dense("bsh,h->bsh", [x, gam], ext, g="mul", agg="none"), x * gam, rtol=1e-15)


def test_sampled_outputs_equal_full_evaluation():
    rng = np.random.default_rng(10)
    ext = dict(a=3, b=4, c=2, d=5, e=6)
    A, B = rnd(rng, (3, 4, 2, 5)), rnd(rng, (2, 5, 6))
    full = O.dense("abcd,cde->abe", [A, B], ext)
    idx = rng.integers(0, full.size, size=17)
    part = O.dense("abcd,cde->abe", [A, B], ext, sample=idx)
    assert np.array_equal(part, full.reshape(-1)[idx])


def test_rejects_malformed_specs():
    ext = {c: 2 for c in "ijkz"}
    x = np.zeros((2, 2))
    for bad in ["ij,jk", "ij,jk->iz", "iij,jk->ik", "ij,jk->iik", "iJ,jk->ik"]:
        lhs = bad.split("->")[0].split(",")
        xs = [np.zeros([2] * len(lt)) for lt in lhs]
        with pytest.raises(O.OracleError):
            O.dense(bad, xs, ext)
    with pytest.raises(O.OracleError):  # reduced letter with no aggregation
        O.dense("ij,jk->ik", [x, x], ext, agg="none")


# --------------------------------------------------------------------------
# bfloat16 rounding against torch's CPU cast
# --------------------------------------------------------------------------

def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(11)
    x32 = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    # exact ties: bf16 value plus half an ulp, either parity
    bits = rng.integers(0x0080, 0x7F00, size=4000, dtype=np.uint32) | (rng.integers(0, 2, 4000, dtype=np.uint32) << 15)
    ties = ((bits << 16) | 0x8000).view(np.float32)
    sub = (rng.integers(1, 1 << 23, size=4000, dtype=np.uint32)).view(np.float32)  # float32 subnormals
    big = np.array([3.3895314e38, 3.39e38, -3.4e38, 1e-45, -0.0, 0.0], dtype=np.float32)
    for arr in (x32, ties, sub, big):
        want = torch.from_numpy(arr).to(torch.bfloat16).to(torch.float64).numpy()
        got = O.round_to(arr.astype(np.float64), "bf16")
        assert np.array_equal(got, want, equal_nan=True)


def test_f32_rounding_is_ieee_single():
    rng = np.random.default_rng(12)
    x = rng.standard_normal(10000) * 1e3
    assert np.array_equal(O.round_to(x, "f32"), x.astype(np.float32).astype(np.float64))


# --------------------------------------------------------------------------
# Relation geometry: tiling (Def. 3.2), padded blocks, Shardy local shapes
# --------------------------------------------------------------------------

def test_shardy_local_shapes():
    rows = [l for l in open(os.path.join(GOLDEN, "shardy_local_shapes.txt")) if l.strip() and l[0] != "#"]
    assert len(rows) == 3
    for row in rows:
        _, blocks, local = row.split("|")
        k0, k1 = map(int, blocks.split())
        l0, l1 = map(int, local.split())
        assert O.block_shape("xy", dict(x=4, y=8), dict(x=k0, y=k1)) == (l0, l1)


@pytest.mark.parametrize("n,k,e", [(96, 5, 20), (300, 7, 43), (1000, 6, 167), (64, 4, 16), (10, 10, 1)])
def test_padded_block_extent(n, k, e):
    assert O.block_shape("a", dict(a=n), dict(a=k)) == (e,)


def test_empty_tail_block_rejected():
    # 10 into 4 blocks: e = 3 covers 12 with 4 blocks, fine; 10 into 6: e = 2, 5 blocks cover 10 -> block 6 empty
    O.block_shape("a", dict(a=10), dict(a=4))
    with pytest.raises(O.OracleError):
        O.block_shape("a", dict(a=10), dict(a=6))


@pytest.mark.parametrize("shape,blk", [((7, 5), (3, 2)), ((6, 5, 5), (2, 3, 2)), ((10,), (4,)), ((4, 8), (2, 8))])
def test_relation_tiles_the_tensor(shape, blk):
    """Every element lands in exactly one block (Def. 3.2), padding holds +0,
    and the round trip to dense is the identity."""
    letters = "abc"[:len(shape)]
    ext = dict(zip(letters, shape))
    bl = dict(zip(letters, blk))
    n = int(np.prod(shape))
    ids = (np.arange(n, dtype=np.int64) + 1).reshape(shape)
    rel = O.to_relation(ids, letters, ext, bl)
    vals = rel[rel != 0]
    assert np.array_equal(np.sort(vals), np.arange(1, n + 1))
    e = O.block_shape(letters, ext, bl)
    assert rel.size == int(np.prod(blk)) * int(np.prod(e))
    assert np.count_nonzero(rel == 0) == rel.size - n
    assert np.array_equal(O.from_relation(rel, letters, ext, bl), ids)
    # the first tuple is the block [0, e) in every letter
    first = rel[: int(np.prod(e))].reshape(e)
    sl = tuple(slice(0, min(ee, s)) for ee, s in zip(e, shape))
    assert np.array_equal(first[sl], ids[sl])


# --------------------------------------------------------------------------
# Join lists: Examples 3.8 / 3.9 and the 3D-matmul accounting of Sec. 4.4
# --------------------------------------------------------------------------

def read_join_cases():
    cases, cur = {}, None
    for line in open(os.path.join(GOLDEN, "ex38_ex39_join.txt")):
        line = line.strip()
        if not line or line[0] == "#":
            continue
        if line.startswith("case"):
            parts = line.split()
            cur = {"blk": {kv.split("=")[0]: int(kv.split("=")[1]) for kv in parts[2:]}, "entries": [], "keys": []}
            cases[parts[1]] = cur
        elif line.startswith("key"):
            cur["keys"].append(list(map(int, line.split()[1:])))
        else:
            cur["entries"].append(list(map(int, line.split())))
    return cases


def test_join_list_examples_3_8_and_3_9():
    cases = read_join_cases()
    assert set(cases) == {"ex3.8", "ex3.9"}
    ext = dict(i=256, j=512, k=256)
    for name, c in cases.items():
        lst = O.join_list("ij,jk->ik", ext, c["blk"])
        assert lst.tolist() == c["entries"], name
        ie, ke = O.block_shape("ik", ext, c["blk"])
        for out_id, ilo, ihi, klo, khi, mult in c["keys"]:
            ki, kk = divmod(out_id, c["blk"]["k"])
            assert (ki * ie, min((ki + 1) * ie, 256), kk * ke, min((kk + 1) * ke, 256)) == (ilo, ihi, klo, khi)
            assert int((lst[:, 0] == out_id).sum()) == mult


@pytest.mark.parametrize("a,b,c", [(4, 4, 4), (2, 1, 4), (1, 8, 1), (2, 3, 2), (8, 1, 1)])
def test_3d_matmul_accounting(a, b, c):
    """Sec. 4.4: an a x b x c grid has abc specs, ac output types each seen b
    times; the joined inputs total (a + c) N^2 numbers and aggregation moves
    (b - 1) N^2."""
    N = 48
    ext = dict(i=N, j=N, k=N)
    blk = dict(i=a, j=b, k=c)
    lst = O.join_list("ij,jk->ik", ext, blk)
    assert lst.shape == (a * b * c, 3)
    keys, counts = np.unique(lst[:, 0], return_counts=True)
    assert len(keys) == a * c and np.all(counts == b)
    ea = O.block_shape("ij", ext, blk)
    eb = O.block_shape("jk", ext, blk)
    eo = O.block_shape("ik", ext, blk)
    gathered = len(lst) * (int(np.prod(ea)) + int(np.prod(eb)))
    aggregated = sum((m - 1) * int(np.prod(eo)) for m in counts)
    assert gathered == (a + c) * N * N
    assert aggregated == (b - 1) * N * N


def test_join_list_is_canonical_and_complete():
    ext = dict(b=3, s=10, t=10, d=4)
    blk = dict(b=1, s=3, t=4, d=2)
    lst = O.join_list("bsd,btd->bst", ext, blk)
    # every combination of block coordinates over all letters, once (Sec. 3.3)
    assert len(lst) == 1 * 3 * 4 * 2
    assert np.all(np.diff(lst[:, 0]) >= 0)
    assert len({tuple(r) for r in lst.tolist()}) == len(lst)
    # within a key, the reduced letter d advances
    for key in np.unique(lst[:, 0]):
        rows = lst[lst[:, 0] == key]
        assert rows[:, 1].tolist() == sorted(rows[:, 1].tolist())


def test_causal_join_keeps_lower_block_triangle():
    ext = dict(s=64, t=64, d=8)
    blk = dict(s=4, t=4, d=1)
    lst = O.join_list("sd,td->st", ext, blk, causal=("s", "t"))
    out = lst[:, 0]
    assert len(lst) == 10  # 4 * 5 / 2 pairs with t-block <= s-block
    assert all((o % 4) <= (o // 4) for o in out)


# --------------------------------------------------------------------------
# Relational form (Def. 3.7) equals the dense form
# --------------------------------------------------------------------------

REL_CASES = [
    ("ij,jk->ik", "mul", "sum", dict(i=9, j=10, k=7), dict(i=2, j=3, k=3), None),
    ("abcd,cde->abe", "mul", "sum", dict(a=7, b=5, c=5, d=3, e=10), dict(a=2, b=2, c=3, d=2, e=4), None),
    ("bhsd,bhtd->bhst", "mul", "sum", dict(b=2, h=1, s=7, t=6, d=5), dict(b=1, h=1, s=3, t=2, d=2), None),
    ("bhst->bhs", "ident", "max", dict(b=2, h=2, s=5, t=11), dict(b=2, h=1, s=2, t=4), None),
    ("bhst,bhs->bhs", "exp_sub", "sum", dict(b=1, h=2, s=5, t=11), dict(b=1, h=2, s=2, t=3), None),
    ("bhst,bhs,bhs->bhst", "exp_sub_div", "none", dict(b=1, h=2, s=5, t=7), dict(b=1, h=1, s=2, t=3), None),
    ("bsh->bs", "square", "sum", dict(b=2, s=5, h=13), dict(b=1, s=2, h=4), None),
    ("bsh,bs,h->bsh", "rms_scale", "none", dict(b=2, s=5, h=9), dict(b=2, s=3, h=2), None),
    ("bsf,bsf->bsf", "silu_mul", "none", dict(b=1, s=4, f=9), dict(b=1, s=2, f=5), None),
    ("bsh,bsh->bsh", "add", "none", dict(b=2, s=3, h=5), dict(b=2, s=2, h=3), None),
    ("ijk->ik", "ident", "sum", dict(i=4, j=7, k=5), dict(i=2, j=3, k=2), None),
    ("sd,td->st", "mul", "sum", dict(s=9, t=9, d=4), dict(s=3, t=3, d=2), ("s", "t")),
    ("qst->qs", "ident", "max", dict(q=2, s=9, t=9), dict(q=1, s=3, t=3), ("s", "t")),
    ("qst,qtd->qsd", "mul", "sum", dict(q=2, s=10, t=10, d=3), dict(q=2, s=4, t=4, d=1), ("s", "t")),
]


@pytest.mark.parametrize("spec,g,agg,ext,blk,causal", REL_CASES)
def test_relational_equals_dense(spec, g, agg, ext, blk, causal):
    rng = np.random.default_rng(abs(hash(spec)) % (1 << 31))
    ins, out = spec.split("->")
    ins = ins.split(",")
    xs = []
    for lt in ins:
        x = rng.uniform(-2, 2, size=[ext[c] for c in lt])
        if g == "exp_sub_div" and lt == ins[2]:
            x = rng.uniform(0.5, 3, size=[ext[c] for c in lt])
        if g == "rms_scale" and lt == ins[1]:
            x = rng.uniform(0.5, 3, size=[ext[c] for c in lt])
        xs.append(x)
    kw = dict(beta=0.1, eps=1e-3) if g == "rms_scale" else {}
    want = O.dense(spec, xs, ext, g=g, agg=agg, causal=causal, **kw)
    rels = [O.to_relation(x, lt, ext, blk) for x, lt in zip(xs, ins)]
    got_rel, present = O.relational(spec, rels, ext, blk, g=g, agg=agg, causal=causal, **kw)
    got = O.from_relation(got_rel, out, ext, blk)
    if causal is None:
        assert present.all()
    if agg == "max":
        assert np.array_equal(got, want)
    else:
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    # padding of the output relation is +0
    pad = O.to_relation(np.ones(want.shape), out, ext, blk) == 0
    assert np.all(got_rel[pad] == 0.0)


def test_relational_matmul_blocks_are_sums_over_j():
    """A matmul is a join on the inner index followed by SUM (Sec. 1): each
    output block equals the sum over j-blocks of the block products."""
    rng = np.random.default_rng(13)
    ext, blk = dict(i=8, j=12, k=6), dict(i=2, j=3, k=2)
    A, B = rng.standard_normal((8, 12)), rng.standard_normal((12, 6))
    rel, _ = O.relational("ij,jk->ik", [O.to_relation(A, "ij", ext, blk), O.to_relation(B, "jk", ext, blk)], ext, blk)
    C = O.from_relation(rel, "ik", ext, blk)
    for bi, bk in itertools.product(range(2), range(2)):
        blkC = sum(A[4 * bi:4 * bi + 4, 4 * bj:4 * bj + 4] @ B[4 * bj:4 * bj + 4, 3 * bk:3 * bk + 3] for bj in range(3))
        np.testing.assert_allclose(C[4 * bi:4 * bi + 4, 3 * bk:3 * bk + 3], blkC, rtol=1e-12)


# --------------------------------------------------------------------------
# Repartition: round trips, dense view, Example 5.4
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape,src_l,src_b,dst_l,dst_b", [
    ((16, 24), "ij", dict(i=4, j=1), "ij", dict(i=1, j=3)),
    ((6, 8, 4, 5), "abcd", dict(a=2, b=4, c=1, d=1), "acbd", dict(a=1, b=1, c=2, d=5)),
    ((7, 10, 5, 10), "abcd", dict(a=2, b=3, c=2, d=4), "dcba", dict(a=3, b=2, c=1, d=2)),
    ((30, 100, 50, 70), "abcd", dict(a=1, b=1, c=1, d=1), "abcd", dict(a=4, b=7, c=3, d=6)),
])
@pytest.mark.parametrize("dtype", [np.uint16, np.uint32])
def test_repartition_round_trip_and_dense_view(shape, src_l, src_b, dst_l, dst_b, dtype):
    rng = np.random.default_rng(14)
    ext = dict(zip(src_l, shape))
    dense = rng.integers(1, np.iinfo(dtype).max, size=shape, dtype=dtype)
    src = O.to_relation(dense, src_l, ext, src_b)
    dst = O.repartition(src, src_l, src_b, dst_l, dst_b, ext)
    back = O.repartition(dst, dst_l, dst_b, src_l, src_b, ext)
    assert np.array_equal(back, src)
    perm = [src_l.index(c) for c in dst_l]
    assert np.array_equal(O.from_relation(dst, dst_l, ext, dst_b), dense.transpose(perm))
    one = {c: 1 for c in dst_l}
    assert np.array_equal(O.repartition(dst, dst_l, dst_b, dst_l, one, ext).reshape(dense.transpose(perm).shape),
                          dense.transpose(perm))


def test_example_5_4_reblocking():
    """Example 5.4: rows blocked {0,128,256} re-blocked to {0,64,128,192,256};
    each consumer block is one atom and each producer block the union of two."""
    f = {}
    for line in open(os.path.join(GOLDEN, "ex54_overlay.txt")):
        if line.strip() and line[0] != "#":
            k, *v = line.split()
            f[k] = list(map(int, v))
    n, kp, kc = f["extent"][0], f["producer"][0], f["consumer"][0]
    ext = dict(i=n, k=8)
    rng = np.random.default_rng(15)
    dense = rng.integers(1, 60000, size=(n, 8), dtype=np.uint16)
    prod = O.to_relation(dense, "ik", ext, dict(i=kp, k=1))
    cons = O.repartition(prod, "ik", dict(i=kp, k=1), "ik", dict(i=kc, k=1), ext)
    split = f["split"]
    assert len(split) - 1 == f["atoms"][0] == kc
    blocks = cons.reshape(kc, -1, 8)
    for a in range(kc):
        assert np.array_equal(blocks[a], dense[split[a]:split[a + 1]])
    pblocks = prod.reshape(kp, -1, 8)
    per = f["per_producer_block"][0]
    for p in range(kp):
        assert np.array_equal(pblocks[p], np.concatenate(list(blocks[p * per:(p + 1) * per])))


@pytest.mark.parametrize("spec,ext", [
    ("ij,jk->ik", dict(i=7, j=13, k=5)),
    ("bsh,hqd->bsqd", dict(b=2, s=5, h=12, q=3, d=4)),
    ("bsqd,qdh->bsh", dict(b=2, s=5, h=12, q=3, d=4)),
    ("bsf,fh->bsh", dict(b=1, s=6, f=9, h=7)),
    ("abcd,cde->abe", dict(a=3, b=4, c=5, d=2, e=6)),
])
def test_blas_contraction_equals_dense_loops(spec, ext):
    """O.contract (numpy's float64 BLAS path) against O.dense's plain loops."""
    ins, _ = spec.split("->")
    gens = np.random.default_rng(7)
    xs = [gens.standard_normal([ext[c] for c in lt]) for lt in ins.split(",")]
    want = O.dense(spec, xs, ext)
    got = O.contract(spec, xs[0], xs[1], ext)
    assert got.shape == want.shape
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


def test_blas_contraction_closed_form():
    """Rank-one operands: A[i,j] = u_i v_j and B[j,k] = v_j w_k give
    C[i,k] = u_i w_k sum_j v_j^2 exactly (small integers, no rounding)."""
    u, v, w = np.arange(1, 5.0), np.array([1.0, -2.0, 3.0]), np.array([2.0, 0.0, -1.0, 5.0, 1.0])
    C = O.contract("ij,jk->ik", np.outer(u, v), np.outer(v, w), dict(i=4, j=3, k=5))
    assert np.array_equal(C, np.outer(u, w) * 14.0)


# Contractions with a recompose map (oracle_dense_recompose): the residual
# form 'mul_plus' and the gated form 'swiglu'.
RECOMPOSE_CASES = [
    ("bsqd,qdh,bsh->bsh", dict(b=2, s=5, q=3, d=4, h=6)),
    ("ij,jk,ik->ik", dict(i=7, j=9, k=5)),
]


@pytest.mark.parametrize("spec,ext", RECOMPOSE_CASES)
def test_mul_plus_matches_numpy(spec, ext):
    ins, _ = spec.split("->")
    rng = np.random.default_rng(11)
    xs = [rng.standard_normal([ext[c] for c in lt]) for lt in ins.split(",")]
    got = O.dense_recompose(spec, "mul_plus", xs, ext, alpha=0.5)
    lt = ins.split(",")
    want = 0.5 * np.einsum(f"{lt[0]},{lt[1]}->{spec.split('->')[1]}", xs[0], xs[1]) + xs[2]
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))
    # special cases: a zero addend is the plain contraction, a zero factor the addend
    zero = O.dense_recompose(spec, "mul_plus", [xs[0], xs[1], np.zeros_like(xs[2])], ext, alpha=0.5)
    assert np.array_equal(zero, O.dense(f"{lt[0]},{lt[1]}->{spec.split('->')[1]}", xs[:2], ext, alpha=0.5))
    only = O.dense_recompose(spec, "mul_plus", [xs[0], np.zeros_like(xs[1]), xs[2]], ext)
    assert np.array_equal(only, xs[2])


def test_swiglu_matches_torch():
    import torch
    spec, ext = "bsh,hf,hf->bsf", dict(b=2, s=6, h=8, f=5)
    rng = np.random.default_rng(12)
    x, wg, wu = (rng.standard_normal([ext[c] for c in lt]) for lt in ("bsh", "hf", "hf"))
    got = O.dense_recompose(spec, "swiglu", [x, wg, wu], ext)
    tx = torch.from_numpy(x)
    want = (torch.nn.functional.silu(tx @ torch.from_numpy(wg)) * (tx @ torch.from_numpy(wu))).numpy()
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))
    # silu(0) = 0: a zero gate weight gives zero
    assert np.array_equal(O.dense_recompose(spec, "swiglu", [x, np.zeros_like(wg), wu], ext), np.zeros((2, 6, 5)))
    # sampled outputs equal the full evaluation
    idx = np.array([0, 7, 33, 59])
    assert np.array_equal(O.dense_recompose(spec, "swiglu", [x, wg, wu], ext, sample=idx), got.reshape(-1)[idx])


def test_recompose_rejects_malformed():
    ext = dict(i=3, j=4, k=5)
    x = [np.ones((3, 4)), np.ones((4, 5)), np.ones((4, 5))]
    with pytest.raises(O.OracleError):  # the addend holds a reduced letter
        O.dense_recompose("ij,jk,jk->ik", "mul_plus", x, ext)
    with pytest.raises(O.OracleError):  # the two sums over different letters
        O.dense_recompose("ij,jk,ik->ik", "swiglu", [x[0], x[1], np.ones((3, 5))], ext)


@pytest.mark.parametrize("kind,spec,ext,blk", [
    ("mul_plus", "bsqd,qdh,bsh->bsh", dict(b=2, s=7, q=3, d=4, h=10), dict(b=1, s=3, q=2, d=1, h=4)),
    ("swiglu", "bsh,hf,hf->bsf", dict(b=1, s=9, h=10, f=7), dict(b=1, s=2, h=3, f=3)),
])
def test_relational_recompose_equals_dense(kind, spec, ext, blk):
    """Def. 3.7 with the recompose map (join, SUM, then the map on the
    aggregated blocks) against the dense definition, ragged blocks included."""
    ins, out = spec.split("->")
    ins = ins.split(",")
    rng = np.random.default_rng(13)
    xs = [rng.standard_normal([ext[c] for c in lt]) for lt in ins]
    rels = [O.to_relation(x, lt, ext, blk) for x, lt in zip(xs, ins)]
    got_rel, present = O.relational_recompose(spec, kind, rels, ext, blk, alpha=0.75)
    assert present.all()
    got = O.from_relation(got_rel, out, ext, blk)
    want = O.dense_recompose(spec, kind, xs, ext, alpha=0.75)
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))
    pad = O.to_relation(np.ones([ext[c] for c in out], dtype=np.uint8), out, ext, blk) == 0
    assert np.all(got_rel[pad] == 0.0)
