"""Pins for interval blockings in the oracle.

"Every Kernel Is a Join" (Ding et al.): a key is a tensor type, an interval
per index (Def. 3.1), and Sec. 3.3 lets an index be split only at legal
positions (Example 3.10: packed sequences split at their ends; query heads
split along with their key-value heads).  A blocking value may therefore be a
list of bounds [0, b_1, ..., n] instead of a block count.

The checks here tie the interval path to slicing in numpy, to literal
hand-worked layouts, to the uniform path (already pinned elsewhere) when the
bounds are the uniform ones, and to the dense definition of each spec.
"""
import os

import numpy as np
import pytest

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden():
    f = {}
    for line in open(os.path.join(GOLDEN, "packed_sequence.txt")):
        if line.strip() and line[0] != "#":
            k, *v = line.split()
            f[k] = list(map(int, v))
    return f


def uniform_bounds(n, k):
    e = -(-n // k)
    return [min(q * e, n) for q in range(k + 1)]


def test_tiny_layout_by_hand():
    """n = 5 split at 2: blocks [0,2) and [2,5), both padded to 3."""
    x = np.array([11, 12, 13, 14, 15], dtype=np.int64)
    assert O.block_shape("i", dict(i=5), dict(i=[0, 2, 5])) == (3,)
    rel = O.to_relation(x, "i", dict(i=5), dict(i=[0, 2, 5]))
    assert rel.tolist() == [11, 12, 0, 13, 14, 15]
    assert O.from_relation(rel, "i", dict(i=5), dict(i=[0, 2, 5])).tolist() == x.tolist()
    # 2-D: rows split at 1 of 3, columns uniform in 2 blocks of 2
    y = np.arange(1, 13, dtype=np.int64).reshape(3, 4)
    rel = O.to_relation(y, "ij", dict(i=3, j=4), dict(i=[0, 1, 3], j=2))
    assert rel.tolist() == [1, 2, 0, 0,   3, 4, 0, 0,
                            5, 6, 9, 10,  7, 8, 11, 12]


def test_packed_sequence_blocks_are_the_sequences():
    f = golden()
    n, bnd = f["extent"][0], f["bounds"]
    rng = np.random.default_rng(21)
    x = rng.integers(1, 60000, size=(n, 4), dtype=np.uint16)
    ext, blk = dict(s=n, d=4), dict(s=bnd, d=1)
    assert O.block_shape("sd", ext, blk) == (f["padded"][0], 4)
    rel = O.to_relation(x, "sd", ext, blk).reshape(len(bnd) - 1, f["padded"][0], 4)
    for m in range(len(bnd) - 1):
        L = f["valid"][m]
        assert bnd[m + 1] - bnd[m] == L
        assert np.array_equal(rel[m, :L], x[bnd[m]:bnd[m + 1]])
        assert not rel[m, L:].any()
    assert np.array_equal(O.from_relation(rel.ravel(), "sd", ext, blk), x)


def test_gqa_query_heads_follow_kv_heads():
    """Example 3.10: the query tensor [heads_q, s, d] viewed as [kv, group, s, d]
    and blocked by kv head gives tuple m = query heads [4m, 4m+4); so does the
    interval blocking of heads_q derived from the kv-head blocking."""
    f = golden()
    hq, hkv, grp = f["heads_q"][0], f["heads_kv"][0], f["group"][0]
    assert hq == hkv * grp
    rng = np.random.default_rng(22)
    q = rng.standard_normal((hq, 6, 5))
    split = O.to_relation(q.reshape(hkv, grp, 6, 5), "grsd", dict(g=hkv, r=grp, s=6, d=5),
                          dict(g=hkv)).reshape(hkv, grp, 6, 5)
    for m in range(hkv):
        assert np.array_equal(split[m], q[grp * m:grp * (m + 1)])
    derived = dict(h=[grp * m for m in range(hkv + 1)])
    via_iv = O.to_relation(q, "hsd", dict(h=hq, s=6, d=5), derived)
    assert np.array_equal(via_iv, split.ravel())


@pytest.mark.parametrize("shape,blk", [
    ((7, 5), dict(a=[0, 3, 7], b=2)),
    ((9, 4, 6), dict(a=[0, 1, 2, 9], b=[0, 3, 4], c=2)),
    ((10,), dict(a=[0, 4, 5, 6, 10])),
    ((4, 8), dict(a=[0, 4], b=[0, 1, 2, 3, 4, 5, 6, 7, 8])),
])
def test_interval_relation_tiles_the_tensor(shape, blk):
    """Every element lands in exactly one block, padding holds +0, the round
    trip to dense is the identity (Def. 3.2 with non-uniform intervals)."""
    letters = "abc"[:len(shape)]
    ext = dict(zip(letters, shape))
    n = int(np.prod(shape))
    ids = (np.arange(n, dtype=np.int64) + 1).reshape(shape)
    rel = O.to_relation(ids, letters, ext, blk)
    vals = rel[rel != 0]
    assert np.array_equal(np.sort(vals), np.arange(1, n + 1))
    counts = [len(v) - 1 if isinstance(v, list) else v for v in (blk.get(c, 1) for c in letters)]
    e = O.block_shape(letters, ext, blk)
    for c, ee in zip(letters, e):
        v = blk.get(c, 1)
        want = max(np.diff(v)) if isinstance(v, list) else -(-ext[c] // v)
        assert ee == want
    assert rel.size == int(np.prod(counts)) * int(np.prod(e))
    assert np.array_equal(O.from_relation(rel, letters, ext, blk), ids)


def test_uniform_bounds_equal_the_uniform_blocking():
    """Bounds that are the uniform ones reproduce the count path exactly:
    relation bytes, join list and relational result."""
    rng = np.random.default_rng(23)
    ext = dict(i=10, j=7, k=9)
    cnt = dict(i=3, j=2, k=2)
    bnd = {c: uniform_bounds(ext[c], cnt[c]) for c in cnt}
    A, B = rng.standard_normal((10, 7)), rng.standard_normal((7, 9))
    for x, lt in ((A, "ij"), (B, "jk")):
        assert np.array_equal(O.to_relation(x, lt, ext, cnt), O.to_relation(x, lt, ext, bnd))
    assert np.array_equal(O.join_list("ij,jk->ik", ext, cnt), O.join_list("ij,jk->ik", ext, bnd))
    ra = [O.to_relation(A, "ij", ext, cnt), O.to_relation(B, "jk", ext, cnt)]
    got_c, _ = O.relational("ij,jk->ik", ra, ext, cnt)
    got_b, _ = O.relational("ij,jk->ik", ra, ext, bnd)
    assert np.array_equal(got_c, got_b)


IV_CASES = [
    # spec, g, agg, extents, blockings, causal
    ("ij,jk->ik", "mul", "sum", dict(i=10, j=12, k=5), dict(i=[0, 4, 10], j=[0, 1, 6, 12], k=2), None),
    ("sh,ho->so", "mul", "sum", dict(s=11, h=6, o=4), dict(s=[0, 3, 4, 11], h=2, o=1), None),
    ("bst->bs", "ident", "max", dict(b=2, s=7, t=8), dict(b=1, s=[0, 5, 7], t=[0, 2, 3, 8]), None),
    ("sd,td->st", "mul", "sum", dict(s=9, t=9, d=4), dict(s=[0, 2, 7, 9], t=[0, 2, 7, 9], d=2), ("s", "t")),
    ("qst,qtd->qsd", "mul", "sum", dict(q=2, s=10, t=10, d=3),
     dict(q=2, s=[0, 6, 10], t=[0, 6, 10], d=1), ("s", "t")),
    ("bsh,bsh->bsh", "add", "none", dict(b=2, s=5, h=5), dict(b=2, s=[0, 1, 5], h=[0, 3, 5]), None),
    ("bsh,bs,h->bsh", "rms_scale", "none", dict(b=2, s=6, h=9), dict(b=1, s=[0, 4, 6], h=[0, 2, 9]), None),
]


@pytest.mark.parametrize("spec,g,agg,ext,blk,causal", IV_CASES)
def test_interval_relational_equals_dense(spec, g, agg, ext, blk, causal):
    """Def. 3.7 over interval keys: join on equal intervals, aggregate,
    recompose; the recomposed result is the dense spec's."""
    rng = np.random.default_rng(sum(map(ord, spec)))
    ins, out = spec.split("->")
    ins = ins.split(",")
    xs = []
    for lt in ins:
        lo = 0.5 if (g == "rms_scale" and lt == ins[1]) else -2.0
        xs.append(rng.uniform(lo, 2.0, size=[ext[c] for c in lt]))
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
    pad = O.to_relation(np.ones(want.shape), out, ext, blk) == 0
    assert np.all(got_rel[pad] == 0.0)


def test_interval_join_list_pairs_equal_intervals():
    """The join keeps a pair only when the shared letter's intervals agree;
    with k_i x k_j x k_k blocks a matmul lists every (i, j, k) block triple."""
    ext = dict(i=10, j=12, k=5)
    blk = dict(i=[0, 4, 10], j=[0, 1, 6, 12], k=2)
    lst = O.join_list("ij,jk->ik", ext, blk)
    assert lst.shape == (2 * 3 * 2, 3)
    for out_id, a, b in lst:
        i_blk, k_blk = divmod(int(out_id), 2)
        ai, aj = divmod(int(a), 3)
        bj, bk = divmod(int(b), 2)
        assert (ai, aj, bk) == (i_blk, bj, k_blk)


def test_interval_attention_equals_dense():
    rng = np.random.default_rng(24)
    ext = dict(h=2, s=10, t=10, d=4, e=3)
    blk = dict(h=2, s=[0, 3, 4, 10], t=[0, 6, 10])
    q, k, v = rng.standard_normal((2, 10, 4)), rng.standard_normal((2, 10, 4)), rng.standard_normal((2, 10, 3))
    for causal in (None, ("s", "t")):
        want = O.attention_dense("hsd,htd,hte->hse", [q, k, v], ext, alpha=0.5, causal=causal)
        rels = [O.to_relation(x, lt, ext, blk) for x, lt in ((q, "hsd"), (k, "htd"), (v, "hte"))]
        got, _ = O.attention_relational("hsd,htd,hte->hse", rels, ext, blk, alpha=0.5, causal=causal)
        np.testing.assert_allclose(O.from_relation(got, "hse", ext, blk), want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("shape,src_l,src_b,dst_l,dst_b", [
    ((4096, 4), "sd", dict(s=[0, 1024, 2560, 4096]), "sd", dict(s=4)),
    ((11, 6), "ij", dict(i=[0, 3, 4, 11], j=2), "ji", dict(i=[0, 5, 11], j=[0, 1, 6])),
    ((7, 5, 6), "abc", dict(a=2, b=[0, 2, 5], c=3), "cab", dict(a=[0, 1, 7], b=1, c=[0, 4, 6])),
])
@pytest.mark.parametrize("dtype", [np.uint16, np.uint32])
def test_interval_repartition_round_trip_and_dense_view(shape, src_l, src_b, dst_l, dst_b, dtype):
    rng = np.random.default_rng(25)
    ext = dict(zip(src_l, shape))
    dense = rng.integers(1, np.iinfo(dtype).max, size=shape, dtype=dtype)
    src = O.to_relation(dense, src_l, ext, src_b)
    dst = O.repartition(src, src_l, src_b, dst_l, dst_b, ext)
    assert np.array_equal(O.repartition(dst, dst_l, dst_b, src_l, src_b, ext), src)
    perm = [src_l.index(c) for c in dst_l]
    assert np.array_equal(O.from_relation(dst, dst_l, ext, dst_b), dense.transpose(perm))


@pytest.mark.parametrize("bounds", [
    [1, 3, 5],        # does not start at 0
    [0, 3, 4],        # does not end at n
    [0, 3, 3, 5],     # empty interval
    [0, 4, 2, 5],     # decreasing
    [0, 5],           # fine: one block
])
def test_bad_bounds_rejected(bounds):
    if bounds == [0, 5]:
        assert O.block_shape("i", dict(i=5), dict(i=bounds)) == (5,)
        return
    with pytest.raises(O.OracleError):
        O.block_shape("i", dict(i=5), dict(i=bounds))


def test_too_many_intervals_rejected():
    with pytest.raises(O.OracleError):
        O.block_shape("i", dict(i=100), dict(i=list(range(0, 66)) + [100]))
