"""Pins for the oracle's attention join-agg (the online-softmax triple).

"Stax (5): Caching and Measurement", chapter summary on Section 9.10 and
exercise 15 on the triple (m, l, a):
attention is tiled like a reduction whose aggregation merges triples; with
"Every Kernel Is a Join" Def. 3.7 that is one join-agg over blocked Q, K, V.
The oracle's dense form is pinned to torch's softmax and matmul in float64
(a library routine), the relational form to the dense form and to the
unfused five-spec chain, the merge to its algebra, and both to closed forms
(uniform scores give prefix means; one dominant key selects its V row).
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O

SPEC = "bsd,btd,bte->bse"


def rand(shape, seed):
    return np.random.default_rng(seed).normal(size=shape)


def torch_attention(Q, K, V, alpha, causal):
    """Q [B, S, D], K [B, T, D], V [B, T, E] in float64 through torch."""
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)) for x in (Q, K, V))
    s = alpha * (q @ k.transpose(1, 2))
    if causal:
        S, T = s.shape[1], s.shape[2]
        mask = torch.arange(T)[None, :] > torch.arange(S)[:, None]
        s = s.masked_fill(mask, float("-inf"))
    return (torch.softmax(s, dim=-1) @ v).numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,S,T,D,E,alpha", [(2, 7, 7, 5, 3, 0.3), (3, 9, 9, 16, 16, 0.25), (1, 4, 11, 3, 6, 1.0)])
def test_dense_matches_torch_softmax(B, S, T, D, E, alpha, causal):
    if causal and S != T:
        pytest.skip("the causal pair compares s and t positions directly")
    Q, K, V = rand((B, S, D), 1), rand((B, T, D), 2), rand((B, T, E), 3)
    ext = dict(b=B, s=S, t=T, d=D, e=E)
    got = O.attention_dense(SPEC, [Q, K, V], ext, alpha=alpha, causal=("s", "t") if causal else None)
    want = torch_attention(Q, K, V, alpha, causal)
    assert np.max(np.abs(got - want)) < 1e-12


def test_dense_multi_letter_roles_match_torch():
    """Two batch letters, two contracted letters (D = xy), two value letters
    (E = uv), with the operands' letters in mixed orders."""
    spec = "hbsxy,btyxh,btuhv->hbsuv"
    ext = dict(h=2, b=3, s=5, t=6, x=3, y=2, u=2, v=3)
    Q = rand((2, 3, 5, 3, 2), 4)
    K = rand((3, 6, 2, 3, 2), 5)
    V = rand((3, 6, 2, 2, 3), 6)
    got = O.attention_dense(spec, [Q, K, V], ext, alpha=0.7)
    q = Q.transpose(0, 1, 2, 3, 4).reshape(2 * 3, 5, 6)                       # [hb, s, xy]
    k = K.transpose(4, 0, 1, 3, 2).reshape(2 * 3, 6, 6)                       # [hb, t, xy]
    v = V.transpose(3, 0, 1, 2, 4).reshape(2 * 3, 6, 6)                       # [hb, t, uv]
    want = torch_attention(q, k, v, 0.7, False).reshape(2, 3, 5, 2, 3)
    assert np.max(np.abs(got - want)) < 1e-12


def test_dense_sampled_equals_full():
    Q, K, V = rand((2, 8, 4), 7), rand((2, 8, 4), 8), rand((2, 8, 5), 9)
    ext = dict(b=2, s=8, t=8, d=4, e=5)
    full = O.attention_dense(SPEC, [Q, K, V], ext, alpha=0.5, causal=("s", "t"))
    idx = np.array([0, 3, 17, 40, 79])
    part = O.attention_dense(SPEC, [Q, K, V], ext, alpha=0.5, causal=("s", "t"), sample=idx)
    assert np.array_equal(part, full.reshape(-1)[idx])


BLOCKINGS = [
    dict(b=1, s=1, t=1, d=1, e=1),
    dict(b=2, s=2, t=3, d=1, e=1),
    dict(b=1, s=3, t=4, d=1, e=2),     # ragged s (10 in 3), t (10 in 4), e (6 in 2)
    dict(b=2, s=5, t=2, d=1, e=3),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("blk", BLOCKINGS)
def test_relational_matches_dense(blk, causal):
    B, S, T, D, E = 2, 10, 10, 7, 6
    Q, K, V = rand((B, S, D), 10), rand((B, T, D), 11), rand((B, T, E), 12)
    ext = dict(b=B, s=S, t=T, d=D, e=E)
    cz = ("s", "t") if causal else None
    want = O.attention_dense(SPEC, [Q, K, V], ext, alpha=0.4, causal=cz)
    rels = [O.to_relation(x, lt, ext, blk) for x, lt in zip((Q, K, V), ("bsd", "btd", "bte"))]
    got_rel, present = O.attention_relational(SPEC, rels, ext, blk, alpha=0.4, causal=cz)
    got = O.from_relation(got_rel, "bse", ext, blk)
    assert np.max(np.abs(got - want)) < 1e-12
    assert present.all()  # every (b, s, e) key joins at least its t <= s tuples
    pad = O.to_relation(np.ones((B, S, E), dtype=np.uint8), "bse", ext, blk) == 0
    assert np.all(got_rel[pad] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_relational_equals_unfused_chain(causal):
    """The five-spec chain (scores, MAX, SUM of exp, normalise, P V) in float64
    with no rounding between stages gives the same attention."""
    B, S, T, D, E = 2, 9, 9, 4, 3
    Q, K, V = rand((B, S, D), 13), rand((B, T, D), 14), rand((B, T, E), 15)
    ext = dict(b=B, s=S, t=T, d=D, e=E)
    cz = ("s", "t") if causal else None
    sc = O.dense("bsd,btd->bst", [Q, K], ext, alpha=0.6, causal=cz)
    if causal:
        sc = np.where(np.arange(T)[None, None, :] > np.arange(S)[None, :, None], -np.inf, sc)
    m = O.dense("bst->bs", [sc], ext, g="ident", agg="max", causal=cz)
    l = O.dense("bst,bs->bs", [sc, m], ext, g="exp_sub", agg="sum", causal=cz)
    p = O.dense("bst,bs,bs->bst", [sc, m, l], ext, g="exp_sub_div", agg="none", causal=cz)
    chain = O.dense("bst,bte->bse", [p, V], ext)
    blk = dict(b=1, s=3, t=3, d=1, e=1)
    rels = [O.to_relation(x, lt, ext, blk) for x, lt in zip((Q, K, V), ("bsd", "btd", "bte"))]
    got_rel, _ = O.attention_relational(SPEC, rels, ext, blk, alpha=0.6, causal=cz)
    got = O.from_relation(got_rel, "bse", ext, blk)
    assert np.max(np.abs(got - chain)) < 1e-12


def test_merge_identity_commutativity_associativity():
    rng = np.random.default_rng(16)
    ident = (-np.inf, 0.0, 0.0)
    for _ in range(200):
        x = (rng.normal() * 10, rng.uniform(0.1, 5), rng.normal())
        y = (rng.normal() * 10, rng.uniform(0.1, 5), rng.normal())
        z = (rng.normal() * 10, rng.uniform(0.1, 5), rng.normal())
        assert O.softmax_merge(x, ident) == x
        assert O.softmax_merge(ident, x) == x
        xy, yx = O.softmax_merge(x, y), O.softmax_merge(y, x)
        assert xy[0] == yx[0] and np.allclose(xy[1:], yx[1:], rtol=1e-14, atol=0)
        left = O.softmax_merge(O.softmax_merge(x, y), z)
        right = O.softmax_merge(x, O.softmax_merge(y, z))
        assert left[0] == right[0] and np.allclose(left[1:], right[1:], rtol=1e-13, atol=0)
    assert O.softmax_merge(ident, ident) == ident


def test_merge_of_two_halves_is_the_whole():
    """Triples of two halves of a score row merge into the triple of the row."""
    rng = np.random.default_rng(17)
    sc, v = rng.normal(size=12) * 4, rng.normal(size=12)

    def triple(s, w):
        m = s.max()
        return (m, np.exp(s - m).sum(), (np.exp(s - m) * w).sum())

    whole = triple(sc, v)
    merged = O.softmax_merge(triple(sc[:5], v[:5]), triple(sc[5:], v[5:]))
    assert merged[0] == whole[0]
    assert np.allclose(merged[1:], whole[1:], rtol=1e-14, atol=0)


def test_uniform_scores_give_prefix_means():
    """Q = 0: every score is 0, so the causal output is the mean of V over t <= s."""
    B, S, D, E = 2, 8, 3, 4
    Q = np.zeros((B, S, D))
    K, V = rand((B, S, D), 18), rand((B, S, E), 19)
    ext = dict(b=B, s=S, t=S, d=D, e=E)
    blk = dict(b=1, s=3, t=2, d=1, e=1)
    rels = [O.to_relation(x, lt, ext, blk) for x, lt in zip((Q, K, V), ("bsd", "btd", "bte"))]
    got_rel, _ = O.attention_relational(SPEC, rels, ext, blk, causal=("s", "t"))
    got = O.from_relation(got_rel, "bse", ext, blk)
    want = np.cumsum(V, axis=1) / np.arange(1, S + 1)[None, :, None]
    assert np.max(np.abs(got - want)) < 1e-14


def test_dominant_key_selects_its_value():
    """With alpha large and one key aligned with the query, the softmax is a
    one-hot on that key (no overflow: the triple subtracts its maximum)."""
    B, S, T, D, E = 1, 4, 9, 4, 3
    Q = np.zeros((B, S, D))
    Q[0, :, 0] = 1.0
    K = np.zeros((B, T, D))
    K[0, 6, 0] = 1.0
    V = rand((B, T, E), 20)
    ext = dict(b=B, s=S, t=T, d=D, e=E)
    blk = dict(b=1, s=2, t=3, d=1, e=1)
    rels = [O.to_relation(x, lt, ext, blk) for x, lt in zip((Q, K, V), ("bsd", "btd", "bte"))]
    got_rel, _ = O.attention_relational(SPEC, rels, ext, blk, alpha=1.0e4)
    got = O.from_relation(got_rel, "bse", ext, blk)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - V[0, 6][None, None, :])) < 1e-12


def test_rejects_malformed_attention():
    ext = dict(b=2, s=4, t=4, d=8, e=3)
    Q, K, V = rand((2, 4, 8), 1), rand((2, 4, 8), 2), rand((2, 4, 3), 3)
    with pytest.raises(O.OracleError):  # the contracted letter cut into blocks
        blk = dict(b=1, s=1, t=1, d=2, e=1)
        rels = [O.to_relation(x, lt, ext, blk) for x, lt in zip((Q, K, V), ("bsd", "btd", "bte"))]
        O.attention_relational(SPEC, rels, ext, blk)
    with pytest.raises(O.OracleError):  # no key letter shared by K and V alone
        O.attention_dense("bsd,btd,bse->bse", [Q, K, rand((2, 4, 3), 4)], ext)
    with pytest.raises(O.OracleError):  # causal letters that are not (s, t)
        O.attention_dense(SPEC, [Q, K, V], ext, causal=("t", "s"))


# Grouped-query attention ("Every Kernel Is a Join", Sec. 3.3, Example 3.10):
# query heads 4m..4m+3 use key-value head m.  Written with a query-group
# letter r that appears in Q and the output only: "grsd,gtd,gte->grse".
GQA = "grsd,gtd,gte->grse"


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_dense_equals_attention_with_repeated_kv_heads(causal):
    g, r, S, D, E = 3, 4, 9, 8, 5
    Q, K, V = rand((g, r, S, D), 41), rand((g, S, D), 42), rand((g, S, E), 43)
    ext = dict(g=g, r=r, s=S, t=S, d=D, e=E)
    got = O.attention_dense(GQA, [Q, K, V], ext, alpha=0.4, causal=("s", "t") if causal else None)
    # torch: flatten the query heads, repeat each kv head for its group
    Kr, Vr = np.repeat(K, r, axis=0), np.repeat(V, r, axis=0)
    want = torch_attention(Q.reshape(g * r, S, D), Kr, Vr, 0.4, causal).reshape(g, r, S, E)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_relational_by_kv_head_equals_dense(causal):
    """Blocking the kv-head letter g into unit intervals gives one joined
    (Q, K, V) combination per kv head and s/t block pair; the query group
    follows its kv head (Example 3.10)."""
    g, r, S, D, E = 4, 2, 10, 4, 3
    Q, K, V = rand((g, r, S, D), 44), rand((g, S, D), 45), rand((g, S, E), 46)
    ext = dict(g=g, r=r, s=S, t=S, d=D, e=E)
    blk = dict(g=4, r=1, s=3, t=3)
    c = ("s", "t") if causal else None
    want = O.attention_dense(GQA, [Q, K, V], ext, alpha=0.7, causal=c)
    rels = [O.to_relation(x, lt, ext, blk) for x, lt in zip((Q, K, V), ("grsd", "gtd", "gte"))]
    got, present = O.attention_relational(GQA, rels, ext, blk, alpha=0.7, causal=c)
    assert present.all()
    np.testing.assert_allclose(O.from_relation(got, "grse", ext, blk), want, rtol=1e-12, atol=1e-13)
    # the query-group letter written innermost-but-one or outermost changes nothing
    Qt = np.ascontiguousarray(Q.transpose(1, 0, 2, 3))
    got2 = O.attention_dense("rgsd,gtd,gte->rgse", [Qt, K, V], ext, alpha=0.7, causal=c)
    np.testing.assert_allclose(got2.transpose(1, 0, 2, 3), want, rtol=1e-12, atol=1e-13)


def test_gqa_causal_letter_must_be_a_query_letter():
    ext = dict(g=2, r=2, s=4, t=4, d=3, e=3)
    Q, K, V = rand((2, 2, 4, 3), 47), rand((2, 4, 3), 48), rand((2, 4, 3), 49)
    with pytest.raises(O.OracleError):
        O.attention_dense(GQA, [Q, K, V], ext, causal=("g", "t"))


# Packed sequences ("Every Kernel Is a Join", Sec. 3.3, Example 3.10): three
# sequences packed end to end; attention never crosses a sequence boundary,
# so the sequence index is cut only at the sequence ends, and the join pairs
# each query block with the key block of the same sequence.
PACK = [0, 5, 7, 16]


@pytest.mark.parametrize("causal", [False, True])
def test_segments_dense_equals_attention_per_sequence(causal):
    B, S, D, E = 2, PACK[-1], 6, 4
    Q, K, V = rand((B, S, D), 51), rand((B, S, D), 52), rand((B, S, E), 53)
    ext = dict(b=B, s=S, t=S, d=D, e=E)
    got = O.attention_dense(SPEC, [Q, K, V], ext, alpha=0.5, causal=("s", "t") if causal else None,
                            segments=("s", "t", PACK))
    for lo, hi in zip(PACK, PACK[1:]):
        want = torch_attention(Q[:, lo:hi], K[:, lo:hi], V[:, lo:hi], 0.5, causal)
        np.testing.assert_allclose(got[:, lo:hi], want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_segments_relational_on_sequence_intervals_equals_dense(causal):
    B, S, D, E = 2, PACK[-1], 4, 3
    Q, K, V = rand((B, S, D), 54), rand((B, S, D), 55), rand((B, S, E), 56)
    ext = dict(b=B, s=S, t=S, d=D, e=E)
    blk = dict(b=2, s=PACK, t=PACK)
    c = ("s", "t") if causal else None
    want = O.attention_dense(SPEC, [Q, K, V], ext, alpha=0.3, causal=c, segments=("s", "t", PACK))
    rels = [O.to_relation(x, lt, ext, blk) for x, lt in zip((Q, K, V), ("bsd", "btd", "bte"))]
    got, present = O.attention_relational(SPEC, rels, ext, blk, alpha=0.3, causal=c, segment=("s", "t"))
    assert present.all()
    np.testing.assert_allclose(O.from_relation(got, "bse", ext, blk), want, rtol=1e-12, atol=1e-13)
    # padding rows of the short sequences stay +0
    pad = O.to_relation(np.ones((B, S, E)), "bse", ext, blk) == 0
    assert pad.any() and np.all(got[pad] == 0.0)


def test_segments_on_uniform_blocks_are_block_local_attention():
    B, S, D, E = 1, 12, 4, 4
    Q, K, V = rand((B, S, D), 57), rand((B, S, D), 58), rand((B, S, E), 59)
    ext = dict(b=B, s=S, t=S, d=D, e=E)
    blk = dict(s=3, t=3)
    rels = [O.to_relation(x, lt, ext, blk) for x, lt in zip((Q, K, V), ("bsd", "btd", "bte"))]
    got, _ = O.attention_relational(SPEC, rels, ext, blk, alpha=0.6, segment=("s", "t"))
    want = O.attention_dense(SPEC, [Q, K, V], ext, alpha=0.6, segments=("s", "t", [0, 4, 8, 12]))
    np.testing.assert_allclose(O.from_relation(got, "bse", ext, blk), want, rtol=1e-12, atol=1e-13)
    for lo in (0, 4, 8):
        np.testing.assert_allclose(want[:, lo:lo + 4], torch_attention(Q[:, lo:lo + 4], K[:, lo:lo + 4],
                                                                      V[:, lo:lo + 4], 0.6, False), rtol=1e-12)


def test_segments_reject_other_letters_and_bad_bounds():
    ext = dict(b=1, s=6, t=6, d=3, e=3)
    Q, K, V = rand((1, 6, 3), 60), rand((1, 6, 3), 61), rand((1, 6, 3), 62)
    with pytest.raises(O.OracleError):  # the pair must be (s, t)
        O.attention_dense(SPEC, [Q, K, V], ext, segments=("b", "t", [0, 1]))
    with pytest.raises(O.OracleError):  # bounds must end at the extent
        O.attention_dense(SPEC, [Q, K, V], ext, segments=("s", "t", [0, 2, 5]))
