"""Host-side logic with no GPU: the benchmark's algorithmic work counts, the
binding's marshalling of interval blockings, and the workload recipes.

FLOP counts are checked against closed forms written out here: 2 per
multiply-add over the unpadded index space; a causal pair keeps the
S(S+1)/2 pairs t <= s; a segment pair keeps the pairs inside each segment.
"""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from tensor_relational_einsum_amd import inputs as I  # noqa: E402
from tensor_relational_einsum_amd import jagg  # noqa: E402


def test_contraction_flops():
    st = I.Step("C", "ij,jk->ik", ["A", "B"], "mul", "sum", "f32", {})
    assert bench.spec_flops(st, dict(i=3, j=5, k=7)) == 2 * 3 * 5 * 7
    st = I.Step("M", "ij->i", ["A"], "ident", "max", "f32", {})
    assert bench.spec_flops(st, dict(i=3, j=5)) == 0.0  # not a contraction


def test_attention_flops_plain_causal_and_segmented():
    ext = dict(b=2, h=3, s=10, t=10, d=4, e=4)
    spec = "bhsd,bhtd,bhte->bhse"
    full = I.Step("O", spec, ["Q", "K", "V"], "attention", "softmax", "f32", {})
    assert bench.spec_flops(full, ext) == 2 * (2 * 2 * 3 * 10 * 10 * 4)
    causal = I.Step("O", spec, ["Q", "K", "V"], "attention", "softmax", "f32", {}, causal=("s", "t"))
    assert bench.spec_flops(causal, ext) == 2 * (2 * 2 * 3 * (10 * 11 // 2) * 4)
    bnd = [0, 3, 4, 10]  # segments of 3, 1, 6
    seg = I.Step("O", spec, ["Q", "K", "V"], "attention", "softmax", "f32", dict(s=bnd, t=bnd), causal=("s", "t"),
                 segment=("s", "t"))
    pairs = 3 * 4 // 2 + 1 + 6 * 7 // 2
    assert bench.spec_flops(seg, ext) == 2 * (2 * 2 * 3 * pairs * 4)
    seg_nc = I.Step("O", spec, ["Q", "K", "V"], "attention", "softmax", "f32", dict(s=bnd, t=bnd),
                    segment=("s", "t"))
    assert bench.spec_flops(seg_nc, ext) == 2 * (2 * 2 * 3 * (9 + 1 + 36) * 4)
    uni = I.Step("O", spec, ["Q", "K", "V"], "attention", "softmax", "f32", dict(s=3, t=3), segment=("s", "t"))
    assert bench.spec_flops(uni, ext) == 2 * (2 * 2 * 3 * (16 + 16 + 4) * 4)  # blocks of 4, 4, 2


def test_gqa_flops_count_every_query_head():
    w = I.attention_gqa(b=1, kv=2, group=3, s=8, d=4, nb=2)
    st = w.chain[0]
    # 6 query heads, causal 8 x 9 / 2 pairs, two products of D = E = 4
    assert bench.spec_flops(st, w.extents) == 2 * (2 * 6 * 36 * 4)


def test_packed_recipe_follows_the_sequence_ends():
    w = I.attention_packed()
    st = w.chain[0]
    assert st.blockings["s"] == [0, 1024, 2560, 4096] == st.blockings["t"]
    assert st.segment == ("s", "t") and st.causal == ("s", "t")
    assert w.extents["s"] == 4096
    rp = I.repartition_packed()
    assert rp.tensors[0][-1] == {"s": [0, 1024, 2560, 4096]} and rp.chain[0].blockings == {"s": 4}


def test_blocking_values_marshal_counts_and_bounds():
    assert jagg.block_count(4) == 4 and jagg.block_count([0, 3, 9]) == 2
    counts, bnd, keep = jagg._bounds([2, [0, 5, 7, 11], 1])
    assert list(counts) == [2, 3, 1]
    assert not bnd[0] and not bnd[2]          # uniform letters pass NULL
    assert [bnd[1][i] for i in range(4)] == [0, 5, 7, 11]
    assert len(keep) == 1


@pytest.mark.parametrize("bounds", [[0, 5, 7, 11], [0, 11]])
def test_interval_relation_size_through_the_binding(bounds):
    # 'ij': i blocked by bounds (padded to the longest interval), j uniform in 2 of 3
    blocks = len(bounds) - 1
    longest = max(b - a for a, b in zip(bounds, bounds[1:]))
    assert jagg.relation_bytes("ij", [11, 6], [bounds, 2], "f32") == 4 * blocks * longest * 2 * 3
    assert jagg.relation_bytes("ij", [11, 6], [bounds, 2], "bf16") == 2 * blocks * longest * 2 * 3


def test_bench_refuses_more_than_one_gpu():
    """The executor has one-GPU scope: bench.py exits with a message before
    touching a device when asked for several GPUs or started under a
    multi-rank launcher."""
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2 and "exactly one GPU" in r.stderr
    env = dict(os.environ, WORLD_SIZE="4")
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py")], capture_output=True, text=True,
                       timeout=300, env=env)
    assert r.returncode == 2 and "exactly one GPU" in r.stderr


@pytest.mark.parametrize("label", list("ABCDE"))
def test_matrix_chain_recipe_matches_the_pages(label):
    """Every Kernel Is a Join, Sec. 6: each multiply of a chain averages about
    8192^3 scalar multiplies; chain C is right-associated; D and E end in one
    large product across a thin neck."""
    w = I.matrix_chain(label)
    macs = []
    for st in w.chain:
        (la, lb) = st.spec.split("->")[0].split(",")
        macs.append(w.extents[la[0]] * w.extents[la[1]] * w.extents[lb[1]])
    assert len(macs) == len(w.tensors) - 1
    assert abs(np.mean(macs) / 8192 ** 3 - 1.0) < 0.05
    # every matrix is used once, in order, and the last product covers M1..Mn
    assert w.chain[-1].out == f"P1_{len(w.tensors)}"
    used = [n for st in w.chain for n in st.ins if n.startswith("M")]
    assert sorted(used, key=lambda s: int(s[1:])) == [f"M{i}" for i in range(1, len(w.tensors) + 1)]
    # the printed dimensions: ends, necks and interior (Sec. 6)
    dims = [w.extents[t[1][0]] for t in w.tensors] + [w.extents[w.tensors[-1][1][1]]]
    printed = {
        "A": [10240] + [16384, 6144] * 4 + [10240],
        "B": [9216] + [20480, 5120] * 2 + [9216],
        "C": [10240, 12288, 32768, 2048],
        "D": [24576, 1536] + [20480] * 6 + [1536, 24576],
        "E": [49152, 1024] + [20480] * 10 + [1024, 49152],
    }
    assert dims == printed[label]
    # the printed parenthesizations, as the order of the products
    order = {
        "A": ["P1_2", "P3_4", "P5_6", "P7_8", "P5_8", "P3_8", "P1_8", "P1_9"],
        "B": ["P1_2", "P3_4", "P3_5", "P1_5"],
        "C": ["P2_3", "P1_3"],
        "D": ["P7_8", "P6_8", "P5_8", "P4_8", "P3_8", "P2_8", "P1_8", "P1_9"],
        "E": ["P11_12", "P10_12", "P9_12", "P8_12", "P7_12", "P6_12", "P5_12", "P4_12", "P3_12", "P2_12",
              "P1_12", "P1_13"],
    }
    assert [st.out for st in w.chain] == order[label]
    if label == "C":
        assert [st.out for st in w.chain] == ["P2_3", "P1_3"]
    if label in "DE":
        last = w.chain[-1].spec.split("->")[0].split(",")
        assert w.extents[last[0][1]] <= 1536 and w.extents[last[0][0]] >= 24576
    for st in w.chain:  # every block a multiple of the 256-wide tile
        for c in st.spec.replace(",", "").replace("->", ""):
            assert (w.extents[c] // st.blockings[c]) % 256 == 0
