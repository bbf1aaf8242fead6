"""Seeded synthetic inputs and workload recipes.

This module is shared by the tests, the benchmark and the smoke check: it
only draws random numbers and describes workloads (shapes, blockings, spec
strings).  It holds none of the method's arithmetic and imports neither the
HIP binding nor the oracle.

Random numbers: ``numpy.random.Generator(PCG64)`` seeded from
``SeedSequence(1000 + config)``, one spawned child stream per tensor, in the
order the tensors are listed in each recipe.  uniform[-1, 1) and N(0, sigma^2)
are drawn in float64, cast to float32, and rounded to bfloat16 (torch's CPU
cast, round-to-nearest-even) where the tensor is bfloat16.  The matrix chains
(up to 3.8e9 elements per chain) use ``normal32`` instead: the tensor's
stream spawns 64 children, child c draws the c-th of 64 equal flat chunks
as float32 N(0, 1), which is scaled by sigma in float32 and rounded to
bfloat16; the chunks are drawn on 16 threads, and the values do not depend
on the thread count.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


def streams(seed: int, n: int):
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(n)]


N_CHUNKS = 64


def _normal32(gen, shape, sigma: float) -> np.ndarray:
    """float32 N(0, sigma^2) in N_CHUNKS flat chunks, chunk c from the c-th
    child of the stream's seed sequence (drawn on a thread pool)."""
    from concurrent.futures import ThreadPoolExecutor

    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    kids = gen.bit_generator.seed_seq.spawn(N_CHUNKS)
    bounds = [n * c // N_CHUNKS for c in range(N_CHUNKS + 1)]

    def fill(c):
        seg = out[bounds[c]:bounds[c + 1]]
        np.random.Generator(np.random.PCG64(kids[c])).standard_normal(seg.size, dtype=np.float32, out=seg)
        if sigma != 1.0:
            np.multiply(seg, np.float32(sigma), out=seg)

    with ThreadPoolExecutor(16) as ex:
        list(ex.map(fill, range(N_CHUNKS)))
    return out.reshape(shape)


def draw(gen, shape, dist: str, dtype: str, sigma: float = 1.0, mean: float = 0.0) -> torch.Tensor:
    """One tensor from one stream. dist: 'uniform' (on [-1,1)), 'normal',
    'normal32' (float32 draws in chunks; mean 0 only)."""
    shape = tuple(int(s) for s in shape)
    if dist == "normal32":
        if mean != 0.0:
            raise ValueError("normal32 draws have mean 0")
        t = torch.from_numpy(_normal32(gen, shape, sigma))
        if dtype == "bf16":
            return t.to(torch.bfloat16)
        if dtype != "f32":
            raise ValueError(dtype)
        return t
    if dist == "uniform":
        x = gen.uniform(-1.0, 1.0, size=shape)
    elif dist == "normal":
        x = gen.standard_normal(size=shape) * sigma + mean
    else:
        raise ValueError(dist)
    t = torch.from_numpy(x).to(torch.float32)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype != "f32":
        raise ValueError(dtype)
    return t


@dataclass
class Step:
    """One join-agg spec of a workload chain (names only, no arithmetic)."""
    out: str
    spec: str
    ins: list
    g: str = "mul"
    agg: str = "sum"
    out_dtype: str = "f32"
    blockings: dict = field(default_factory=dict)
    alpha: float = 1.0
    beta: float = 0.0
    eps: float = 0.0
    causal: tuple | None = None
    segment: tuple | None = None  # (s, t): attention within blocks only (packed sequences)


@dataclass
class Relayout:
    """Re-block a relation (letters and blocking of the destination)."""
    out: str
    src: str
    letters: str
    blockings: dict


@dataclass
class Workload:
    name: str
    extents: dict
    tensors: list            # (name, letters, dist, dtype, sigma, mean, blockings)
    chain: list              # Step / Relayout in execution order
    seed: int


def matmul_256(n: int = 256, nb: int = 4) -> Workload:
    """'ij,jk->ik', I=J=K=256 fp32, each index in 4 blocks, uniform[-1,1)."""
    ext = {"i": n, "j": n, "k": n}
    blk = {"i": nb, "j": nb, "k": nb}
    return Workload(
        name=f"matmul_ij_jk_{n}_fp32_blk{nb}", extents=ext,
        tensors=[("A", "ij", "uniform", "f32", 1.0, 0.0, blk), ("B", "jk", "uniform", "f32", 1.0, 0.0, blk)],
        chain=[Step("C", "ij,jk->ik", ["A", "B"], blockings=blk)], seed=1001)


def repartition_2d(n: int = 8192) -> Workload:
    """n x n bf16 N(0,1), {i8, j1} row blocks -> {i1, j8} column blocks."""
    ext = {"i": n, "j": n}
    return Workload(
        name=f"repartition_ij_{n}_bf16_i8j1_to_i1j8", extents=ext,
        tensors=[("X", "ij", "normal", "bf16", 1.0, 0.0, {"i": 8, "j": 1})],
        chain=[Relayout("Y", "X", "ij", {"i": 1, "j": 8})], seed=1002)


def repartition_4d(shape=(32, 128, 64, 64)) -> Workload:
    """'abcd' bf16 N(0,1) {a4,b8,c1,d1} -> 'acbd' {a1,b1,c4,d2}."""
    ext = dict(zip("abcd", shape))
    return Workload(
        name="repartition_abcd_32x128x64x64_bf16_to_acbd", extents=ext,
        tensors=[("X", "abcd", "normal", "bf16", 1.0, 0.0, {"a": 4, "b": 8, "c": 1, "d": 1})],
        chain=[Relayout("Y", "X", "acbd", {"a": 1, "b": 1, "c": 4, "d": 2})], seed=1002)


PACKED_ENDS = (0, 1024, 2560, 4096)  # three sequences packed into 4096 positions


def repartition_packed(b=8, s=4096, h=4096, bounds=PACKED_ENDS, to_packed=False) -> Workload:
    """'bsh' bf16 N(0,1): token blocks cut at the ends of packed sequences
    ("Every Kernel Is a Join", Sec. 3.3, Example 3.10: three sequences ending
    at 1024, 2560 and 4096) <-> four uniform token blocks."""
    ext = {"b": b, "s": s, "h": h}
    packed, uniform = {"s": list(bounds)}, {"s": 4}
    src, dst = (uniform, packed) if to_packed else (packed, uniform)
    name = "uniform_to_packed" if to_packed else "packed_to_uniform"
    return Workload(
        name=f"repartition_bsh_{b}x{s}x{h}_bf16_{name}", extents=ext,
        tensors=[("X", "bsh", "normal", "bf16", 1.0, 0.0, src)],
        chain=[Relayout("Y", "X", "bsh", dst)], seed=1004)


def attention_chain(b=4, h=32, s=2048, d=128, nb=16, fused=False) -> Workload:
    """Attention as join-aggs.  Unfused: QK^T, row MAX, row SUM of exp,
    normalize, PV (five specs).  Fused: one spec whose aggregation merges
    online-softmax triples.  No 1/sqrt(d) scale; Q, K, V bf16 N(0,1); s and
    t each in `nb` blocks."""
    ext = {"b": b, "h": h, "s": s, "t": s, "d": d, "e": d}
    blk = {"b": 1, "h": 1, "s": nb, "t": nb, "d": 1, "e": 1}
    tens = [("Q", "bhsd", "normal", "bf16", 1.0, 0.0, blk), ("K", "bhtd", "normal", "bf16", 1.0, 0.0, blk),
            ("V", "bhtd", "normal", "bf16", 1.0, 0.0, blk)]
    if fused:
        chain = [Step("O", "bhsd,bhtd,bhte->bhse", ["Q", "K", "V"], "attention", "softmax", "f32", blk)]
        return Workload(name=f"attention_fused_b{b}_h{h}_s{s}_d{d}_bf16_st{nb}", extents=ext, tensors=tens,
                        chain=chain, seed=1003)
    chain = [
        Step("S", "bhsd,bhtd->bhst", ["Q", "K"], "mul", "sum", "f32", blk),
        Step("M", "bhst->bhs", ["S"], "ident", "max", "f32", blk),
        Step("L", "bhst,bhs->bhs", ["S", "M"], "exp_sub", "sum", "f32", blk),
        Step("P", "bhst,bhs,bhs->bhst", ["S", "M", "L"], "exp_sub_div", "none", "bf16", blk),
        Step("O", "bhst,bhtd->bhsd", ["P", "V"], "mul", "sum", "f32", blk),
    ]
    return Workload(name=f"attention_chain_b{b}_h{h}_s{s}_d{d}_bf16_st{nb}", extents=ext, tensors=tens,
                    chain=chain, seed=1003)


def attention_gqa(b=4, kv=8, group=4, s=2048, d=128, nb=16) -> Workload:
    """Causal grouped-query attention as one join-agg ("Every Kernel Is a
    Join", Example 3.10: 32 query heads over 8 key-value heads, query heads
    4m..4m+3 on kv head m).  Q 'bgrsd' (g kv head, r member of its group),
    K and V 'bgtd'; the kv heads in unit intervals, s and t in `nb` blocks;
    scale 1/sqrt(d); bf16 N(0,1)."""
    ext = {"b": b, "g": kv, "r": group, "s": s, "t": s, "d": d, "e": d}
    blk = {"b": 1, "g": kv, "r": 1, "s": nb, "t": nb, "d": 1, "e": 1}
    tens = [("Q", "bgrsd", "normal", "bf16", 1.0, 0.0, blk), ("K", "bgtd", "normal", "bf16", 1.0, 0.0, blk),
            ("V", "bgtd", "normal", "bf16", 1.0, 0.0, blk)]
    chain = [Step("O", "bgrsd,bgtd,bgte->bgrse", ["Q", "K", "V"], "attention", "softmax", "bf16", blk,
                  alpha=1.0 / math.sqrt(d), causal=("s", "t"))]
    return Workload(name=f"attention_gqa_causal_b{b}_kv{kv}x{group}_s{s}_d{d}_bf16_st{nb}", extents=ext,
                    tensors=tens, chain=chain, seed=1005)


def attention_packed(b=2, kv=8, group=4, ends=PACKED_ENDS, d=128) -> Workload:
    """Causal grouped-query attention over packed sequences ("Every Kernel
    Is a Join", Example 3.10: 32 query heads over 8 kv heads; three
    sequences packed into 4096 positions, ending at 1024, 2560 and 4096).
    s and t are cut at the sequence ends and paired as a segment, so each
    query attends within its own sequence; bf16 N(0,1), scale 1/sqrt(d)."""
    n = ends[-1]
    ext = {"b": b, "g": kv, "r": group, "s": n, "t": n, "d": d, "e": d}
    blk = {"b": 1, "g": kv, "r": 1, "s": list(ends), "t": list(ends), "d": 1, "e": 1}
    tens = [("Q", "bgrsd", "normal", "bf16", 1.0, 0.0, blk), ("K", "bgtd", "normal", "bf16", 1.0, 0.0, blk),
            ("V", "bgtd", "normal", "bf16", 1.0, 0.0, blk)]
    chain = [Step("O", "bgrsd,bgtd,bgte->bgrse", ["Q", "K", "V"], "attention", "softmax", "bf16", blk,
                  alpha=1.0 / math.sqrt(d), causal=("s", "t"), segment=("s", "t"))]
    return Workload(name=f"attention_packed_causal_b{b}_kv{kv}x{group}_seq{'-'.join(map(str, ends[1:]))}_d{d}_bf16",
                    extents=ext, tensors=tens, chain=chain, seed=1006)


def llama_block(b=4, s=2048, hid=4096, heads=32, d=128, ffn=11008, s_blk=16, h_blk=4, q_blk=4, f_blk=8,
                fused_attention=False, fused_epilogues=False) -> Workload:
    """LLaMA-7B-shaped decoder block, every op a join-agg spec.

    x (fp32) -> RMSNorm*g1 -> Q,K,V -> causal attention (scale 1/sqrt(d)) ->
    Wo -> +x -> RMSNorm*g2 -> gate, up -> silu(gate)*up -> down -> +residual.
    No RoPE, no biases.  Attention is either the five-spec chain between
    relayouts to head-major order and back, or one spec whose aggregation
    merges online-softmax triples, read and written in the projections'
    own layout (no relayout).  With ``fused_epilogues`` the residual adds
    and the SiLU gate are the recompose maps of the contractions that feed
    them (g = mul_plus: x2 = x + O Wo, y = x2 + H Wd; g = swiglu: H =
    silu(r2 Wg) * (r2 Wu)), so A, G, U and D are never stored.
    """
    ext = {"b": b, "s": s, "t": s, "h": hid, "q": heads, "d": d, "e": d, "f": ffn}
    proj = {"b": 1, "s": s_blk, "t": s_blk, "h": h_blk, "q": q_blk, "d": 1}
    att = {"b": 1, "q": 1, "s": s_blk, "t": s_blk, "d": 1}
    ffb = {"b": 1, "s": s_blk, "h": h_blk, "f": f_blk}
    w = 0.02
    tens = [
        ("x", "bsh", "normal", "f32", 1.0, 0.0, proj),
        ("g1", "h", "normal", "bf16", w, 1.0, proj),
        ("Wq", "hqd", "normal", "bf16", w, 0.0, proj),
        ("Wk", "hqd", "normal", "bf16", w, 0.0, proj),
        ("Wv", "hqd", "normal", "bf16", w, 0.0, proj),
        ("Wo", "qdh", "normal", "bf16", w, 0.0, proj),
        ("g2", "h", "normal", "bf16", w, 1.0, ffb),
        ("Wg", "hf", "normal", "bf16", w, 0.0, ffb),
        ("Wu", "hf", "normal", "bf16", w, 0.0, ffb),
        ("Wd", "fh", "normal", "bf16", w, 0.0, ffb),
    ]
    inv_h = 1.0 / hid
    c = ("s", "t")
    chain = [
        Step("ss1", "bsh->bs", ["x"], "square", "sum", "f32", proj),
        Step("r1", "bsh,bs,h->bsh", ["x", "ss1", "g1"], "rms_scale", "none", "bf16", proj, beta=inv_h, eps=1e-6),
        Step("Qp", "bsh,hqd->bsqd", ["r1", "Wq"], "mul", "sum", "bf16", proj),
        Step("Kp", "bth,hqd->btqd", ["r1", "Wk"], "mul", "sum", "bf16", proj),
        Step("Vp", "bth,hqd->btqd", ["r1", "Wv"], "mul", "sum", "bf16", proj),
    ]
    if fused_attention:
        fa = dict(proj, e=1)
        chain += [Step("O", "bsqd,btqd,btqe->bsqe", ["Qp", "Kp", "Vp"], "attention", "softmax", "bf16", fa,
                       alpha=1.0 / math.sqrt(d), causal=c)]
    else:
        chain += [
            Relayout("Q", "Qp", "bqsd", att),
            Relayout("K", "Kp", "bqtd", att),
            Relayout("V", "Vp", "bqtd", att),
            Step("S", "bqsd,bqtd->bqst", ["Q", "K"], "mul", "sum", "f32", att, alpha=1.0 / math.sqrt(d), causal=c),
            Step("M", "bqst->bqs", ["S"], "ident", "max", "f32", att, causal=c),
            Step("L", "bqst,bqs->bqs", ["S", "M"], "exp_sub", "sum", "f32", att, causal=c),
            Step("P", "bqst,bqs,bqs->bqst", ["S", "M", "L"], "exp_sub_div", "none", "bf16", att, causal=c),
            Step("Oh", "bqst,bqtd->bqsd", ["P", "V"], "mul", "sum", "bf16", att, causal=c),
            Relayout("O", "Oh", "bsqd", proj),
        ]
    if fused_epilogues:
        chain += [
            Step("x2", "bsqd,qdh,bsh->bsh", ["O", "Wo", "x"], "mul_plus", "sum", "f32", proj),
            Step("ss2", "bsh->bs", ["x2"], "square", "sum", "f32", ffb),
            Step("r2", "bsh,bs,h->bsh", ["x2", "ss2", "g2"], "rms_scale", "none", "bf16", ffb, beta=inv_h, eps=1e-6),
            Step("H", "bsh,hf,hf->bsf", ["r2", "Wg", "Wu"], "swiglu", "sum", "bf16", ffb),
            Step("y", "bsf,fh,bsh->bsh", ["H", "Wd", "x2"], "mul_plus", "sum", "f32", ffb),
        ]
    else:
        chain += [
            Step("A", "bsqd,qdh->bsh", ["O", "Wo"], "mul", "sum", "f32", proj),
            Step("x2", "bsh,bsh->bsh", ["x", "A"], "add", "none", "f32", proj),
            Step("ss2", "bsh->bs", ["x2"], "square", "sum", "f32", ffb),
            Step("r2", "bsh,bs,h->bsh", ["x2", "ss2", "g2"], "rms_scale", "none", "bf16", ffb, beta=inv_h,
                 eps=1e-6),
            Step("G", "bsh,hf->bsf", ["r2", "Wg"], "mul", "sum", "f32", ffb),
            Step("U", "bsh,hf->bsf", ["r2", "Wu"], "mul", "sum", "f32", ffb),
            Step("H", "bsf,bsf->bsf", ["G", "U"], "silu_mul", "none", "bf16", ffb),
            Step("D", "bsf,fh->bsh", ["H", "Wd"], "mul", "sum", "f32", ffb),
            Step("y", "bsh,bsh->bsh", ["x2", "D"], "add", "none", "f32", ffb),
        ]
    name = f"llama7b_block_b{b}_s{s}_bf16_" + ("fused_attention" if fused_attention else "attention_chain")
    if fused_epilogues:
        name += "_fused_epilogues"
    return Workload(name=name, extents=ext, tensors=tens, chain=chain, seed=1004)


def multi_index(a=96, b=300, c=64, d=48, e=1000, blk=(5, 7, 4, 3, 6)) -> Workload:
    """'abcd,cde->abe' fp32 uniform[-1,1), padded tail blocks, SUM over c, d."""
    ext = dict(zip("abcde", (a, b, c, d, e)))
    bl = dict(zip("abcde", blk))
    return Workload(
        name=f"contract_abcd_cde_{a}x{b}x{c}x{d}x{e}_fp32_blk" + "".join(map(str, blk)), extents=ext,
        tensors=[("A", "abcd", "uniform", "f32", 1.0, 0.0, bl), ("B", "cde", "uniform", "f32", 1.0, 0.0, bl)],
        chain=[Step("C", "abcd,cde->abe", ["A", "B"], "mul", "sum", "f32", bl)], seed=1005)


# Matrix chains A-E ("Every Kernel Is a Join", Sec. 6, the second workload
# family): dimensions d_0 .. d_n (matrix M_i is d_(i-1) x d_i) and the printed
# parenthesization, as nested tuples of 1-based matrix numbers.
CHAINS = {
    # nine matrices, interior dimensions alternating 16384 and 6144, ends 10240
    "A": ([10240] + [16384, 6144] * 4 + [10240], (((1, 2), ((3, 4), ((5, 6), (7, 8)))), 9)),
    # five matrices, interior alternating 20480 and 5120, ends 9216
    "B": ([9216, 20480, 5120, 20480, 5120, 9216], ((1, 2), ((3, 4), 5))),
    # three matrices 10240 x 12288 x 32768 x 2048, right-associated
    "C": ([10240, 12288, 32768, 2048], (1, (2, 3))),
    # nine matrices: ends 24576, necks 1536, interior 20480
    "D": ([24576, 1536] + [20480] * 6 + [1536, 24576], ((1, (2, (3, (4, (5, (6, (7, 8))))))), 9)),
    # thirteen matrices: ends 49152, necks 1024, interior 20480
    "E": ([49152, 1024] + [20480] * 10 + [1024, 49152],
          ((1, (2, (3, (4, (5, (6, (7, (8, (9, (10, (11, 12))))))))))), 13)),
}
CHAIN_LETTERS = "abcdefghijklmnopqrstuvwxyz"


def chain_blocks(n: int) -> int:
    """Blocks per chain index: 4 where that leaves blocks that are multiples
    of 256, else 2 (the 1536-wide necks: 768-wide blocks)."""
    return 4 if n % 1024 == 0 else (2 if n % 512 == 0 else 1)


def matrix_chain(label: str) -> Workload:
    """Matrix chain `label` (A-E): M_1 ... M_n in bf16, every product a
    contraction 'xy,yz->xz' (bf16 output, fp32 accumulation) in the printed
    parenthesization.  Index i (between M_i and M_(i+1)) is letter i of the
    alphabet, blocked by chain_blocks.  M_1 ~ N(0, 1) and M_i ~ N(0, 1/d_(i-1))
    for i >= 2, so every partial product has entries of order one whatever
    the association."""
    dims, tree = CHAINS[label]
    n = len(dims) - 1
    L = CHAIN_LETTERS
    ext = {L[i]: dims[i] for i in range(n + 1)}
    blk = {L[i]: chain_blocks(dims[i]) for i in range(n + 1)}
    tens = []
    for i in range(1, n + 1):
        sigma = 1.0 if i == 1 else 1.0 / math.sqrt(dims[i - 1])
        tens.append((f"M{i}", L[i - 1] + L[i], "normal32", "bf16", sigma, 0.0, blk))
    chain = []

    def walk(t):
        """Appends the products of subtree t; returns (name, first, last)."""
        if isinstance(t, int):
            return f"M{t}", t, t
        (la, a0, a1), (rb, b0, b1) = walk(t[0]), walk(t[1])
        assert b0 == a1 + 1
        name = f"P{a0}_{b1}"
        spec = f"{L[a0 - 1]}{L[a1]},{L[a1]}{L[b1]}->{L[a0 - 1]}{L[b1]}"
        chain.append(Step(name, spec, [la, rb], "mul", "sum", "bf16", blk))
        return name, a0, b1

    walk(tree)
    return Workload(name=f"matrix_chain_{label}_{n}x_bf16", extents=ext, tensors=tens, chain=chain,
                    seed=1010 + "ABCDE".index(label) + 1)


def generate(w: Workload) -> dict:
    """Dense CPU tensors for every input of a workload, in recipe order."""
    gens = streams(w.seed, len(w.tensors))
    out = {}
    for gen, (name, letters, dist, dtype, sigma, mean, _) in zip(gens, w.tensors):
        shape = [w.extents[c] for c in letters]
        out[name] = draw(gen, shape, dist, dtype, sigma, mean)
    return out


def tensor_info(w: Workload, name: str):
    for t in w.tensors:
        if t[0] == name:
            return t
    raise KeyError(name)
