"""Full-size workloads checked from their original seeded inputs.

The LLaMA-7B-shaped block (4 x 2048 tokens, hidden 4096, 32 heads of 128,
SwiGLU 11008), recorded as one graph and replayed as bench.py times it: the
replayed outputs are compared on sampled token rows with the oracle's
evaluation of the whole block from x and the weights (every cast point
mirrored; tests/parity_util.llama_block_rows), so the rounding compounded
over the 4096- and 11008-deep bf16 contractions is inside the check.  Bar:
normwise error 2e-2 per compared relation (bf16 with fp32 accumulation).

The grouped-query causal attention (b4, 8 kv x 4 query heads, s 2048, d 128)
and the packed-sequence attention (b2, three sequences ending at 1024, 2560
and 4096) at the sizes bench.py reports, on sampled query rows (every
output column of a row), against the oracle's attention: 8e-3 normwise (one
bf16 rounding of the probabilities and one of the output).
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tensor_relational_einsum_amd import inputs as I
from tensor_relational_einsum_amd import jagg
from tensor_relational_einsum_amd.runner import ChainRunner
from parity_util import llama_block_rows, normwise_err, to_np

pytestmark = pytest.mark.gpu

CHAIN_TOL = 2e-2
ATT_TOL = 8e-3
# (batch index, token rows): first rows, both sides of the 128-token block
# edges, and the last rows of the sequence
LLAMA_ROWS = [(0, [0, 1, 127, 128, 1000, 2047]), (1, [64, 1111]), (2, [300]), (3, [5, 1500, 2046])]


@pytest.fixture(scope="module")
def sctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    s = torch.cuda.Stream()  # capture needs a stream other than the null stream
    with torch.cuda.stream(s):
        c = jagg.Context(0, s)
        yield c
        torch.cuda.synchronize()
        c.close()


@pytest.mark.parametrize("fused,epi", [(True, True), (True, False), (False, False)],
                         ids=["fused_attention_fused_epilogues", "fused_attention", "attention_chain"])
def test_llama_block_graph_rows_from_original_inputs(sctx, fused, epi):
    w = I.llama_block(fused_attention=fused, fused_epilogues=epi)
    dense = I.generate(w)
    want = {b: llama_block_rows(w, dense, b, rows) for b, rows in LLAMA_ROWS}
    with torch.cuda.stream(sctx.stream):
        run = ChainRunner(sctx, w, dense)
        run.run()
        torch.cuda.synchronize()
        graph = run.capture()
        for rep in range(2):
            for name in ("O", "x2", "y"):
                run.rel[name].data.fill_(float("nan"))
            graph.launch()
            torch.cuda.synchronize()
            got = {name: run.dense(name) for name in ("O", "x2", "y")}
            torch.cuda.synchronize()
            for b, rows in LLAMA_ROWS:
                for name in ("O", "x2", "y"):
                    g = to_np(got[name][b, rows])
                    err = normwise_err(g, want[b][name])
                    print(f"replay {rep} b{b} {name}: normwise error {err:.3e}")
                    assert err < CHAIN_TOL, f"replay {rep}, batch {b}, {name}: normwise error {err:.3e}"
        graph.close()


def sampled_attention_rows(ctx, w, rows, segments=None):
    """Runs a one-spec attention workload at full size and compares whole
    output rows (every column of the value letter) with the oracle."""
    dense = I.generate(w)
    run = ChainRunner(ctx, w, dense)
    st = w.chain[0]
    run.rel[st.out].data.fill_(float("nan"))
    run.run()
    torch.cuda.synchronize()
    out_l = st.spec.split("->")[1]
    got = to_np(run.dense(st.out))
    shp = [w.extents[c] for c in out_l]
    idx = np.concatenate([np.ravel_multi_index(tuple(r) + (np.arange(shp[-1]),), shp) for r in rows])
    xs = [to_np(dense[n]) for n in st.ins]
    want = O.round_to(O.attention_dense(st.spec, xs, w.extents, alpha=st.alpha, causal=st.causal, sample=idx,
                                        segments=segments), st.out_dtype)
    err = normwise_err(got.reshape(-1)[idx], want)
    print(f"{w.name}: {len(rows)} rows, normwise error {err:.3e}")
    assert err < ATT_TOL, f"normwise error {err:.3e}"
    assert not np.isnan(got).any(), "every output element must be written"


def test_gqa_causal_attention_full_size_rows(sctx):
    w = I.attention_gqa()
    B, G, R, S = (w.extents[c] for c in "bgrs")
    rng = np.random.default_rng(11)
    rows = [(int(rng.integers(B)), int(rng.integers(G)), int(rng.integers(R)), int(rng.integers(S)))
            for _ in range(20)]
    rows += [(0, 0, 0, 0), (B - 1, G - 1, R - 1, S - 1), (1, 3, 2, 127), (2, 5, 1, 128), (3, 7, 3, 2047)]
    with torch.cuda.stream(sctx.stream):
        sampled_attention_rows(sctx, w, rows)


def test_packed_sequence_attention_full_size_rows(sctx):
    w = I.attention_packed()
    B, G, R = (w.extents[c] for c in "bgr")
    ends = list(I.PACKED_ENDS)
    rng = np.random.default_rng(12)
    rows = [(int(rng.integers(B)), int(rng.integers(G)), int(rng.integers(R)), int(rng.integers(ends[-1])))
            for _ in range(16)]
    # first and last position of every sequence
    for q, e in enumerate(ends[1:]):
        rows += [(q % B, q % G, q % R, ends[q]), ((q + 1) % B, (q + 3) % G, (q + 1) % R, e - 1)]
    with torch.cuda.stream(sctx.stream):
        sampled_attention_rows(sctx, w, rows, segments=("s", "t", ends))
