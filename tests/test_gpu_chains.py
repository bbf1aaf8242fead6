"""Matrix chains A-E ("Every Kernel Is a Join", Sec. 6: the second workload
family, each multiply about 8192^3 scalar multiplies, in the printed
parenthesizations) on one GPU, through the C ABI.

Each product is a contraction 'xy,yz->xz' of bf16 relations (every index in
4 blocks, the 1536-wide necks in 2) with fp32 accumulation and a bf16
output.  Two checks per chain:

- every product on a grid of sampled rows and columns against the oracle fed
  the GPU's own stored operands (one bf16 rounding of an fp32-accumulated
  result: 8e-3 normwise);
- sampled rows of the chain's final product against the exact product of
  the original matrices, evaluated left to right in float64 (the HIP path
  rounds every partial product to bf16: 2e-2 normwise, the bar for bf16 with
  fp32 accumulation).
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tensor_relational_einsum_amd import inputs as I
from tensor_relational_einsum_amd import jagg
from tensor_relational_einsum_amd.runner import ChainRunner
from parity_util import normwise_err, to_np

pytestmark = pytest.mark.gpu

SPEC_TOL = 8e-3
CHAIN_TOL = 2e-2


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    c = jagg.Context(0)
    yield c
    torch.cuda.synchronize()
    c.close()


def pick(rng, n, k):
    """k sampled positions of [0, n) plus both ends."""
    return np.unique(np.concatenate([rng.integers(0, n, size=k), [0, n - 1]]))


@pytest.mark.parametrize("label", list("ABCDE"))
def test_matrix_chain(ctx, label):
    w = I.matrix_chain(label)
    dense = I.generate(w)
    run = ChainRunner(ctx, w, dense)
    for st in w.chain:
        run.rel[st.out].data.fill_(float("nan"))
    run.run()
    torch.cuda.synchronize()
    rng = np.random.default_rng(100 + ord(label))
    for st in w.chain:
        (la, lb), out = st.spec.split("->")[0].split(","), st.spec.split("->")[1]
        m, k, n = w.extents[la[0]], w.extents[la[1]], w.extents[lb[1]]
        rows, cols = pick(rng, m, 4), pick(rng, n, 46)
        a = to_np(run.dense(st.ins[0])[rows])
        b = to_np(run.dense(st.ins[1])[:, cols])
        y = to_np(run.dense(st.out)[rows][:, cols])
        want = O.round_to(O.dense("ij,jk->ik", [a, b], dict(i=rows.size, j=k, k=cols.size)), "bf16")
        err = normwise_err(y, want)
        print(f"chain {label} {st.out} ({m}x{k}x{n}): normwise error {err:.3e}")
        assert err < SPEC_TOL, f"{st.out}: normwise error {err:.3e}"
    # the final product from the original matrices, exact, left to right
    final = w.chain[-1].out
    n_mat = len(w.tensors)
    rows = pick(rng, w.extents[I.CHAIN_LETTERS[0]], 6)
    v = to_np(dense["M1"][rows])
    for i in range(2, n_mat + 1):
        lt = I.CHAIN_LETTERS
        v = O.contract("ij,jk->ik", v, to_np(dense[f"M{i}"]),
                       dict(i=rows.size, j=w.extents[lt[i - 1]], k=w.extents[lt[i]]))
    got = to_np(run.dense(final)[rows])
    assert not np.isnan(got).any()
    err = normwise_err(got, v)
    print(f"chain {label}: final rows against the exact product, normwise error {err:.3e}")
    assert err < CHAIN_TOL, f"chain {label}: normwise error {err:.3e}"
    del run
    torch.cuda.empty_cache()
