"""The row-sampled evaluation of the LLaMA-shaped block (parity_util.
llama_block_rows) against the oracle's evaluation of the whole chain, on a
small block: both attention forms, rows at the first position, at block
edges and at the last position.  The sampled form must give the very rows
of the full evaluation (same cast points), up to float64 summation order
before the final rounding."""
import numpy as np
import pytest

from tensor_relational_einsum_amd import inputs as I
from parity_util import llama_block_rows, oracle_chain


@pytest.mark.parametrize("fused,epi", [(True, False), (False, False), (True, True)])
def test_block_rows_equal_full_chain(fused, epi):
    w = I.llama_block(b=2, s=48, hid=256, heads=2, d=128, ffn=320, s_blk=3, h_blk=2, q_blk=2, f_blk=2,
                      fused_attention=fused, fused_epilogues=epi)
    dense = I.generate(w)
    full = oracle_chain(w, dense)
    for b, rows in ((0, [0, 1, 15, 16, 47]), (1, [7, 30])):
        got = llama_block_rows(w, dense, b, rows)
        o_full = full["O"][b] if fused else full["Oh"][b].transpose(1, 0, 2)
        for name, ref in (("O", o_full[rows]), ("x2", full["x2"][b, rows]), ("y", full["y"][b, rows])):
            err = np.max(np.abs(got[name] - ref)) / np.max(np.abs(ref))
            # identical cast points: any difference is a float64 summation
            # order moving a final rounding by one unit of its dtype
            assert err < 2 ** -7, f"{name}: {err:.3e}"
            assert np.mean(got[name] != ref) < 0.01, f"{name}: too many rounding differences"
