"""Graph capture of a call chain (jagg_capture_begin / jagg_capture_end /
jagg_graph_launch), through the C ABI.

"Every Kernel Is a Join" (Ding et al.), Sec. 5.1: the executable artifact is
a graph of GPU kernels; "Stax (5): Caching and Measurement", Section 11.3:
replaying a recorded graph removes the per-launch host cost.  Every kernel
of the path is deterministic (no atomics), so a replay must reproduce the
eager results bit for bit.  Each test replays several times, with eager work
and synchronisations between the replays, and checks every replay: bit for
bit against the eager run, and against the oracle's evaluation of the chain
from the original inputs (normwise error under the chain's tolerance: 1e-5
for an fp32 chain, 2e-2 for a bf16 chain with fp32 accumulation, 8e-3 for
one fused attention spec with a bf16 output).
"""
import numpy as np
import pytest
import torch

from tensor_relational_einsum_amd import inputs as I
from tensor_relational_einsum_amd import jagg
from tensor_relational_einsum_amd.runner import ChainRunner
from parity_util import normwise_err, oracle_chain, rel_dense

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    s = torch.cuda.Stream()  # capture needs a stream other than the null stream
    with torch.cuda.stream(s):
        c = jagg.Context(0, s)
        yield c
        torch.cuda.synchronize()
        c.close()


def check_chain_graph(ctx, w, outs, tol, reps=3):
    with torch.cuda.stream(ctx.stream):
        dense = I.generate(w)
        ref = oracle_chain(w, dense)
        run = ChainRunner(ctx, w, dense)
        run.run()
        torch.cuda.synchronize()
        want = {o: run.dense(o).clone() for o in outs}
        g = run.capture()
        for rep in range(reps):
            for o in outs:
                run.rel[o].data.fill_(7)
            g.launch()
            torch.cuda.synchronize()
            for o in outs:
                got = run.dense(o)
                assert torch.equal(got, want[o]), f"replay {rep}: {o} differs from the eager run"
                err = normwise_err(rel_dense(run.rel[o], w.extents), ref[o])
                assert err < tol, f"replay {rep}: {o} normwise error {err:.3e} against the oracle"
            # eager work between the replays, checked as well
            run.run()
            torch.cuda.synchronize()
            for o in outs:
                assert torch.equal(run.dense(o), want[o]), f"eager run after replay {rep}: {o} differs"
        g.close()


def test_graph_llama_block_small(sctx):
    w = I.llama_block(b=1, s=256, hid=512, heads=4, d=128, ffn=1376, s_blk=2, h_blk=4, q_blk=2, f_blk=8,
                      fused_attention=True)
    check_chain_graph(sctx, w, ["Qp", "O", "G", "y"], 2e-2)


def test_graph_attention_chain_with_relayouts(sctx):
    w = I.attention_chain(b=1, h=2, s=256, d=64, nb=4)
    check_chain_graph(sctx, w, [st.out for st in w.chain][-1:], 2e-2)


def test_graph_matmul_config(sctx):
    w = I.matmul_256()
    check_chain_graph(sctx, w, ["C"], 1e-5, reps=4)


def test_graph_capture_errors(sctx):
    h = jagg.ctypes.c_void_p()
    with pytest.raises(jagg.JaggError):  # end without a begin
        sctx._check(jagg.lib().jagg_capture_end(sctx.handle, jagg.ctypes.byref(h)))
    sctx._check(jagg.lib().jagg_capture_begin(sctx.handle))
    with pytest.raises(jagg.JaggError):  # a second begin on a capturing context
        sctx._check(jagg.lib().jagg_capture_begin(sctx.handle))
    sctx._check(jagg.lib().jagg_capture_end(sctx.handle, jagg.ctypes.byref(h)))  # an empty graph is fine
    jagg.Graph(sctx, h).close()


def test_graph_packed_attention_with_interval_relayouts(sctx):
    """Packed-sequence GQA attention (segment pair over interval-blocked s and
    t) and the interval relayouts around it, recorded and replayed."""
    w = I.attention_packed(b=1, kv=2, group=2, ends=(0, 100, 356, 512), d=64)
    with torch.cuda.stream(sctx.stream):
        dense = I.generate(w)
        run = ChainRunner(sctx, w, dense)
        q = run.rel["Q"]
        uni = jagg.relation_like(sctx, q.letters, dict(zip(q.letters, q.extents)), dict(s=4), q.dtype)
        back = jagg.relation_like(sctx, q.letters, dict(zip(q.letters, q.extents)), q.blocking(), q.dtype)

        def chain():
            run.run()
            jagg.repartition(sctx, q, uni)
            jagg.repartition(sctx, uni, back)

        chain()
        torch.cuda.synchronize()
        want_o, want_b = run.rel["O"].data.clone(), back.data.clone()
        assert torch.equal(want_b, q.data)
        ref = oracle_chain(w, dense)["O"]
        g = jagg.capture(sctx, chain)
        for rep in range(3):
            run.rel["O"].data.fill_(7)
            back.data.fill_(7)
            g.launch()
            torch.cuda.synchronize()
            assert torch.equal(run.rel["O"].data, want_o), f"replay {rep}: attention output differs"
            err = normwise_err(rel_dense(run.rel["O"], w.extents), ref)
            assert err < 8e-3, f"replay {rep}: attention normwise error {err:.3e} against the oracle"
            assert torch.equal(back.data, want_b), f"replay {rep}: interval relayout round trip differs"
            chain()
            torch.cuda.synchronize()
            assert torch.equal(run.rel["O"].data, want_o)
        g.close()
