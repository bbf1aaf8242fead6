"""Runs a workload chain (see ``inputs``) through the C ABI.

Builds every relation and workspace once, then ``run()`` issues one library
call per step on the context's stream; nothing is computed in Python.  By
default every einsum step is a prepared plan (jagg_plan_create at set-up:
host planning and join once; jagg_plan_run per step); ``planned=False``
calls jagg_einsum every time instead.
"""
from __future__ import annotations

import torch

from . import jagg
from .inputs import Relayout, Step, Workload


class ChainRunner:
    def __init__(self, ctx: jagg.Context, w: Workload, dense: dict, planned: bool = True):
        self.ctx, self.w, self.planned = ctx, w, planned
        dev = f"cuda:{ctx.device}"
        self.rel: dict[str, jagg.Relation] = {}
        self.dense_dev = {}
        for name, letters, _dist, _dt, _s, _m, blk in w.tensors:
            x = dense[name].to(dev)
            self.dense_dev[name] = x
            self.rel[name] = jagg.from_dense(ctx, x, letters, blk)
        self.calls = []  # (kind, object, name)
        ws = None
        for st in w.chain:
            if isinstance(st, Step):
                ins = [self.rel[n] for n in st.ins]
                call = jagg.EinsumCall(ctx, st.spec, ins, st.blockings, g=st.g, agg=st.agg, out_dtype=st.out_dtype,
                                       alpha=st.alpha, beta=st.beta, eps=st.eps, causal=st.causal, workspace=ws,
                                       segment=st.segment)
                if ws is None or call.workspace.numel() > ws.numel():
                    ws = call.workspace
                self.rel[st.out] = call.out
                self.calls.append(("einsum", call, st.out))
            elif isinstance(st, Relayout):
                src = self.rel[st.src]
                dst = jagg.relation_like(ctx, st.letters, dict(zip(src.letters, src.extents)), st.blockings,
                                         src.dtype)
                self.rel[st.out] = dst
                self.calls.append(("relayout", (src, dst), st.out))
            else:
                raise TypeError(st)
        # every einsum shares the largest workspace (calls run in stream order)
        for kind, obj, _ in self.calls:
            if kind == "einsum" and obj.workspace.numel() < ws.numel():
                obj.workspace = ws
        self.workspace = ws
        if planned:
            for kind, obj, _ in self.calls:
                if kind == "einsum":
                    obj.prepare()

    def run(self):
        for i in range(len(self.calls)):
            self.run_step(i)

    def capture(self) -> jagg.Graph:
        """The whole chain recorded into one graph (every buffer it uses is
        already allocated, so replays repeat the same launches)."""
        return jagg.capture(self.ctx, self.run)

    def run_step(self, i: int):
        kind, obj, _ = self.calls[i]
        if kind == "einsum":
            if self.planned:
                obj.run_plan()
            else:
                obj.run()
        else:
            jagg.repartition(self.ctx, obj[0], obj[1])

    def dense(self, name: str) -> torch.Tensor:
        return jagg.to_dense(self.ctx, self.rel[name])
