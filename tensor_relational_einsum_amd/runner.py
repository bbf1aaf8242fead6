"""Runs a workload chain (see ``inputs``) through the C ABI.

Builds every relation and workspace once, then ``run()`` issues one library
call per step on the context's stream; nothing is computed in Python.  By
default every einsum step is a prepared plan (jagg_plan_create at set-up:
host planning and join once; jagg_plan_run per step), and consecutive
einsum steps that do not read each other's outputs run as one plan group
(jagg_plan_group: contractions of one form share a launch), and a
sum-of-squares reduce followed by the RMS-scale map that reads it runs as
one fused plan (jagg_plan_fuse) where the pair has the form that allows it
(``fuse_norms``); ``units`` lists what one pass launches.  ``planned=False``
calls jagg_einsum for every step instead.
"""
from __future__ import annotations

import torch

from . import jagg
from .inputs import Relayout, Step, Workload


class ChainRunner:
    def __init__(self, ctx: jagg.Context, w: Workload, dense: dict, planned: bool = True, fuse_norms: bool = True):
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
        # units of one pass: (kind, object, step indices)
        self.units = []
        i = 0
        while i < len(self.calls):
            kind, obj, name = self.calls[i]
            if planned and fuse_norms and self._norm_pair(i):
                try:
                    fused = jagg.PlanFused(ctx, obj, self.calls[i + 1][1])
                except jagg.JaggError as e:
                    if e.status != -4:  # anything but "unsupported form" is an error
                        raise
                    fused = None
                if fused is not None:
                    self.units.append(("fused", fused, [i, i + 1]))
                    i += 2
                    continue
            j = i + 1
            if planned and kind == "einsum":
                written = {name}
                while j < len(self.calls) and self.calls[j][0] == "einsum":
                    ins = {n for n in w.chain[j].ins}
                    if ins & written or self.calls[j][2] in written:
                        break
                    written.add(self.calls[j][2])
                    j += 1
            if j - i > 1:
                self.units.append(("group", jagg.PlanGroup(ctx, [self.calls[k][1] for k in range(i, j)]),
                                   list(range(i, j))))
            else:
                self.units.append((kind, obj, [i]))
            i = j

    def _norm_pair(self, i: int) -> bool:
        """Steps i and i+1 are a sum of squares and the RMS-scale map that
        reads it together with the same input."""
        if i + 1 >= len(self.calls) or self.calls[i][0] != "einsum" or self.calls[i + 1][0] != "einsum":
            return False
        a, b = self.w.chain[i], self.w.chain[i + 1]
        return ((a.g, a.agg, b.g, b.agg) == ("square", "sum", "rms_scale", "none")
                and list(b.ins[:2]) == [a.ins[0], a.out])

    def run(self):
        for u in range(len(self.units)):
            self.run_unit(u)

    def run_unit(self, u: int):
        kind, obj, steps = self.units[u]
        if kind in ("group", "fused"):
            obj.run()
        else:
            self.run_step(steps[0])

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
