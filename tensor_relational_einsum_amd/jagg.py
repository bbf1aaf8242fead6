"""ctypes binding of libjagg.so (include/jagg.h): argument marshalling only.

PyTorch provides device memory and the stream; every step of a join-agg
spec runs in the library's HIP kernels.  There is no fallback: if the
library is missing or a call fails, a JaggError is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libjagg.so")

G = {"mul": 0, "ident": 1, "square": 2, "exp_sub": 3, "exp_sub_div": 4, "rms_scale": 5, "silu_mul": 6, "add": 7,
     "attention": 8, "mul_plus": 9, "swiglu": 10}
AGG = {"none": 0, "sum": 1, "max": 2, "softmax": 3}
DT = {"f32": 0, "bf16": 1}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
ESZ = {"f32": 4, "bf16": 2}
STATUS = {0: "ok", -1: "invalid argument", -2: "shape mismatch", -3: "bad blocking", -4: "unsupported spec",
          -5: "workspace too small", -6: "device error"}

NOALLOC_SCRATCH_BYTES = 32 << 20  # JAGG_NOALLOC_SCRATCH_BYTES in jagg.h

EXPORTS = ["jagg_ctx_create", "jagg_ctx_destroy", "jagg_relation_bytes", "jagg_relation_create",
           "jagg_relation_bytes_iv", "jagg_relation_create_iv", "jagg_relation_destroy", "jagg_repartition",
           "jagg_einsum_workspace", "jagg_einsum", "jagg_einsum_noalloc", "jagg_plan_create", "jagg_plan_run",
           "jagg_plan_destroy", "jagg_plan_group", "jagg_plan_fuse", "jagg_join_shape",
           "jagg_join_list", "jagg_capture_begin", "jagg_capture_end", "jagg_graph_launch", "jagg_graph_destroy",
           "jagg_status_str", "jagg_last_error"]


class JaggError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class jagg_spec(ctypes.Structure):
    _fields_ = [("einsum", ctypes.c_char_p), ("g", ctypes.c_int), ("agg", ctypes.c_int), ("out_dtype", ctypes.c_int),
                ("alpha", ctypes.c_float), ("beta", ctypes.c_float), ("eps", ctypes.c_float),
                ("causal_s", ctypes.c_char), ("causal_t", ctypes.c_char), ("seg_s", ctypes.c_char),
                ("seg_t", ctypes.c_char)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Loads libjagg.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise JaggError(-6, f"{_LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64p, i32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)
        L.jagg_ctx_create.argtypes = [ctypes.c_int, vp, ctypes.POINTER(vp)]
        L.jagg_ctx_destroy.argtypes = [vp]
        L.jagg_relation_bytes.argtypes = [ctypes.c_char_p, i64p, i32p, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
        L.jagg_relation_create.argtypes = [vp, ctypes.c_char_p, i64p, i32p, ctypes.c_int, vp, ctypes.c_size_t,
                                           ctypes.POINTER(vp)]
        i64pp = ctypes.POINTER(i64p)
        L.jagg_relation_bytes_iv.argtypes = [ctypes.c_char_p, i64p, i32p, i64pp, ctypes.c_int,
                                             ctypes.POINTER(ctypes.c_size_t)]
        L.jagg_relation_create_iv.argtypes = [vp, ctypes.c_char_p, i64p, i32p, i64pp, ctypes.c_int, vp,
                                              ctypes.c_size_t, ctypes.POINTER(vp)]
        L.jagg_relation_destroy.argtypes = [vp]
        L.jagg_repartition.argtypes = [vp, vp, vp]
        L.jagg_einsum_workspace.argtypes = [vp, ctypes.POINTER(jagg_spec), ctypes.POINTER(vp), ctypes.c_int, i32p,
                                            ctypes.POINTER(ctypes.c_size_t)]
        L.jagg_einsum.argtypes = [vp, ctypes.POINTER(jagg_spec), ctypes.POINTER(vp), ctypes.c_int, i32p, vp, vp,
                                  ctypes.c_size_t]
        L.jagg_einsum_noalloc.argtypes = [vp, ctypes.POINTER(jagg_spec), ctypes.POINTER(vp), ctypes.c_int, i32p, vp]
        L.jagg_plan_create.argtypes = [vp, ctypes.POINTER(jagg_spec), ctypes.POINTER(vp), ctypes.c_int, i32p, vp, vp,
                                       ctypes.c_size_t, ctypes.POINTER(vp)]
        L.jagg_plan_run.argtypes = [vp, vp]
        L.jagg_plan_destroy.argtypes = [vp]
        L.jagg_plan_group.argtypes = [vp, ctypes.c_int, ctypes.POINTER(vp), ctypes.POINTER(vp)]
        L.jagg_plan_fuse.argtypes = [vp, vp, vp, ctypes.POINTER(vp)]
        L.jagg_join_shape.argtypes = [ctypes.POINTER(jagg_spec), i64p, i32p, i64p, i64p]
        L.jagg_join_list.argtypes = [vp, ctypes.POINTER(jagg_spec), i64p, i32p, vp, vp]
        L.jagg_capture_begin.argtypes = [vp]
        L.jagg_capture_end.argtypes = [vp, ctypes.POINTER(vp)]
        L.jagg_graph_launch.argtypes = [vp, vp]
        L.jagg_graph_destroy.argtypes = [vp]
        L.jagg_status_str.argtypes = [ctypes.c_int]
        L.jagg_status_str.restype = ctypes.c_char_p
        L.jagg_last_error.argtypes = [vp]
        L.jagg_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _i64(vals):
    return (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])


def _i32(vals):
    return (ctypes.c_int32 * len(vals))(*[int(v) for v in vals])


def parse(einsum: str):
    lhs, out = einsum.split("->")
    ins = lhs.split(",")
    order = ""
    for lt in ins:
        for c in lt:
            if c not in order:
                order += c
    return ins, out, order


def make_spec(einsum, g="mul", agg="sum", out_dtype="f32", alpha=1.0, beta=0.0, eps=0.0, causal=None,
              segment=None) -> jagg_spec:
    s = jagg_spec()
    s._einsum_bytes = einsum.encode()  # keep the string alive with the struct
    s.einsum = s._einsum_bytes
    s.g, s.agg, s.out_dtype = G[g], AGG[agg], DT[out_dtype]
    s.alpha, s.beta, s.eps = alpha, beta, eps
    s.causal_s = causal[0].encode() if causal else b"\0"
    s.causal_t = causal[1].encode() if causal else b"\0"
    s.seg_s = segment[0].encode() if segment else b"\0"
    s.seg_t = segment[1].encode() if segment else b"\0"
    return s


class Context:
    """A jagg context bound to one device and one HIP stream (torch's current
    stream by default)."""

    def __init__(self, device: int = 0, stream: torch.cuda.Stream | None = None):
        self.device = device
        self.stream = stream if stream is not None else torch.cuda.current_stream(device)
        h = ctypes.c_void_p()
        self._check(lib().jagg_ctx_create(device, ctypes.c_void_p(self.stream.cuda_stream), ctypes.byref(h)), None)
        self.handle = h

    def _check(self, rc, h=...):
        if rc != 0:
            msg = lib().jagg_last_error(self.handle if h is ... else h)
            raise JaggError(rc, (msg or b"").decode())

    def close(self):
        if getattr(self, "handle", None):
            lib().jagg_ctx_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def block_count(b) -> int:
    """A blocking value is a block count or a list of interval bounds."""
    return len(b) - 1 if isinstance(b, (list, tuple)) else int(b)


def _bounds(blocks):
    """(count array, bounds pointer array, keep-alive) for per-letter blocking
    values; a NULL bounds pointer marks a uniformly blocked letter."""
    p64 = ctypes.POINTER(ctypes.c_int64)
    keep, ptrs = [], []
    for b in blocks:
        if isinstance(b, (list, tuple)):
            arr = _i64(b)
            keep.append(arr)
            ptrs.append(ctypes.cast(arr, p64))
        else:
            ptrs.append(p64())
    return _i32([block_count(b) for b in blocks]), (p64 * len(ptrs))(*ptrs), keep


def relation_bytes(letters, extents, nblocks, dtype) -> int:
    out = ctypes.c_size_t()
    counts, bnd, _keep = _bounds(nblocks)
    rc = lib().jagg_relation_bytes_iv(letters.encode(), _i64(extents), counts, bnd, DT[dtype], ctypes.byref(out))
    if rc != 0:
        raise JaggError(rc, f"relation {letters} {list(extents)} / {list(nblocks)}")
    return out.value


class Relation:
    """Tensor relation over a flat torch device buffer (padded blocks in
    canonical tuple order).  ``extents`` / ``nblocks`` follow ``letters``; an
    entry of ``nblocks`` is a block count or a list of interval bounds."""

    def __init__(self, ctx: Context, letters: str, extents, nblocks, dtype: str, buffer: torch.Tensor | None = None,
                 zeroed: bool = False):
        self.ctx, self.letters, self.dtype = ctx, letters, dtype
        self.extents = [int(v) for v in extents]
        self.bounds = [[int(x) for x in b] if isinstance(b, (list, tuple)) else None for b in nblocks]
        self.nblocks = [block_count(b) for b in nblocks]
        nbytes = relation_bytes(letters, self.extents, self._blocks(), dtype)
        if buffer is None:
            alloc = torch.zeros if zeroed else torch.empty
            buffer = alloc(nbytes // ESZ[dtype], dtype=TORCH_DT[dtype], device=f"cuda:{ctx.device}")
        self.data = buffer
        self.nbytes = nbytes
        h = ctypes.c_void_p()
        counts, bnd, _keep = _bounds(self._blocks())
        ctx._check(lib().jagg_relation_create_iv(ctx.handle, letters.encode(), _i64(self.extents), counts, bnd,
                                                 DT[dtype], ctypes.c_void_p(buffer.data_ptr()),
                                                 buffer.numel() * buffer.element_size(), ctypes.byref(h)))
        self.handle = h

    def _blocks(self):
        return [b if b is not None else k for b, k in zip(self.bounds, self.nblocks)]

    def blocking(self) -> dict:
        return dict(zip(self.letters, self._blocks()))

    def __del__(self):
        try:
            if getattr(self, "handle", None):
                lib().jagg_relation_destroy(self.handle)
                self.handle = None
        except Exception:
            pass


class Graph:
    """A recorded chain of calls on one context (jagg_capture_begin ..
    jagg_capture_end); launch() replays it on the context's stream.  The
    relations and workspaces the recorded calls used must stay alive."""

    def __init__(self, ctx: Context, handle):
        self.ctx, self.handle = ctx, handle

    def launch(self):
        self.ctx._check(lib().jagg_graph_launch(self.ctx.handle, self.handle))

    def close(self):
        if getattr(self, "handle", None):
            lib().jagg_graph_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def capture(ctx: Context, record) -> Graph:
    """Records every call `record()` makes on `ctx` into a graph."""
    ctx._check(lib().jagg_capture_begin(ctx.handle))
    try:
        record()
    finally:
        h = ctypes.c_void_p()
        rc = lib().jagg_capture_end(ctx.handle, ctypes.byref(h))
    ctx._check(rc)
    return Graph(ctx, h)


def repartition(ctx: Context, src: Relation, dst: Relation) -> Relation:
    ctx._check(lib().jagg_repartition(ctx.handle, src.handle, dst.handle))
    return dst


def relation_like(ctx, letters, extents: dict, blockings: dict, dtype) -> Relation:
    return Relation(ctx, letters, [extents[c] for c in letters], [blockings.get(c, 1) for c in letters], dtype)


def from_dense(ctx: Context, x: torch.Tensor, letters: str, blockings: dict) -> Relation:
    """Device tensor (row-major over `letters`) -> blocked relation, through the
    repartition kernel (a dense tensor is a relation with one block per letter)."""
    dtype = {torch.float32: "f32", torch.bfloat16: "bf16"}[x.dtype]
    x = x.contiguous()
    dense = Relation(ctx, letters, list(x.shape), [1] * len(letters), dtype, buffer=x.view(-1))
    out = Relation(ctx, letters, list(x.shape), [blockings.get(c, 1) for c in letters], dtype)
    repartition(ctx, dense, out)
    out._keep = x
    return out


def to_dense(ctx: Context, rel: Relation) -> torch.Tensor:
    """Blocked relation -> dense device tensor, through the repartition kernel."""
    buf = torch.empty(int(torch.tensor(rel.extents).prod().item()), dtype=TORCH_DT[rel.dtype],
                      device=rel.data.device)
    dense = Relation(ctx, rel.letters, rel.extents, [1] * len(rel.letters), rel.dtype, buffer=buf)
    repartition(ctx, rel, dense)
    return buf.view(*rel.extents)


class EinsumCall:
    """One join-agg spec bound to its relations, with arguments marshalled
    once; ``run()`` is a single call into the library."""

    def __init__(self, ctx: Context, einsum: str, inputs, blockings: dict, out: Relation | None = None, g="mul",
                 agg="sum", out_dtype="f32", alpha=1.0, beta=0.0, eps=0.0, causal=None,
                 workspace: torch.Tensor | None = None, segment=None):
        ins, out_letters, order = parse(einsum)
        self.ctx, self.einsum = ctx, einsum
        self.spec = make_spec(einsum, g, agg, out_dtype, alpha, beta, eps, causal, segment)
        self.inputs = list(inputs)
        self.blk = _i32([block_count(blockings.get(c, 1)) for c in order])
        self.in_arr = (ctypes.c_void_p * len(self.inputs))(*[r.handle.value for r in self.inputs])
        if out is None:
            ext = {}
            for lt, r in zip(ins, self.inputs):
                for c, n in zip(lt, r.extents):
                    ext[c] = n
            # under a causal pair on two output letters the tuples above the
            # block diagonal are absent and never written: clear them once
            absent = causal is not None and causal[0] in out_letters and causal[1] in out_letters
            out = Relation(ctx, out_letters, [ext[c] for c in out_letters], [blockings.get(c, 1) for c in out_letters],
                           out_dtype, zeroed=absent)
        self.out = out
        need = ctypes.c_size_t()
        ctx._check(lib().jagg_einsum_workspace(ctx.handle, ctypes.byref(self.spec), self.in_arr, len(self.inputs),
                                               self.blk, ctypes.byref(need)))
        self.ws_bytes = need.value
        if workspace is None or workspace.numel() < need.value:
            workspace = torch.empty(max(need.value, 256), dtype=torch.uint8, device=f"cuda:{ctx.device}")
        self.workspace = workspace

    def run(self) -> Relation:
        self.ctx._check(lib().jagg_einsum(self.ctx.handle, ctypes.byref(self.spec), self.in_arr, len(self.inputs),
                                          self.blk, self.out.handle, ctypes.c_void_p(self.workspace.data_ptr()),
                                          self.workspace.numel()))
        return self.out

    def prepare(self) -> "EinsumCall":
        """Plans the call once (jagg_plan_create: the host planning and the
        join, into a workspace of the plan's own); run_plan() then launches
        the block kernel only."""
        if getattr(self, "plan", None) is None:
            self.plan_ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=f"cuda:{self.ctx.device}")
            h = ctypes.c_void_p()
            self.ctx._check(lib().jagg_plan_create(self.ctx.handle, ctypes.byref(self.spec), self.in_arr,
                                                   len(self.inputs), self.blk, self.out.handle,
                                                   ctypes.c_void_p(self.plan_ws.data_ptr()), self.plan_ws.numel(),
                                                   ctypes.byref(h)))
            self.plan = h
        return self

    def run_plan(self) -> Relation:
        self.ctx._check(lib().jagg_plan_run(self.ctx.handle, self.plan))
        return self.out

    def __del__(self):
        try:
            if getattr(self, "plan", None):
                lib().jagg_plan_destroy(self.plan)
                self.plan = None
        except Exception:
            pass

    def run_noalloc(self, out: Relation | None = None) -> Relation:
        """The same spec through jagg_einsum_noalloc (the library's static
        device scratch instead of this call's workspace)."""
        out = out if out is not None else self.out
        self.ctx._check(lib().jagg_einsum_noalloc(self.ctx.handle, ctypes.byref(self.spec), self.in_arr,
                                                  len(self.inputs), self.blk, out.handle))
        return out


class PlanGroup:
    """Independent prepared calls run as one unit (jagg_plan_group): members
    of one contraction form share a launch.  The calls (and their relations
    and workspaces) must stay alive."""

    def __init__(self, ctx: Context, calls):
        # prepared calls, or fused pairs (PlanFused), which are plans already
        self.ctx, self.calls = ctx, [c if isinstance(c, PlanFused) else c.prepare() for c in calls]
        arr = (ctypes.c_void_p * len(self.calls))(
            *[c.handle.value if isinstance(c, PlanFused) else c.plan.value for c in self.calls])
        h = ctypes.c_void_p()
        ctx._check(lib().jagg_plan_group(ctx.handle, len(self.calls), arr, ctypes.byref(h)))
        self.handle = h

    def run(self):
        self.ctx._check(lib().jagg_plan_run(self.ctx.handle, self.handle))

    def __del__(self):
        try:
            if getattr(self, "handle", None):
                lib().jagg_plan_destroy(self.handle)
                self.handle = None
        except Exception:
            pass


class PlanFused:
    """A sum-of-squares reduce and the RMS-scale map that reads it, run as
    one pass (jagg_plan_fuse).  Raises JaggError (status -4, unsupported)
    when the pair does not have that form.  The calls (and their relations
    and workspaces) must stay alive."""

    def __init__(self, ctx: Context, first: "EinsumCall", second: "EinsumCall"):
        self.ctx, self.calls = ctx, [first.prepare(), second.prepare()]
        h = ctypes.c_void_p()
        ctx._check(lib().jagg_plan_fuse(ctx.handle, first.plan, second.plan, ctypes.byref(h)))
        self.handle = h

    def run(self):
        self.ctx._check(lib().jagg_plan_run(self.ctx.handle, self.handle))

    def __del__(self):
        try:
            if getattr(self, "handle", None):
                lib().jagg_plan_destroy(self.handle)
                self.handle = None
        except Exception:
            pass


def einsum(ctx: Context, einsum: str, inputs, blockings: dict, out: Relation | None = None, **kw) -> Relation:
    return EinsumCall(ctx, einsum, inputs, blockings, out, **kw).run()


def join_shape(einsum: str, extents: dict, blockings: dict, causal=None):
    _, _, order = parse(einsum)
    spec = make_spec(einsum, causal=causal)
    nk, pk = ctypes.c_int64(), ctypes.c_int64()
    rc = lib().jagg_join_shape(ctypes.byref(spec), _i64([extents[c] for c in order]),
                               _i32([blockings.get(c, 1) for c in order]), ctypes.byref(nk), ctypes.byref(pk))
    if rc != 0:
        raise JaggError(rc, f"join shape of {einsum}")
    return nk.value, pk.value


def join_list(ctx: Context, einsum: str, extents: dict, blockings: dict, causal=None):
    """Runs the join-enumeration kernel; returns (list [n_keys, per_key, 1+n_in],
    counts [n_keys]) as int32 device tensors."""
    ins, _, order = parse(einsum)
    nk, pk = join_shape(einsum, extents, blockings, causal)
    spec = make_spec(einsum, causal=causal)
    dev = f"cuda:{ctx.device}"
    lst = torch.empty((nk, pk, 1 + len(ins)), dtype=torch.int32, device=dev)
    cnt = torch.empty(nk, dtype=torch.int32, device=dev)
    ctx._check(lib().jagg_join_list(ctx.handle, ctypes.byref(spec), _i64([extents[c] for c in order]),
                                    _i32([blockings.get(c, 1) for c in order]), ctypes.c_void_p(lst.data_ptr()),
                                    ctypes.c_void_p(cnt.data_ptr())))
    return lst, cnt
