"""Python face of the CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this module.  The product
library never loads it, and it imports nothing from the product package.

Every routine computes in IEEE double; see ``oracle.c`` for which passage of
"Every Kernel Is a Join" (Ding et al.) each part follows.  Values are passed
as numpy arrays: dense tensors are row-major in their operand's letter order,
relations are flat buffers of padded blocks in canonical tuple order.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# the oracle's own names for g and the aggregation; mapped to its C enums
G_CODES = {"mul": 0, "ident": 1, "square": 2, "exp_sub": 3, "exp_sub_div": 4,
           "rms_scale": 5, "silu_mul": 6, "add": 7}
AGG_CODES = {"none": 0, "sum": 1, "max": 2}
DTYPE_CODES = {"f32": 0, "bf16": 1}


class OracleError(RuntimeError):
    pass


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with the host C compiler."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        i64p = ctypes.POINTER(ctypes.c_int64)
        i32p = ctypes.POINTER(ctypes.c_int32)
        dpp = ctypes.POINTER(ctypes.c_void_p)
        lib.oracle_dense.argtypes = [ctypes.c_char_p, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                     ctypes.c_double, ctypes.c_double, ctypes.c_int, ctypes.c_int,
                                     i64p, dpp, i64p, ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_relational_iv.argtypes = [ctypes.c_char_p, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                             ctypes.c_double, ctypes.c_double, ctypes.c_int, ctypes.c_int,
                                             i64p, i32p, i64p, dpp, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_join_list_iv.argtypes = [ctypes.c_char_p, i64p, i32p, i64p, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_void_p, ctypes.c_int64, i64p]
        lib.oracle_relation_elems.argtypes = [ctypes.c_char_p, i64p, i32p, i64p]
        lib.oracle_to_relation.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_char_p, i64p, i32p,
                                           ctypes.c_void_p]
        lib.oracle_from_relation.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_char_p, i64p, i32p,
                                             ctypes.c_void_p]
        lib.oracle_repartition.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_char_p, i32p,
                                           ctypes.c_void_p, ctypes.c_char_p, i32p, i64p]
        lib.oracle_block_shape.argtypes = [ctypes.c_char_p, i64p, i32p, i64p]
        lib.oracle_relation_elems_iv.argtypes = [ctypes.c_char_p, i64p, i32p, i64p, i64p]
        lib.oracle_to_relation_iv.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_char_p, i64p, i32p, i64p,
                                              ctypes.c_void_p]
        lib.oracle_from_relation_iv.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_char_p, i64p, i32p, i64p,
                                                ctypes.c_void_p]
        lib.oracle_repartition_iv.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_char_p, i32p, i64p,
                                              ctypes.c_void_p, ctypes.c_char_p, i32p, i64p, i64p]
        lib.oracle_block_shape_iv.argtypes = [ctypes.c_char_p, i64p, i32p, i64p, i64p]
        lib.oracle_attention_dense.argtypes = [ctypes.c_char_p, ctypes.c_double, ctypes.c_int, ctypes.c_int, i64p,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, i64p,
                                               ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_attention_relational_seg.argtypes = [ctypes.c_char_p, ctypes.c_double, ctypes.c_int,
                                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, i64p, i32p, i64p,
                                                        dpp, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_attention_dense_seg.argtypes = [ctypes.c_char_p, ctypes.c_double, ctypes.c_int, ctypes.c_int,
                                                   ctypes.c_int, ctypes.c_int, i64p, ctypes.c_int, i64p,
                                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, i64p,
                                                   ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_softmax_merge.argtypes = [ctypes.c_double] * 6 + [ctypes.c_void_p]
        lib.oracle_softmax_merge.restype = None
        lib.oracle_dense_recompose.argtypes = [ctypes.c_char_p, ctypes.c_int, ctypes.c_double, i64p, dpp, i64p,
                                               ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_round.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
        lib.oracle_round.restype = None
        _lib = lib
    return _lib


def _ext26(extents: dict) -> np.ndarray:
    a = np.zeros(26, dtype=np.int64)
    for k, v in extents.items():
        a[ord(k) - 97] = int(v)
    return a


MAX_INTERVALS = 64  # ORIV in oracle.c


def _nblk26(blockings: dict) -> np.ndarray:
    """Block count per letter.  A blocking value is a count (uniform blocks)
    or a list of interval bounds [0, b_1, ..., n] (k = len - 1 blocks)."""
    a = np.ones(26, dtype=np.int32)
    for k, v in blockings.items():
        a[ord(k) - 97] = len(v) - 1 if isinstance(v, (list, tuple)) else int(v)
    return a


def _bnd26(blockings: dict) -> np.ndarray:
    """26 rows of MAX_INTERVALS+1 bounds; a row starting with -1 is uniform."""
    a = np.full((26, MAX_INTERVALS + 1), -1, dtype=np.int64)
    for k, v in blockings.items():
        if isinstance(v, (list, tuple)):
            if len(v) - 1 > MAX_INTERVALS:
                raise OracleError(f"letter {k}: more than {MAX_INTERVALS} intervals")
            a[ord(k) - 97, :len(v)] = [int(b) for b in v]
    return a


def _has_iv(blockings: dict) -> bool:
    return any(isinstance(v, (list, tuple)) for v in blockings.values())


def _i64p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _i32p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _causal(causal):
    if causal is None:
        return -1, -1
    s, t = causal
    return ord(s) - 97, ord(t) - 97


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} failed with status {rc}")


def _parse(spec: str):
    if spec.count("->") != 1:
        raise OracleError(f"malformed spec {spec!r}")
    lhs, out = spec.split("->")
    return lhs.split(","), out


def dense(spec, inputs, extents, g="mul", agg="sum", alpha=1.0, beta=0.0, eps=0.0,
          causal=None, sample=None):
    """Dense form: out[o] = alpha * AGG_r g(in_1, ..., in_n), unrounded (float64).

    ``sample`` is an optional array of row-major flat output indices; then only
    those outputs are computed and a 1-D array is returned.
    """
    lib = _load()
    ins, out_letters = _parse(spec)
    arrs = []
    for lt, x in zip(ins, inputs):
        x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
        want = tuple(int(extents.get(c, -1)) for c in lt)
        if x.shape != want:
            raise OracleError(f"input {lt} has shape {x.shape}, expected {want}")
        arrs.append(x)
    ptrs = (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    ext = _ext26(extents)
    cs, ct = _causal(causal)
    if sample is None:
        shape = tuple(max(0, int(extents.get(c, 0))) for c in out_letters)
        out = np.zeros(shape, dtype=np.float64)
        rc = lib.oracle_dense(spec.encode(), G_CODES[g], AGG_CODES[agg], alpha, beta, eps, cs, ct,
                              _i64p(ext), ptrs, None, 0, out.ctypes.data)
    else:
        idx = np.ascontiguousarray(np.asarray(sample, dtype=np.int64))
        out = np.zeros(idx.shape[0], dtype=np.float64)
        rc = lib.oracle_dense(spec.encode(), G_CODES[g], AGG_CODES[agg], alpha, beta, eps, cs, ct,
                              _i64p(ext), ptrs, _i64p(idx), idx.shape[0], out.ctypes.data)
    _check(rc, "oracle_dense")
    return out


def relation_elems(letters, extents, blockings) -> int:
    lib = _load()
    n = np.zeros(1, dtype=np.int64)
    ext, nb, bd = _ext26(extents), _nblk26(blockings), _bnd26(blockings)
    _check(lib.oracle_relation_elems_iv(letters.encode(), _i64p(ext), _i32p(nb), _i64p(bd), _i64p(n)),
           "relation_elems")
    return int(n[0])


def block_shape(letters, extents, blockings):
    """Padded block extents, in the relation's letter order."""
    lib = _load()
    e = np.zeros(max(1, len(letters)), dtype=np.int64)
    ext, nb, bd = _ext26(extents), _nblk26(blockings), _bnd26(blockings)
    _check(lib.oracle_block_shape_iv(letters.encode(), _i64p(ext), _i32p(nb), _i64p(bd), _i64p(e)), "block_shape")
    return tuple(int(v) for v in e[:len(letters)])


def to_relation(x, letters, extents, blockings):
    """Dense row-major array (any fixed-size dtype) -> relation buffer, padding +0."""
    lib = _load()
    x = np.ascontiguousarray(x)
    n = relation_elems(letters, extents, blockings)
    out = np.zeros(n, dtype=x.dtype)
    ext, nb, bd = _ext26(extents), _nblk26(blockings), _bnd26(blockings)
    _check(lib.oracle_to_relation_iv(x.ctypes.data, x.dtype.itemsize, letters.encode(), _i64p(ext), _i32p(nb),
                                     _i64p(bd), out.ctypes.data), "to_relation")
    return out


def from_relation(rel, letters, extents, blockings):
    """Relation buffer -> dense row-major array (padding dropped)."""
    lib = _load()
    rel = np.ascontiguousarray(rel)
    shape = tuple(int(extents[c]) for c in letters)
    out = np.zeros(shape, dtype=rel.dtype)
    ext, nb, bd = _ext26(extents), _nblk26(blockings), _bnd26(blockings)
    _check(lib.oracle_from_relation_iv(rel.ctypes.data, rel.dtype.itemsize, letters.encode(), _i64p(ext),
                                       _i32p(nb), _i64p(bd), out.ctypes.data), "from_relation")
    return out


def repartition(src, src_letters, src_blockings, dst_letters, dst_blockings, extents):
    """Densify, then re-block in the destination letter order (bytewise exact)."""
    lib = _load()
    src = np.ascontiguousarray(src)
    n = relation_elems(dst_letters, extents, dst_blockings)
    dst = np.zeros(n, dtype=src.dtype)
    ext = _ext26(extents)
    sb, db = _nblk26(src_blockings), _nblk26(dst_blockings)
    sv, dv = _bnd26(src_blockings), _bnd26(dst_blockings)
    _check(lib.oracle_repartition_iv(src.ctypes.data, src.dtype.itemsize, src_letters.encode(), _i32p(sb),
                                     _i64p(sv), dst.ctypes.data, dst_letters.encode(), _i32p(db), _i64p(dv),
                                     _i64p(ext)), "repartition")
    return dst


def join_list(spec, extents, blockings, causal=None):
    """Canonical join list: int64 array [n_entries, 1 + n_in] of [out_id, in_ids...]."""
    lib = _load()
    ins, _ = _parse(spec)
    ext, nb, bd = _ext26(extents), _nblk26(blockings), _bnd26(blockings)
    cs, ct = _causal(causal)
    n = np.zeros(1, dtype=np.int64)
    _check(lib.oracle_join_list_iv(spec.encode(), _i64p(ext), _i32p(nb), _i64p(bd), cs, ct, None, 0, _i64p(n)),
           "join_list")
    lst = np.zeros((int(n[0]), 1 + len(ins)), dtype=np.int64)
    _check(lib.oracle_join_list_iv(spec.encode(), _i64p(ext), _i32p(nb), _i64p(bd), cs, ct, lst.ctypes.data,
                                   int(n[0]), _i64p(n)), "join_list")
    return lst


def relational(spec, rel_inputs, extents, blockings, g="mul", agg="sum", alpha=1.0, beta=0.0, eps=0.0,
               causal=None):
    """Def. 3.7 evaluation over relation buffers (float64 values).

    Returns (out_relation float64 unrounded, present uint8 per output tuple).
    """
    lib = _load()
    ins, out_letters = _parse(spec)
    arrs = [np.ascontiguousarray(np.asarray(r, dtype=np.float64)) for r in rel_inputs]
    for lt, a in zip(ins, arrs):
        if a.size != relation_elems(lt, extents, blockings):
            raise OracleError(f"relation {lt} has {a.size} elements")
    ptrs = (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    n_out = relation_elems(out_letters, extents, blockings)
    out = np.zeros(n_out, dtype=np.float64)
    n_tuples = 1
    for c in out_letters:
        n_tuples *= int(_nblk26(blockings)[ord(c) - 97])
    present = np.zeros(n_tuples, dtype=np.uint8)
    ext, nb, bd = _ext26(extents), _nblk26(blockings), _bnd26(blockings)
    cs, ct = _causal(causal)
    rc = lib.oracle_relational_iv(spec.encode(), G_CODES[g], AGG_CODES[agg], alpha, beta, eps, cs, ct,
                                  _i64p(ext), _i32p(nb), _i64p(bd), ptrs, out.ctypes.data, present.ctypes.data)
    _check(rc, "oracle_relational")
    return out, present


def attention_dense(spec, inputs, extents, alpha=1.0, causal=None, sample=None, segments=None):
    """Attention by its definition: out[X,s,E] = sum_t softmax_t(alpha sum_D Q K) V
    (unrounded float64); roles as in oracle.c.  ``sample``: flat output indices.
    ``segments``: (s, t, bounds) -- packed sequences: s attends only to the
    t of its own interval of ``bounds``."""
    lib = _load()
    ins, out_letters = _parse(spec)
    if len(ins) != 3:
        raise OracleError("attention takes Q, K, V")
    arrs = []
    for lt, x in zip(ins, inputs):
        x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
        want = tuple(int(extents.get(c, -1)) for c in lt)
        if x.shape != want:
            raise OracleError(f"input {lt} has shape {x.shape}, expected {want}")
        arrs.append(x)
    ext = _ext26(extents)
    cs, ct = _causal(causal)
    if sample is None:
        out = np.zeros(tuple(int(extents[c]) for c in out_letters), dtype=np.float64)
        idx_p, n = None, 0
    else:
        idx = np.ascontiguousarray(np.asarray(sample, dtype=np.int64))
        out = np.zeros(idx.shape[0], dtype=np.float64)
        idx_p, n = _i64p(idx), idx.shape[0]
    ss, st, sb, sk = -1, -1, np.zeros(1, dtype=np.int64), 0
    if segments is not None:
        ss, st = ord(segments[0]) - 97, ord(segments[1]) - 97
        sb = np.ascontiguousarray(np.asarray(segments[2], dtype=np.int64))
        sk = sb.size - 1
    rc = lib.oracle_attention_dense_seg(spec.encode(), alpha, cs, ct, ss, st, _i64p(sb), sk, _i64p(ext),
                                        arrs[0].ctypes.data, arrs[1].ctypes.data, arrs[2].ctypes.data, idx_p, n,
                                        out.ctypes.data)
    _check(rc, "oracle_attention_dense")
    return out


def attention_relational(spec, rel_inputs, extents, blockings, alpha=1.0, causal=None, segment=None):
    """Attention as one join-agg over relation buffers: per joined tuple the
    online-softmax triple, merged per output key, recomposed as a / l.
    ``segment``: (s, t) -- the join keeps only combinations whose s and t
    intervals coincide (packed sequences blocked at their ends).
    Returns (out_relation float64 unrounded, present uint8 per output tuple)."""
    lib = _load()
    ins, out_letters = _parse(spec)
    arrs = [np.ascontiguousarray(np.asarray(r, dtype=np.float64)) for r in rel_inputs]
    for lt, a in zip(ins, arrs):
        if a.size != relation_elems(lt, extents, blockings):
            raise OracleError(f"relation {lt} has {a.size} elements")
    ptrs = (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    out = np.zeros(relation_elems(out_letters, extents, blockings), dtype=np.float64)
    n_tuples = 1
    for c in out_letters:
        n_tuples *= int(_nblk26(blockings)[ord(c) - 97])
    present = np.zeros(n_tuples, dtype=np.uint8)
    ext, nb, bd = _ext26(extents), _nblk26(blockings), _bnd26(blockings)
    cs, ct = _causal(causal)
    ss, st = _causal(segment)
    rc = lib.oracle_attention_relational_seg(spec.encode(), alpha, cs, ct, ss, st, _i64p(ext), _i32p(nb), _i64p(bd),
                                             ptrs, out.ctypes.data, present.ctypes.data)
    _check(rc, "oracle_attention_relational")
    return out, present


def softmax_merge(t1, t2):
    """The merge of two online-softmax triples (m, l, a) -> (m, l, a)."""
    lib = _load()
    res = np.zeros(3, dtype=np.float64)
    lib.oracle_softmax_merge(*(float(v) for v in t1), *(float(v) for v in t2), res.ctypes.data)
    return tuple(float(v) for v in res)


def round_to(x, dtype):
    """Round float64 values once, to nearest-even, to 'f32' or 'bf16' (returned as float64)."""
    lib = _load()
    y = np.array(x, dtype=np.float64, copy=True, order="C")
    lib.oracle_round(y.ctypes.data, y.size, DTYPE_CODES[dtype])
    return y


def contract(spec, a, b, extents):
    """A two-operand contraction (g = MUL, aggregation SUM over the letters
    absent from the output), unrounded float64: the dense form of a
    contraction, out[o] = sum_r a[...] b[...] ("Every Kernel Is a Join",
    Sec. 1: a matmul is the join on the inner index followed by SUM).  The
    library routine numpy.einsum evaluates it in float64 (its BLAS path); it
    is the same value as ``dense`` up to float64 rounding and is used where
    the loops of ``dense`` would be too slow (whole token prefixes of a
    projection)."""
    ins, out_letters = _parse(spec)
    if len(ins) != 2:
        raise OracleError("contract takes two operands")
    xs = []
    for lt, x in zip(ins, (a, b)):
        x = np.asarray(x, dtype=np.float64)
        want = tuple(int(extents.get(c, -1)) for c in lt)
        if x.shape != want:
            raise OracleError(f"input {lt} has shape {x.shape}, expected {want}")
        xs.append(x)
    return np.einsum(spec, xs[0], xs[1], optimize=True)


RECOMPOSE_CODES = {"mul_plus": 0, "swiglu": 1}


def dense_recompose(spec, kind, inputs, extents, alpha=1.0, sample=None):
    """A contraction whose recompose step maps the aggregated value, dense
    form, unrounded float64 (see oracle.c, oracle_dense_recompose):
    'mul_plus': alpha * sum_r in0 in1 + in2 (in2 over output letters only);
    'swiglu': alpha * silu(sum_r in0 in1) * sum_r in0 in2.
    ``sample``: flat output indices, as for ``dense``."""
    lib = _load()
    ins, out_letters = _parse(spec)
    arrs = []
    for lt, x in zip(ins, inputs):
        x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
        want = tuple(int(extents.get(c, -1)) for c in lt)
        if x.shape != want:
            raise OracleError(f"input {lt} has shape {x.shape}, expected {want}")
        arrs.append(x)
    ptrs = (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    ext = _ext26(extents)
    if sample is None:
        out = np.zeros(tuple(int(extents[c]) for c in out_letters), dtype=np.float64)
        rc = lib.oracle_dense_recompose(spec.encode(), RECOMPOSE_CODES[kind], alpha, _i64p(ext), ptrs, None, 0,
                                        out.ctypes.data)
    else:
        idx = np.ascontiguousarray(np.asarray(sample, dtype=np.int64))
        out = np.zeros(idx.shape[0], dtype=np.float64)
        rc = lib.oracle_dense_recompose(spec.encode(), RECOMPOSE_CODES[kind], alpha, _i64p(ext), ptrs, _i64p(idx),
                                        idx.shape[0], out.ctypes.data)
    _check(rc, "oracle_dense_recompose")
    return out


def relational_recompose(spec, kind, rel_inputs, extents, blockings, alpha=1.0):
    """The relational form (Def. 3.7) of ``dense_recompose``: the join and
    SUM of the contraction(s) by ``relational``, then the recompose map on
    the aggregated output blocks -- plus the addend relation's block of the
    same key ('mul_plus'), or silu(a) * b of the two sums ('swiglu').  The
    addend must be blocked like the output.  Returns (out relation float64
    unrounded, present per output tuple)."""
    ins, out_letters = _parse(spec)
    if len(ins) != 3:
        raise OracleError("a recompose spec takes three inputs")
    sub = f"{ins[0]},{ins[1]}->{out_letters}"
    a, present = relational(sub, rel_inputs[:2], extents, blockings, alpha=1.0)
    if kind == "mul_plus":
        if sorted(ins[2]) != sorted(out_letters):
            raise OracleError("the addend must hold exactly the output letters")
        addend = repartition(np.asarray(rel_inputs[2], dtype=np.float64), ins[2], blockings, out_letters, blockings,
                             extents)
        return alpha * a + addend, present
    if kind == "swiglu":
        b, _ = relational(f"{ins[0]},{ins[2]}->{out_letters}", [rel_inputs[0], rel_inputs[2]], extents, blockings,
                          alpha=1.0)
        return alpha * (a / (1.0 + np.exp(-a))) * b, present
    raise OracleError(kind)
