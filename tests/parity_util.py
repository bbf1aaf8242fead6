"""Helpers shared by the GPU parity tests: moving relation buffers between
the device and numpy, and the error measure used by the tolerances.

Error measure (the gate for floating point): e = max_i |y_i - yhat_i| /
max_i |yhat_i| over the valid elements of an output, y from the HIP path and
yhat from the oracle.  Pointwise relative error is not used as the gate
because it is meaningless where the exact result cancels to near zero.
"""
import numpy as np
import torch

from oracle import oracle as O
from tensor_relational_einsum_amd import inputs as I


def to_np(t: torch.Tensor) -> np.ndarray:
    """Device/host tensor -> float64 numpy (exact for f32 and bf16)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw element bits of a tensor as unsigned numpy integers."""
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    raise TypeError(t.dtype)


def normwise_err(y, yhat) -> float:
    y = np.asarray(y, dtype=np.float64)
    yhat = np.asarray(yhat, dtype=np.float64)
    den = np.max(np.abs(yhat)) if yhat.size else 0.0
    num = np.max(np.abs(y - yhat)) if y.size else 0.0
    return float(num / den) if den > 0 else float(num)


def rel_dense(rel, extents: dict) -> np.ndarray:
    """A jagg.Relation's buffer densified on the host by the oracle (float64)."""
    blk = rel.blocking()
    return O.from_relation(to_np(rel.data), rel.letters, extents, blk)


def padding_mask(letters, extents, blockings) -> np.ndarray:
    """True at the padding positions of a relation buffer."""
    return O.to_relation(np.ones([extents[c] for c in letters], dtype=np.uint8), letters, extents, blockings) == 0


def oracle_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values already rounded to `dtype` -> their bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return bits(t)


def oracle_chain(w, dense, stop=None):
    """Evaluates a workload chain on the oracle, rounding each result to its
    stored dtype exactly where the HIP path stores it."""
    vals = {k: to_np(v) for k, v in dense.items()}
    for st in w.chain:
        if isinstance(st, I.Step):
            ins = st.spec.split("->")[0].split(",")
            xs = []
            for name, lt in zip(st.ins, ins):
                xs.append(vals[name])
            if st.g == "attention":
                seg = None
                if st.segment is not None:
                    seg = (st.segment[0], st.segment[1], st.blockings[st.segment[0]])
                y = O.attention_dense(st.spec, xs, w.extents, alpha=st.alpha, causal=st.causal, segments=seg)
            elif st.g in ("mul_plus", "swiglu"):
                y = O.dense_recompose(st.spec, st.g, xs, w.extents, alpha=st.alpha)
            else:
                y = O.dense(st.spec, xs, w.extents, g=st.g, agg=st.agg, alpha=st.alpha, beta=st.beta, eps=st.eps,
                            causal=st.causal)
            vals[st.out] = O.round_to(y, st.out_dtype)
        else:
            src_letters = None
            for t in w.tensors:
                if t[0] == st.src:
                    src_letters = t[1]
            if src_letters is None:
                src_letters = next(s for s in w.chain if getattr(s, "out", None) == st.src).spec.split("->")[1]
            perm = [src_letters.index(c) for c in st.letters]
            vals[st.out] = np.ascontiguousarray(vals[st.src].transpose(perm))
        if stop is not None and st.out == stop:
            break
    return vals


def llama_block_rows(w, dense, b, rows):
    """The LLaMA-shaped block evaluated by the oracle from its original
    inputs, for the query rows `rows` of batch index `b` only.

    The block is causal in its token letter: output row s depends on the
    input rows t <= s alone (every other step is row-wise).  So the key and
    value projections run over the token prefix [0, max(rows)] and every
    other step over the sampled rows, each step rounded to its stored dtype
    where the HIP path stores it, with the alpha / beta / eps of the
    workload's own steps.  Both attention forms of the recipe are followed:
    the fused spec (softmax inside one aggregation, probabilities exact) or
    the five-spec chain (S fp32, P bf16).  Returns {name: array [len(rows),
    ...]} for the attention output "O", "x2" and "y"."""
    steps = {st.out: st for st in w.chain if isinstance(st, I.Step)}
    ext = dict(w.extents)
    Hd, Q_, D_ = ext["h"], ext["q"], ext["d"]
    P = max(rows) + 1
    x = to_np(dense["x"])[b:b + 1]
    g1, g2 = to_np(dense["g1"]), to_np(dense["g2"])
    Wq, Wk, Wv, Wo = (to_np(dense[n]) for n in ("Wq", "Wk", "Wv", "Wo"))
    Wg, Wu, Wd = (to_np(dense[n]) for n in ("Wg", "Wu", "Wd"))
    rnd = O.round_to

    def rms(xs, g, st, n):
        e = dict(ext, b=1, s=n)
        ss = rnd(O.dense("bsh->bs", [xs], e, g="square", agg="sum"), steps[st[0]].out_dtype)
        r = O.dense("bsh,bs,h->bsh", [xs, ss, g], e, g="rms_scale", agg="none", beta=steps[st[1]].beta,
                    eps=steps[st[1]].eps)
        return rnd(r, steps[st[1]].out_dtype)

    r1 = rms(x[:, :P], g1, ("ss1", "r1"), P)
    ep = dict(ext, b=1, s=P)
    K = rnd(O.contract("bsh,hqd->bsqd", r1, Wk, ep), steps["Kp"].out_dtype)
    V = rnd(O.contract("bsh,hqd->bsqd", r1, Wv, ep), steps["Vp"].out_dtype)
    R = len(rows)
    er = dict(ext, b=1, s=R)
    xr = x[:, rows]
    Qr = rnd(O.contract("bsh,hqd->bsqd", r1[:, rows], Wq, er), steps["Qp"].out_dtype)
    Orows = []
    for i, s in enumerate(rows):
        e1 = dict(ext, b=1, s=1, t=s + 1)
        q1 = Qr[:, i:i + 1]
        k1, v1 = K[:, :s + 1], V[:, :s + 1]
        if "O" in steps and steps["O"].g == "attention":
            st = steps["O"]
            o = O.attention_dense("bsqd,btqd,btqe->bsqe", [q1, k1, v1], dict(e1, e=D_), alpha=st.alpha)
            Orows.append(rnd(o, st.out_dtype))
        else:
            # the five-spec chain in head-major order; t <= s is every t here
            qh, kh, vh = (np.ascontiguousarray(a.transpose(0, 2, 1, 3)) for a in (q1, k1, v1))
            S = rnd(O.dense("bqsd,bqtd->bqst", [qh, kh], e1, alpha=steps["S"].alpha), steps["S"].out_dtype)
            M = O.dense("bqst->bqs", [S], e1, g="ident", agg="max")
            L = rnd(O.dense("bqst,bqs->bqs", [S, M], e1, g="exp_sub"), steps["L"].out_dtype)
            Pp = rnd(O.dense("bqst,bqs,bqs->bqst", [S, M, L], e1, g="exp_sub_div", agg="none"),
                     steps["P"].out_dtype)
            oh = rnd(O.dense("bqst,bqtd->bqsd", [Pp, vh], e1), steps["Oh"].out_dtype)
            Orows.append(np.ascontiguousarray(oh.transpose(0, 2, 1, 3)))
    Oa = np.concatenate(Orows, axis=1)
    if steps["x2"].g == "mul_plus":
        # the residual adds and the SiLU gate as recompose maps of the
        # contractions feeding them: sums in float64, one rounding each
        x2 = rnd(O.dense_recompose("bsqd,qdh,bsh->bsh", "mul_plus", [Oa, Wo, xr], er), steps["x2"].out_dtype)
        r2 = rms(x2, g2, ("ss2", "r2"), R)
        Hh = rnd(O.dense_recompose("bsh,hf,hf->bsf", "swiglu", [r2, Wg, Wu], er), steps["H"].out_dtype)
        y = rnd(O.dense_recompose("bsf,fh,bsh->bsh", "mul_plus", [Hh, Wd, x2], er), steps["y"].out_dtype)
    else:
        A = rnd(O.contract("bsqd,qdh->bsh", Oa, Wo, er), steps["A"].out_dtype)
        x2 = rnd(O.dense("bsh,bsh->bsh", [xr, A], er, g="add", agg="none"), steps["x2"].out_dtype)
        r2 = rms(x2, g2, ("ss2", "r2"), R)
        G = rnd(O.contract("bsh,hf->bsf", r2, Wg, er), steps["G"].out_dtype)
        U = rnd(O.contract("bsh,hf->bsf", r2, Wu, er), steps["U"].out_dtype)
        Hh = rnd(O.dense("bsf,bsf->bsf", [G, U], er, g="silu_mul", agg="none"), steps["H"].out_dtype)
        Dd = rnd(O.contract("bsf,fh->bsh", Hh, Wd, er), steps["D"].out_dtype)
        y = rnd(O.dense("bsh,bsh->bsh", [x2, Dd], er, g="add", agg="none"), steps["y"].out_dtype)
    assert Oa.shape == (1, R, Q_, D_) and y.shape == (1, R, Hd)
    return {"O": Oa[0], "x2": x2[0], "y": y[0]}
