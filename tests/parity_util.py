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
