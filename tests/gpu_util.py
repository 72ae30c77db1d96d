"""Helpers shared by the GPU tests: moving seeded numpy inputs to the
device in a given dtype, reading results back exactly, and the error
metrics the tolerances are stated in."""
import numpy as np


def torch_dtype(name):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def to_dev(a, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch_dtype(dtype) if isinstance(dtype, str) else dtype).cuda()


def exact64(t):
    """Device tensor -> float64 numpy (exact for fp32 and bf16)."""
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def rel_frobenius(got, want):
    d = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (d if d > 0 else 1.0))


def sigma_dev(got, want):
    """Max |sigma_i(got) - sigma_i(want)|, both sorted descending."""
    a = np.linalg.svd(got, compute_uv=False)
    b = np.linalg.svd(want, compute_uv=False)
    return float(np.max(np.abs(a - b)))


def bf16_ulp(x):
    """Spacing of bfloat16 values at |x| (normal range)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def bf16_param_excess(p_before, p_after, O, lr):
    """Error of a bf16 param update p_after ~ RNE(p_before - lr*O) measured
    beyond the final rounding: the part of |p_after - (p_before - lr*O)|
    above half an ulp of the stored value, relative to ||lr*O||_F.  Returns
    (relative excess, share of elements that differ from RNE of the exact
    value)."""
    import oracle
    exact = p_before - lr * O
    excess = np.maximum(np.abs(p_after - exact) - 0.5 * bf16_ulp(p_after) * 1.0001, 0)
    e = float(np.linalg.norm(excess) / (lr * np.linalg.norm(O)))
    frac = float(np.mean(p_after != oracle.round_to_bf16(exact)))
    return e, frac
