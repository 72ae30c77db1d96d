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


def singular_values_gram(a):
    """Singular values of a (descending) from the eigenvalues of its smaller
    Gram matrix: O(p^2 q) instead of an SVD, for full-size outputs whose
    singular values sit near 1 (well conditioned, so squaring loses nothing
    at the 2e-2 tolerance)."""
    a = np.asarray(a, dtype=np.float64)
    g = a.T @ a if a.shape[0] > a.shape[1] else a @ a.T
    w = np.linalg.eigvalsh(g)[::-1]
    return np.sqrt(np.maximum(w, 0.0))


def sigma_dev_gram(got, want):
    """sigma_dev through singular_values_gram."""
    return float(np.max(np.abs(singular_values_gram(got) - singular_values_gram(want))))


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


def bf16_param_check(p_before, p_after, O, lr):
    """A bf16 param update p_after against r = RNE(p_before - lr*O), the
    exact update rounded once.  Returns (largest |p_after - r| in units of
    the bf16 spacing at the element's scale, share of elements that differ
    from r at all).  The element's scale is the largest of |p_before|, |r|
    and the rms of p_before: at an element's own magnitude alone the test
    would be meaningless where p_before and lr*O nearly cancel (r tiny, its
    spacing far below the error any NS leaves in lr*O), while an NS error
    below a spacing of the tensor's typical value moves an element by at most
    one spacing (a rounding boundary crossed)."""
    import oracle
    r = oracle.round_to_bf16(p_before - lr * O)
    rms = float(np.sqrt(np.mean(np.square(p_before))))
    scale = np.maximum(np.maximum(np.abs(p_before), np.abs(r)), rms)
    dist = np.abs(p_after - r) / bf16_ulp(scale)
    return float(dist.max()), float(np.mean(p_after != r))


def bf16_frac_cap(p_before, O, lr, tol, floor=0.05):
    """Largest share of bf16 params allowed to differ from RNE(p - lr*O):
    `floor`, or, where lr*O spans several bf16 spacings of p (small
    matrices, whose O entries are larger), the share that an NS error at the
    tolerance would move across a rounding boundary: an additive error of
    rms tol * rms(lr*O) crosses the boundary of an element with spacing s
    with probability about E|e|/s = sqrt(2/pi) * tol * rms(lr*O) / s."""
    s = bf16_ulp(np.abs(p_before))
    e = np.sqrt(2.0 / np.pi) * tol * float(np.sqrt(np.mean(np.square(lr * O))))
    return max(floor, float(np.mean(np.minimum(1.0, e / s))))
