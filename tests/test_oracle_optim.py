"""Pins for the fp64 oracle of gradient clipping and AdamW, against facts that
do not come from the oracle: hand-evaluated closed forms, the printed
defaults, and PyTorch's own CPU implementations (``clip_grad_norm_``,
``torch.optim.AdamW``) run in float64.  Plausible slips planted in copies of
the oracle functions must fail at least one pin.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import optim_ref as ref

torch = pytest.importorskip("torch")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- clipping --

def _torch_clip(grads, max_norm, norm_type):
    ps = []
    for g in grads:
        p = torch.zeros(np.shape(g), dtype=torch.float64, requires_grad=True)
        p.grad = torch.tensor(np.asarray(g, np.float64))
        ps.append(p)
    tot = torch.nn.utils.clip_grad_norm_(ps, max_norm, norm_type=norm_type)
    return float(tot), [p.grad.numpy().copy() for p in ps]


def _clip_battery(clip):
    """Names of the pins the clipping function fails."""
    bad = []
    # hand case: |(3, 4)| = 5, max_norm 1 -> everything times 1 / (5 + 1e-6)
    out, st = clip([np.array([3.0, 4.0])], 1.0, 2.0, None)
    c = 1.0 / (5.0 + 1e-6)
    if not (abs(st[0]["total_norm"] - 5.0) < 1e-15 and abs(st[0]["clip_coef"] - c) < 1e-15
            and np.allclose(out[0], [3 * c, 4 * c], rtol=1e-15, atol=0) and st[0]["clipped"]):
        bad.append("hand-3-4")
    # below the limit: unchanged
    out, st = clip([np.array([0.3, 0.4])], 1.0, 2.0, None)
    if not (np.array_equal(out[0], [0.3, 0.4]) and not st[0]["clipped"]):
        bad.append("no-clip")
    # stats only
    out, st = clip([np.array([3.0, 4.0])], None, 2.0, None)
    if not (np.array_equal(out[0], [3.0, 4.0]) and st[0]["total_norm"] == 5.0):
        bad.append("stats-only")
    # PyTorch, several norms, one bucket
    rng = np.random.default_rng(3)
    grads = [rng.standard_normal((5, 7)) * 3, rng.standard_normal((4, 2)), rng.standard_normal(9)]
    for p in (2.0, 1.0, 3.0, math.inf):
        for mx in (0.5, 1e3):
            t_tot, t_out = _torch_clip(grads, mx, p)
            out, st = clip(grads, mx, p, None)
            ok = abs(st[0]["total_norm"] - t_tot) <= 1e-12 * t_tot and all(
                np.allclose(a, b, rtol=1e-12, atol=0) for a, b in zip(out, t_out))
            if not ok:
                bad.append(f"torch-p{p}-max{mx}")
    # buckets: segment-local, i.e. each bucket as if clipped alone
    buckets = [1, 0, 1]
    out, st = clip(grads, 0.5, 2.0, buckets)
    for b in (0, 1):
        members = [i for i, k in enumerate(buckets) if k == b]
        t_tot, t_out = _torch_clip([grads[i] for i in members], 0.5, 2.0)
        ok = abs(st[b]["total_norm"] - t_tot) <= 1e-12 * t_tot and all(
            np.allclose(out[i], t, rtol=1e-12, atol=0) for i, t in zip(members, t_out))
        if not ok:
            bad.append(f"bucket{b}")
    # non-finite: inf -> coefficient 0 (PyTorch multiplies anyway), NaN -> NaN
    out, st = clip([np.array([1.0, math.inf])], 1.0, 2.0, None)
    if not (st[0]["found_inf"] and math.isinf(st[0]["total_norm"]) and out[0][0] == 0.0):
        bad.append("inf")
    out, st = clip([np.array([1.0, math.nan])], 1.0, math.inf, None)
    if not (st[0]["found_inf"] and math.isnan(st[0]["total_norm"]) and np.isnan(out[0]).all()):
        bad.append("nan-inf-norm")
    return bad


def _oracle_clip(g, mx, p, b):
    return ref.clip_grad_norm(g, mx, norm_type=p, buckets=b)


def test_clip_oracle_passes():
    assert _clip_battery(_oracle_clip) == []


def _clip_variant(eps=1e-6, clamp=True, root=True, buckets=True, nan_max=True):
    def norm(gs, p):
        a = np.concatenate([np.abs(np.asarray(g, np.float64)).ravel() for g in gs])
        if math.isinf(p):
            return float(np.max(a)) if nan_max else float(np.nanmax(a))
        s = float(np.sum(a ** p))
        return s ** (1.0 / p) if root else s

    def clip(grads, mx, p, bk):
        grads = [np.asarray(g, np.float64) for g in grads]
        bk = [0] * len(grads) if (bk is None or not buckets) else bk
        out = [g.copy() for g in grads]
        st = []
        for b in range(max(bk) + 1):
            mem = [i for i, k in enumerate(bk) if k == b]
            tot = norm([grads[i] for i in mem], p)
            coef = 1.0 if mx is None else mx / (tot + eps)
            if mx is not None:
                s = min(coef, 1.0) if clamp else coef
                for i in mem:
                    out[i] = grads[i] * s
            st.append({"total_norm": tot, "clip_coef": coef, "clipped": coef < 1.0,
                       "found_inf": not math.isfinite(tot)})
        while len(st) < 2:
            st.append(st[-1])
        return out, st
    return clip


CLIP_MUTANTS = {
    "no-eps": _clip_variant(eps=0.0),
    "unclamped": _clip_variant(clamp=False),
    "squared-norm": _clip_variant(root=False),
    "global-buckets": _clip_variant(buckets=False),
    "nan-ignoring-max": _clip_variant(nan_max=False),
}


@pytest.mark.parametrize("name", sorted(CLIP_MUTANTS))
def test_clip_pins_reject_mutant(name):
    assert _clip_battery(CLIP_MUTANTS[name]) != []


# ------------------------------------------------------------------- AdamW --

def _torch_adamw(p0, grads, **hp):
    p = torch.tensor(np.asarray(p0, np.float64), requires_grad=True)
    opt = torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"], foreach=False)
    for g in grads:
        p.grad = torch.tensor(np.asarray(g, np.float64))
        opt.step()
    st = opt.state[p]
    return p.detach().numpy().copy(), st["exp_avg"].numpy().copy(), st["exp_avg_sq"].numpy().copy()


def _adamw_battery(adamw):
    bad = []
    hp = dict(ref.ADAMW_DEFAULTS)
    rng = np.random.default_rng(5)
    p0 = rng.standard_normal((6, 5))
    grads = [rng.standard_normal((6, 5)) * s for s in (1.0, 0.1, 3.0, 1e-3)]
    # against PyTorch, four steps, defaults and a second setting
    for h in (hp, {"lr": 0.05, "beta1": 0.8, "beta2": 0.95, "eps": 1e-6, "weight_decay": 0.3}):
        tp, tm, tv = _torch_adamw(p0, grads, **h)
        p, m, v = p0, np.zeros_like(p0), np.zeros_like(p0)
        for t, g in enumerate(grads, start=1):
            p, m, v = adamw(p, g, m, v, t, **h)
        if not (np.allclose(p, tp, rtol=1e-12, atol=1e-15) and np.allclose(m, tm, rtol=1e-12)
                and np.allclose(v, tv, rtol=1e-12)):
            bad.append(f"torch-lr{h['lr']}")
    # step 1 from zero state: m^ = g, v^ = g^2
    g = grads[0]
    p, _, _ = adamw(p0, g, np.zeros_like(g), np.zeros_like(g), 1, **hp)
    want = p0 * (1 - hp["lr"] * hp["weight_decay"]) - hp["lr"] * g / (np.abs(g) + hp["eps"])
    if not np.allclose(p, want, rtol=1e-13, atol=1e-16):
        bad.append("step1")
    # constant gradient, no decay: the bias-corrected moments stay (g, g^2)
    h0 = dict(hp, weight_decay=0.0)
    p, m, v = p0, np.zeros_like(p0), np.zeros_like(p0)
    for t in range(1, 8):
        p, m, v = adamw(p, g, m, v, t, **h0)
    want = p0 - 7 * hp["lr"] * g / (np.abs(g) + hp["eps"])
    if not np.allclose(p, want, rtol=1e-12, atol=1e-15):
        bad.append("constant-grad")
    return bad


def test_adamw_oracle_passes():
    assert _adamw_battery(ref.adamw_step) == []


def _adamw_variant(bc1=True, bc2=True, eps_inside=False, coupled=False, decay_after=False):
    def step(p, g, m, v, t, lr, beta1, beta2, eps, weight_decay):
        p = np.asarray(p, np.float64)
        g = np.asarray(g, np.float64)
        if coupled:
            g = g + weight_decay * p
        elif not decay_after:
            p = p * (1 - lr * weight_decay)
        m = beta1 * m + (1 - beta1) * g
        v = beta2 * v + (1 - beta2) * g * g
        mh = m / (1 - beta1 ** t) if bc1 else m
        vh = v / (1 - beta2 ** t) if bc2 else v
        den = np.sqrt(vh + eps) if eps_inside else np.sqrt(vh) + eps
        p = p - lr * mh / den
        if decay_after and not coupled:
            p = p * (1 - lr * weight_decay)
        return p, m, v
    return step


ADAMW_MUTANTS = {
    "no-bias-correction-m": _adamw_variant(bc1=False),
    "no-bias-correction-v": _adamw_variant(bc2=False),
    "eps-inside-sqrt": _adamw_variant(eps_inside=True),
    "coupled-l2": _adamw_variant(coupled=True),
    "decay-after-update": _adamw_variant(decay_after=True),
}


@pytest.mark.parametrize("name", sorted(ADAMW_MUTANTS))
def test_adamw_pins_reject_mutant(name):
    assert _adamw_battery(ADAMW_MUTANTS[name]) != []


def test_defaults_match_the_printed_signatures():
    with open(os.path.join(GOLDEN, "dmuon_api_constants.json")) as f:
        gold = json.load(f)
    a = gold["muon_adamw_defaults"]
    assert oracle.ADAMW_DEFAULTS == {"lr": a["adamw_lr"], "beta1": a["adamw_betas"][0],
                                     "beta2": a["adamw_betas"][1], "eps": a["adamw_eps"],
                                     "weight_decay": a["adamw_weight_decay"]}
    import inspect
    assert (inspect.signature(ref.clip_grad_norm).parameters["norm_type"].default
            == gold["clip_grad_norm_defaults"]["norm_type"])
