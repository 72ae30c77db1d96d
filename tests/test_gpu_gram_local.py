"""GPU parity of Gram-space NS on column shards (dmuon_gram_local_*) against
the fp64 oracle, through the C ABI.

Several ranks of a shard group are stood in for by several call sequences on
one GPU, each with its own workspace: between the calls the test sums the
ranks' buckets (the group's all-reduce) and writes the sum back into every
bucket.  Tolerance: fp32 NS, <= 1e-4 relative Frobenius.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import exact64, rel_frobenius, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import newton_schulz_06_amd as dm  # noqa: E402


def _split(G, transposed, widths):
    cuts = np.cumsum([0] + list(widths))
    if transposed:
        return [G[a:b, :] for a, b in zip(cuts[:-1], cuts[1:])]
    return [G[:, a:b] for a, b in zip(cuts[:-1], cuts[1:])]


def _group_run(rank_blocks, transposed, dtype="f32", in_place=False, repeat=1, **kw):
    """rank_blocks[r] = list of rank r's blocks (numpy, one per matrix).
    Returns (inputs as run, outputs) per rank, float64."""
    ins = [[to_dev(b, dtype) for b in blocks] for blocks in rank_blocks]
    outs = [list(x) if in_place else [torch.empty_like(t) for t in x] for x in ins]
    snap = [[exact64(t) for t in x] for x in ins]
    for _ in range(repeat):
        if in_place:  # restore the inputs for each repeat
            for x, s in zip(ins, snap):
                for t, v in zip(x, s):
                    t.copy_(torch.from_numpy(v).to(t.dtype))
        runs = [dm.GramLocal(x, o, transposed=transposed, **kw) for x, o in zip(ins, outs)]
        for r in runs:
            r.begin()
        for w in range(runs[0].windows):
            total = runs[0].bucket.clone()
            for r in runs[1:]:
                total += r.bucket
            for r in runs:
                r.bucket.copy_(total)
            for r in runs:
                r.advance(w)
    torch.cuda.synchronize()
    return snap, [[exact64(t) for t in o] for o in outs]


def _check(snap, outs, transposed, tol=1e-4, **kw):
    nmat = len(snap[0])
    for i in range(nmat):
        shards = [s[i] for s in snap]
        want = oracle.gram_newton_schulz_distributed_local(shards, transposed, **kw)
        for r, (o, w) in enumerate(zip(outs, want)):
            e = rel_frobenius(o[i], w)
            assert e <= tol, (i, r, o[i].shape, e)


def _mat(m, n, seed, kind="gauss"):
    return workloads.grad_np(kind, m, n, 93, seed, 0)


@pytest.mark.parametrize("transposed,shapes", [
    (0, [(64, 64), (100, 300), (1, 7), (520, 1100), (33, 33)]),
    (1, [(300, 100), (7, 1), (700, 257), (129, 129)]),
    (0, [(300, 100), (257, 64)]),   # forced: p is the longer side
    (1, [(100, 300), (64, 257)]),
])
def test_one_rank_is_gram_ns(transposed, shapes):
    blocks = [_mat(m, n, i) for i, (m, n) in enumerate(shapes)]
    snap, outs = _group_run([blocks], transposed)
    _check(snap, outs, transposed)
    # where the flag agrees with the auto rule, this is the Gram backend's result
    for g, o in zip(snap[0], outs[0]):
        if (g.shape[0] > g.shape[1]) == bool(transposed) or g.shape[0] == g.shape[1]:
            assert rel_frobenius(o, oracle.gram_newton_schulz(g)) <= 1e-4


@pytest.mark.parametrize("transposed", [0, 1])
@pytest.mark.parametrize("restarts", [None, [], [1, 3]])
def test_three_ranks_ragged(transposed, restarts):
    # oriented p x q matrices split into column blocks of unequal widths
    specs = [(96, [40, 40, 20]), (300, [128, 100, 72]), (200, [13, 300, 7])]
    rank_blocks = [[], [], []]
    for i, (p, widths) in enumerate(specs):
        q = sum(widths)
        G = _mat(q, p, 10 + i) if transposed else _mat(p, q, 10 + i)
        for r, b in enumerate(_split(G, transposed, widths)):
            rank_blocks[r].append(b)
    snap, outs = _group_run(rank_blocks, transposed, restart_iterations=restarts)
    _check(snap, outs, transposed, restart_iterations=restarts)


def test_you_coefficients_two_ranks():
    table = oracle.YOU_COEFFICIENTS
    G = _mat(256, 1000, 3)
    rank_blocks = [[b] for b in _split(G, 0, [500, 500])]
    snap, outs = _group_run(rank_blocks, 0, coefficients=table, restart_iterations=[1, 2, 3, 4])
    _check(snap, outs, 0, coefficients=table, restart_iterations=[1, 2, 3, 4])


def test_bf16_blocks_in_place_and_repeated():
    G = _mat(700, 192, 5, "lowrank")
    rank_blocks = [[b] for b in _split(G, 1, [300, 400])]
    snap, outs = _group_run(rank_blocks, 1, dtype="bf16", prec="auto", in_place=True, repeat=2)
    # bf16 output: the final rounding on top of the fp32 NS bound
    _check(snap, outs, 1, tol=1e-2)


def test_llama_gate_tp8_shards_full_size():
    """A Llama-8B gate matrix (14336 x 4096, oriented 4096 x 14336) split 8
    ways along its long side: blocks of 1792 x 4096, the shards of a TP-8
    group.  The joined output is checked against the full matrix's NS."""
    G = workloads.grad_np("gauss", 14336, 4096, 94, 0, 0)
    blocks = _split(G, 1, [1792] * 8)
    snap, outs = _group_run([[b] for b in blocks], 1)
    joined = np.concatenate([o[0] for o in outs], axis=0)
    g = np.concatenate([s[0] for s in snap], axis=0)
    want = oracle.gram_newton_schulz(np.asfortranarray(g))
    assert rel_frobenius(joined, want) <= 1e-4
