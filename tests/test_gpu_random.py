"""Seeded random sweep of single-sequence steps against the fp64 oracle.

Each case draws a shape (L up to 2500, d a multiple of 8 up to 384, V from
33 to 4000), a mask density, a window, a block size (or none), k, a ranking
score and, for some, a threshold, then checks rows, the library's own
selection rule and the committed set exactly as the policy tests do.  The
shapes stay inside what the GEMM variants support (d % 8 == 0), and
every combination of window, block, k and policy is legal input; the point
is combinations nobody picked by hand."""
import numpy as np
import pytest

from test_gpu_policy import _inputs, _policy_case

pytestmark = pytest.mark.gpu

SCORES = ("conf", "margin", "neg_entropy")


def _draw(seed):
    r = np.random.default_rng(1000 + seed)
    L = int(r.integers(1, 2501))
    d = 32 * int(r.integers(1, 13)) if r.random() < 0.5 else 8 * int(r.integers(1, 49))
    V = int(r.integers(33, 4001))
    frac = float(r.choice([0.0, 1.0, r.uniform(0.0, 1.0), r.uniform(0.0, 1.0)]))
    lo = int(r.integers(0, L + 1))
    hi = int(r.integers(lo, L + 1))
    block = 0 if r.random() < 0.5 else int(r.integers(1, 65))
    k = int(r.integers(0, 65))
    score = SCORES[int(r.integers(0, 3))]
    tau = None
    if r.random() < 0.4:
        tau = float(r.uniform(-8.0, 0.0)) if score == "neg_entropy" else float(r.uniform(0.0, 1.0))
    return L, d, V, frac, lo, hi, block, k, score, tau


@pytest.mark.parametrize("seed", range(32))
def test_random_step(seed):
    L, d, V, frac, lo, hi, block, k, score, tau = _draw(seed)
    H, W, mask, tokens = _inputs(seed, L, d, V, frac)
    _policy_case(H, W, mask, tokens, k, lo, hi, block, score=score, tau=tau, where=f"random{seed}")


def _draw_batch(seed):
    r = np.random.default_rng(2000 + seed)
    B = int(r.choice([1, 2, 3, 5, 8, 17]))
    L = int(r.integers(1, 700))
    d = 32 * int(r.integers(1, 9)) if r.random() < 0.5 else 8 * int(r.integers(1, 33))
    V = int(r.integers(33, 3000))
    frac = float(r.choice([0.0, 1.0, r.uniform(0.0, 1.0), r.uniform(0.0, 1.0)]))
    block = 0 if r.random() < 0.5 else int(r.integers(1, 40))
    seqs = []
    for _ in range(B):
        lo = int(r.integers(0, L + 1))
        seqs.append((int(r.integers(0, 24)), lo, int(r.integers(lo, L + 1))))
    score = SCORES[int(r.integers(0, 3))]
    tau = None
    if r.random() < 0.4:
        tau = float(r.uniform(-8.0, 0.0)) if score == "neg_entropy" else float(r.uniform(0.0, 1.0))
    return B, L, d, V, frac, block, seqs, score, tau


@pytest.mark.parametrize("seed", range(16))
def test_random_batch_step(seed):
    from _parity import run_batch, to_dev
    from test_gpu_batch import _check_batch, _readout
    from test_gpu_batch import _inputs as _batch_inputs
    B, L, d, V, frac, block, seqs, score, tau = _draw_batch(seed)
    H, W, mask, tokens = _batch_inputs(seed, B, L, d, V, frac)
    Wt, Ht, mt, tt = to_dev(W, H, mask, tokens)
    rd = _readout(Wt, B * L, max(1, max(k for k, _, _ in seqs)))
    print(f"[case] random batch {seed} B={B} L={L} d={d} V={V} block={block} score={score} tau={tau}", flush=True)
    g = run_batch(rd, Ht, mt, tt, seqs, block, score=score, tau=tau, ext=True)
    _check_batch(g, H, W, mask, tokens, seqs, block, score=score, tau=tau, where=f"random batch {seed}")


@pytest.mark.parametrize("seed", range(8))
def test_random_ffn(seed):
    """The chunked SwiGLU FFN on random legal shapes (d % 256 == 0,
    F % 128 == 0), chunk sizes from 1 row to more than L, in place or not,
    held to the FFN tests' error bounds."""
    from test_gpu_ffn import RMS_REL, _bf, _check, _run
    import workloads as WL
    r = np.random.default_rng(3000 + seed)
    L = int(r.integers(1, 1500))
    d = 256 * int(r.integers(1, 5))
    F = 128 * int(r.integers(1, 13))
    chunk = int(r.integers(1, 2001)) if r.random() < 0.8 else int(r.integers(1, 9))
    inplace = r.random() < 0.3
    rng = np.random.default_rng(4000 + seed)
    X = WL.bf16_round(rng.standard_normal((L, d)).astype(np.float32))
    Wg, Wu, Wd = _bf(rng, (F, d), 0.05), _bf(rng, (F, d), 0.05), _bf(rng, (d, F), 0.05)
    print(f"[case] random ffn {seed} L={L} d={d} F={F} chunk={chunk} inplace={inplace}", flush=True)
    Yg, _ = _run(X, Wg, Wu, Wd, chunk, "inplace" if inplace else None)
    rel = _check(Yg, X, Wg, Wu, Wd, where=f"random ffn {seed}")
    assert rel < RMS_REL
