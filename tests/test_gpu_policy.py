"""GPU parity of the selection policies against the fp64 oracle: ranking by
confidence, top-2 margin or negative entropy (computed in the same streaming
pass as the argmax and log-sum-exp), top-k or threshold (adaptive parallel
decoding: commit every row whose score clears tau, at least one, at most k),
on all three GEMM variants (few rows, persistent, streaming fallback for
d % 32 != 0).  Every call goes through the C ABI (dllm_masked_readout_step_ex).

Inputs: N(0,1) hidden rows each scaled by a log-uniform factor in [0.25, 16]
(an inverse temperature), so confidences, margins and entropies spread over
their whole range instead of clustering; W_lm ~ N(0, 0.05).
"""
import numpy as np
import pytest

import oracle
import workloads as WL
from _parity import (check_commit, check_ext_rows, check_rank_order, check_rows, check_selection,
                     check_self_selection, oracle_score, run_step, score_gap, threshold_n_bounds, to_dev)

pytestmark = pytest.mark.gpu

SCORES = ("conf", "margin", "neg_entropy")


def _readout(Wt, L_max, k_max):
    import masked_token_logits_amd as mtl
    return mtl.MaskedReadout(Wt, L_max, k_max)


def _inputs(seed, L, d, V, frac):
    rng = np.random.default_rng(seed)
    scale = np.exp(rng.uniform(np.log(0.25), np.log(16.0), size=(L, 1))).astype(np.float32)
    H = WL.bf16_round((rng.standard_normal((L, d)).astype(np.float32) * scale))
    W = WL.bf16_round((rng.standard_normal((V, d)) * 0.05).astype(np.float32))
    mask = (rng.random(L) < frac).astype(np.uint8)
    tokens = rng.integers(0, V, L).astype(np.int32)
    tokens[mask != 0] = V
    return H, W, mask, tokens


def _policy_case(H, W, mask, tokens, k, lo=0, hi=None, block=0, score="conf", tau=None, rd=None, where=""):
    """One step with ext outputs: rows, the library's self-consistency, and
    the committed set against the oracle.  ``tau`` is in the score's units
    (a probability for "conf")."""
    L = len(mask)
    hi = L if hi is None else hi
    Wt, Ht, mt, tt = to_dev(W, H, mask, tokens)
    if rd is None:
        rd = _readout(Wt, L, max(k, 1))
    print(f"[case] {where} L={L} d={H.shape[1]} V={W.shape[0]} k={k} win=({lo},{hi}) block={block} "
          f"score={score} tau={tau}", flush=True)
    g = run_step(rd, Ht, mt, tt, k, lo, hi, block, score=score, tau=tau, ext=True)
    o = oracle.readout_step(H, W, mask, tokens, k, lo, hi, block, score=score, tau=tau)
    assert g["M"] == o.M, f"{where}: M {g['M']} vs {o.M}"
    np.testing.assert_array_equal(g["row_idx"], o.positions)
    check_rows(g["row_tok"], g["row_conf"], g["row_lse"], o.stats, where)
    check_ext_rows(g["row_margin"], g["row_entropy"], o.stats, where)
    n = check_self_selection(g, score, k, tau, where)
    so, gap = oracle_score(o.stats, score), score_gap(score)
    if tau is not None:
        t_o = tau
        if score == "conf":                                # compared on log-confidence
            t_o = np.log(tau) if tau > 0 else -np.inf
        n_lo, n_hi = threshold_n_bounds(so, t_o, k, gap)
        assert n_lo <= n <= n_hi, f"{where}: threshold n={n} outside oracle range [{n_lo}, {n_hi}]"
    else:
        assert n == len(o.sel)
    band = check_selection(g["sel_idx"], o.positions, so, n, where, gap=gap)
    check_rank_order(g["sel_idx"], o.positions, so, where, gap=gap)
    check_commit(mask, tokens, g, lo, hi)
    return g, o, band


# (path, seed, L, d, V, frac, lo, hi, block, k)
PATHS = {
    "few_rows": (21, 400, 256, 5000, 0.7, 100, 132, 0, 6),      # window of 32 rows
    "persistent": (22, 700, 256, 3001, 0.6, 0, 700, 0, 40),     # d % 32 == 0, ragged V and rows
    "streaming": (23, 650, 200, 2500, 0.6, 0, 650, 0, 40),      # d % 32 != 0 (fallback GEMM)
}


@pytest.mark.parametrize("path", sorted(PATHS))
@pytest.mark.parametrize("score", SCORES)
def test_topk_by_score(path, score):
    seed, L, d, V, frac, lo, hi, block, k = PATHS[path]
    H, W, mask, tokens = _inputs(seed, L, d, V, frac)
    _policy_case(H, W, mask, tokens, k, lo, hi, block, score=score, where=f"topk {path} {score}")


def _clear_tau(score_sorted_desc, frac_lo, frac_hi, gap):
    """A threshold in the widest gap of the sorted scores between the given
    rank fractions (so the rule's n is decided well away from rounding)."""
    s = score_sorted_desc
    M = len(s)
    a, b = max(1, int(M * frac_lo)), max(2, int(M * frac_hi))
    j = a + int(np.argmax(s[a - 1:b - 1] - s[a:b]))
    assert s[j - 1] - s[j] > 4 * gap, "no clear gap for the threshold"
    return 0.5 * (s[j - 1] + s[j]), j


@pytest.mark.parametrize("path", sorted(PATHS))
@pytest.mark.parametrize("score", SCORES)
def test_threshold_by_score(path, score):
    seed, L, d, V, frac, lo, hi, block, k = PATHS[path]
    H, W, mask, tokens = _inputs(seed + 100, L, d, V, frac)
    C = oracle.candidate_positions(mask, lo, hi, block)
    st = oracle.readout_rows(H, W, C)
    so = np.sort(oracle_score(st, score))[::-1]
    gap = score_gap(score)
    t_in, j = _clear_tau(so, 0.1, 0.5, gap)
    to_tau = (lambda t: float(np.exp(t))) if score == "conf" else (lambda t: float(t))
    Wt = to_dev(W, H, mask, tokens)[0]
    big_k = len(C)
    rd = _readout(Wt, L, big_k)
    # a threshold inside the score range: n = the rows above it
    g, _, _ = _policy_case(H, W, mask, tokens, big_k, lo, hi, block, score, to_tau(t_in), rd=rd,
                           where=f"thr {path} {score} mid")
    assert g["n"] == j
    # capped by k
    g, _, _ = _policy_case(H, W, mask, tokens, max(1, j // 3), lo, hi, block, score, to_tau(t_in), rd=rd,
                           where=f"thr {path} {score} cap")
    assert g["n"] == max(1, j // 3)
    # above every score: exactly one row (the best) commits
    g, _, _ = _policy_case(H, W, mask, tokens, big_k, lo, hi, block, score, to_tau(so[0] + 1.0), rd=rd,
                           where=f"thr {path} {score} above")
    assert g["n"] == 1
    # below every score: all candidates, up to k
    g, _, _ = _policy_case(H, W, mask, tokens, big_k, lo, hi, block, score, to_tau(so[-1] - 1.0), rd=rd,
                           where=f"thr {path} {score} below")
    assert g["n"] == len(C)


def test_threshold_degenerate_cases():
    H, W, mask, tokens = _inputs(31, 300, 64, 500, 0.5)
    L = len(mask)
    Wt = to_dev(W, H, mask, tokens)[0]
    rd = _readout(Wt, L, 64)
    for score in SCORES:
        g, _, _ = _policy_case(H, W, np.zeros(L, np.uint8), tokens, 5, score=score, tau=0.5, rd=rd,
                               where=f"M=0 {score}")
        assert g["n"] == 0 and g["M"] == 0
        g, _, _ = _policy_case(H, W, mask, tokens, 0, score=score, tau=-1e30, rd=rd, where=f"k=0 {score}")
        assert g["n"] == 0
        one = np.zeros(L, np.uint8)
        one[77] = 1
        g, _, _ = _policy_case(H, W, one, tokens, 5, score=score, tau=1e30, rd=rd, where=f"M=1 {score}")
        assert g["n"] == 1 and list(g["sel_idx"]) == [77]
        # few-row path, same rules
        g, _, _ = _policy_case(H, W, mask, tokens, 8, 0, 30, score=score, tau=1e30, rd=rd,
                               where=f"few rows above {score}")
        assert g["n"] == 1


def test_identical_rows_threshold_commits_lowest_positions():
    """Equal scores: the rule counts all of them, the cap keeps the lowest positions."""
    rng = np.random.default_rng(33)
    L, d, V = 500, 128, 1500
    row = WL.bf16_round(rng.standard_normal(d).astype(np.float32) * 4)
    H = np.tile(row, (L, 1))
    W = WL.bf16_round((rng.standard_normal((V, d)) * 0.05).astype(np.float32))
    mask = (rng.random(L) < 0.7).astype(np.uint8)
    tokens = np.full(L, V, np.int32)
    for score in SCORES:
        g, _, _ = _policy_case(H, W, mask, tokens, 40, score=score, tau=-1e30, where=f"identical {score}")
        assert list(g["sel_idx"]) == list(np.flatnonzero(mask)[:40])
        assert len(set(g["row_margin"].tolist())) == 1 and len(set(g["row_entropy"].tolist())) == 1


def test_exact_argmax_ties_give_zero_margin():
    """Duplicated W_lm rows give bit-identical largest logits: the margin is
    exactly 0 (the second-largest logit equals the largest)."""
    rng = np.random.default_rng(35)
    L, d, V = 260, 64, 2000
    H, W, mask, tokens = _inputs(35, L, d, V, 1.0)
    o = oracle.readout_rows(H, W, np.arange(L))
    W2 = W.copy()
    for t in np.unique(o["tok"])[:40]:
        dst = min(V - 1, int(t) + 700)
        if dst != t:
            W2[dst] = W[t]
    o2 = oracle.readout_rows(H, W2, np.arange(L))
    tie = o2["gap2"] == 0.0
    assert tie.sum() >= 20
    for slices in (1, 3, 8):
        Wt, Ht, mt, tt = to_dev(W2, H, mask, tokens)
        rd = _readout(Wt, L, 8)
        rd.set_slices(slices)
        g = run_step(rd, Ht, mt, tt, 8, 0, L, score="margin", ext=True)
        assert np.all(g["row_margin"][tie] == 0.0)
        assert np.all(g["row_margin"][~tie] > 0.0)
        check_ext_rows(g["row_margin"], g["row_entropy"], o2, f"ties slices={slices}")


def test_zero_rows_closed_form():
    """All-zero hidden rows: every logit is 0, so p = 1/V, entropy = ln V,
    margin = 0, lse = ln V (closed form, on every GEMM variant)."""
    for d, lo, hi in ((256, 0, 300), (200, 0, 300), (256, 10, 40)):
        L, V = 300, 3001
        H = np.zeros((L, d), np.uint16)
        W = WL.bf16_round((np.random.default_rng(37).standard_normal((V, d)) * 0.05).astype(np.float32))
        mask = np.ones(L, np.uint8)
        tokens = np.full(L, V, np.int32)
        Wt, Ht, mt, tt = to_dev(W, H, mask, tokens)
        rd = _readout(Wt, L, 4)
        g = run_step(rd, Ht, mt, tt, 4, lo, hi, score="neg_entropy", ext=True)
        np.testing.assert_allclose(g["row_entropy"], np.log(V), rtol=1e-6)
        np.testing.assert_allclose(g["row_lse"], np.log(V), rtol=1e-6)
        np.testing.assert_allclose(g["row_conf"], 1.0 / V, rtol=1e-5)
        assert np.all(g["row_margin"] == 0.0) and np.all(g["row_tok"] == 0)
        assert list(g["sel_idx"]) == list(range(lo, lo + 4))


def test_ext_statistics_do_not_change_confidence_ranking():
    """Asking for margin / entropy outputs keeps the confidence path's results."""
    H, W, mask, tokens = _inputs(39, 900, 256, 6000, 0.8)
    L = len(mask)
    Wt, Ht, mt, tt = to_dev(W, H, mask, tokens)
    rd = _readout(Wt, L, 32)
    for lo, hi in ((0, L), (200, 232)):
        a = run_step(rd, Ht, mt.clone(), tt.clone(), 32, lo, hi)
        b = run_step(rd, Ht, mt.clone(), tt.clone(), 32, lo, hi, ext=True)
        for key in ("row_idx", "row_tok", "sel_idx", "sel_tok", "mask", "tokens"):
            np.testing.assert_array_equal(a[key], b[key])
        np.testing.assert_allclose(a["row_conf"], b["row_conf"], rtol=1e-6)
        np.testing.assert_allclose(a["row_lse"], b["row_lse"], rtol=1e-6)


def test_policy_slice_invariance():
    H, W, mask, tokens = _inputs(41, 900, 256, 6000, 0.8)
    L = len(mask)
    Wt, Ht, mt, tt = to_dev(W, H, mask, tokens)
    rd = _readout(Wt, L, 32)
    ref = None
    for slices in (1, 2, 7, 23, 0):
        rd.set_slices(slices)
        g = run_step(rd, Ht, mt.clone(), tt.clone(), 32, 0, L, score="margin", ext=True)
        if ref is None:
            ref = g
            continue
        np.testing.assert_array_equal(g["row_tok"], ref["row_tok"])
        np.testing.assert_allclose(g["row_margin"], ref["row_margin"], rtol=1e-4, atol=1e-7)
        np.testing.assert_allclose(g["row_entropy"], ref["row_entropy"], rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("score,tau", [("conf", None), ("margin", 0.05)])
def test_largest_k(score, tau):
    """k = k_max = 4096, the largest the library accepts, with about 6400
    candidates: the selection holds 4096 winners in LDS and sorts them."""
    import masked_token_logits_amd as mtl
    k = mtl.DLLM_K_MAX_LIMIT
    H, W, mask, tokens = _inputs(77, 8000, 64, 500, 0.8)
    g, o, _ = _policy_case(H, W, mask, tokens, k, score=score, tau=tau, where=f"k=4096 {score} {tau}")
    assert g["M"] > k


@pytest.mark.parametrize("V", [2, 7, 31])
@pytest.mark.parametrize("path", sorted(PATHS))
def test_small_vocabulary(path, V):
    """Vocabularies smaller than one 32-wide MFMA block: every vocabulary
    tile is mostly padding, whose rows are clamped on load and whose logits
    are dropped; all three scores, and a threshold on the margin."""
    _, L, d, _, frac, lo, hi, block, k = PATHS[path]
    H, W, mask, tokens = _inputs(V + L, L, d, V, frac)
    for score, tau in (("conf", None), ("margin", None), ("neg_entropy", None), ("margin", 0.2)):
        _policy_case(H, W, mask, tokens, k, lo, hi, block, score=score, tau=tau,
                     where=f"V={V} {path} {score} {tau}")
