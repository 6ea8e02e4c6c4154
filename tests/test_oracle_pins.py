"""Pins of the fp64 oracle to things other than itself: brute force on tiny
inputs, closed forms, library routines and invariants.

The pages print no worked example of the readout, so every pin here is
mathematical: exact sums of exactly representable products, textbook
softmax / log-sum-exp identities, and selection by repeated linear scan.
"""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
from oracle import readout as O
import workloads as WL


def _bf16_bits_of(x):
    """bf16 bit patterns of float32 values that are exactly representable."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def _rand_bf16(rng, shape, std=1.0):
    return WL.bf16_round((rng.standard_normal(shape) * std).astype(np.float32))


# ----------------------------------------------------------------- bf16 widening

def test_widen_bf16_textbook_values():
    bits = np.array([0x0000, 0x3F80, 0xC000, 0x3F00, 0x4049, 0x7F7F, 0x0001, 0x8000], dtype=np.uint16)
    want = [0.0, 1.0, -2.0, 0.5, 3.140625, 3.3895313892515355e38, 2.0 ** -133, -0.0]
    got = oracle.widen_bf16(bits)
    assert got.dtype == np.float64
    for g, w in zip(got, want):
        assert g == w


# ----------------------------------------------------------------- logits

def test_logits_match_exact_fsum():
    """bf16 x bf16 products are exact in fp64; math.fsum of them is the
    correctly rounded exact logit.  Shapes are non-square so a transposed
    operand cannot pass."""
    rng = np.random.default_rng(11)
    M, d, V = 5, 24, 37
    H = _rand_bf16(rng, (M, d))
    W = _rand_bf16(rng, (V, d), 0.02)
    Z = oracle.logits(oracle.widen_bf16(H), oracle.widen_bf16(W))
    assert Z.shape == (M, V)
    h = oracle.widen_bf16(H)
    w = oracle.widen_bf16(W)
    for i in range(M):
        for v in range(V):
            exact = math.fsum(float(h[i, j]) * float(w[v, j]) for j in range(d))
            scale = math.fsum(abs(float(h[i, j]) * float(w[v, j])) for j in range(d))
            assert abs(Z[i, v] - exact) <= 1e-12 * scale + 1e-300


# ----------------------------------------------------------------- per-row statistics

def _brute_row(z):
    """Pure-Python readout of one row of logits."""
    V = len(z)
    best, tok = z[0], 0
    for v in range(1, V):
        if z[v] > best:
            best, tok = z[v], v
    other = max((z[v] for v in range(V) if v != tok), default=-math.inf)
    e = [math.exp(z[v] - best) for v in range(V)]
    s = math.fsum(e)
    p = [x / s for x in e]
    p_sorted = sorted(p, reverse=True)
    ent = -math.fsum(x * math.log(x) for x in p if x > 0)
    return dict(tok=tok, mx=best, gap2=best - other, conf=p[tok], lse=best + math.log(s),
                margin=p[tok] - (p_sorted[1] if V > 1 else 0.0), entropy=ent)


def test_row_stats_brute_force():
    rng = np.random.default_rng(3)
    Z = rng.standard_normal((9, 53)) * 3.0
    Z[4, 10] = Z[4, 30] = Z[4].max() + 1.0          # duplicated maximum
    st = oracle.row_stats(Z)
    for i in range(Z.shape[0]):
        b = _brute_row(list(Z[i]))
        assert st["tok"][i] == b["tok"]
        for key in ("mx", "gap2", "conf", "lse", "margin", "entropy"):
            assert st[key][i] == pytest.approx(b[key], rel=1e-12, abs=1e-12), key
    assert st["tok"][4] == 10 and st["gap2"][4] == 0.0


def test_readout_rows_chunks_match_brute_force():
    """The chunked readout (row_chunk = 7 over 23 unsorted positions: three
    full chunks and a ragged one) gives per position exactly the pure-Python
    readout of its exact logits (math.fsum of exact bf16 products), in the
    order the positions were given, and bit for bit what one chunk gives."""
    rng = np.random.default_rng(17)
    L, d, V = 40, 16, 50
    H = _rand_bf16(rng, (L, d))
    W = _rand_bf16(rng, (V, d), std=0.5)
    pos = rng.permutation(L)[:23]
    st7 = oracle.readout_rows(H, W, pos, row_chunk=7)
    st1 = oracle.readout_rows(H, W, pos, row_chunk=1000)
    for key in st1:
        assert np.array_equal(st7[key], st1[key]), key
    Hf = oracle.widen_bf16(H)
    Wf = oracle.widen_bf16(W)
    for i, p in enumerate(pos):
        z = [math.fsum(float(a) * float(b) for a, b in zip(Hf[p], Wf[v])) for v in range(V)]
        b = _brute_row(z)
        assert st7["tok"][i] == b["tok"], i
        for key in ("mx", "conf", "lse", "margin", "entropy"):
            assert st7[key][i] == pytest.approx(b[key], rel=1e-12, abs=1e-12), (i, key)


def test_zero_row_closed_form():
    for V in (1, 2, 7, 4096):
        st = oracle.row_stats(np.zeros((1, V)))
        assert st["tok"][0] == 0
        assert st["conf"][0] == pytest.approx(1.0 / V, rel=1e-15)
        assert st["lse"][0] == pytest.approx(math.log(V), rel=1e-15, abs=1e-300)
        assert st["entropy"][0] == pytest.approx(math.log(V), rel=1e-12, abs=1e-15)
        if V > 1:
            assert st["gap2"][0] == 0.0 and st["margin"][0] == 0.0


@pytest.mark.parametrize("delta", [2.5, 0.75, -1.5, 9.0])
def test_two_level_logits_closed_form(delta):
    """W rows a * e_v (d >= V) and h = (delta / a) e_0 give z = (delta, 0, .., 0)
    through the full step, so every statistic has a closed form."""
    V, d, a = 6, 8, 0.5
    W = np.zeros((V, d), dtype=np.float32)
    for v in range(V):
        W[v, v] = a
    h = np.zeros((1, d), dtype=np.float32)
    h[0, 0] = delta / a
    res = oracle.readout_step(_bf16_bits_of(h), _bf16_bits_of(W), np.array([1], np.uint8),
                              np.array([V], np.int32), k=1)
    st = res.stats
    q = math.exp(-abs(delta))
    if delta > 0:
        conf = 1.0 / (1.0 + (V - 1) * q)
        lse = delta + math.log(1.0 + (V - 1) * q)
        tok, margin = 0, conf * (1.0 - q)
        ent = -(conf * math.log(conf) + (V - 1) * (q * conf) * math.log(q * conf))
    else:
        conf = 1.0 / (q + V - 1)
        lse = math.log(q + V - 1)
        tok, margin = 1, 0.0                       # zeros tie: lowest index 1
        ent = -((V - 1) * conf * math.log(conf) + q * conf * math.log(q * conf))
    assert st["tok"][0] == tok
    assert st["conf"][0] == pytest.approx(conf, rel=1e-14)
    assert st["lse"][0] == pytest.approx(lse, rel=1e-14)
    assert st["margin"][0] == pytest.approx(margin, rel=1e-12, abs=1e-15)
    assert st["entropy"][0] == pytest.approx(ent, rel=1e-12)
    assert list(res.sel) == [0] and list(res.tokens) == [tok] and list(res.mask) == [0]


def test_softmax_lse_match_scipy():
    rng = np.random.default_rng(5)
    Z = rng.standard_normal((16, 300)) * 4.0
    st = oracle.row_stats(Z)
    lse = scipy.special.logsumexp(Z, axis=1)
    P = scipy.special.softmax(Z, axis=1)
    np.testing.assert_allclose(st["lse"], lse, rtol=1e-14)
    np.testing.assert_allclose(st["conf"], P.max(axis=1), rtol=1e-13)
    np.testing.assert_allclose(st["entropy"], scipy.stats.entropy(P, axis=1), rtol=1e-12)


def test_invariants_random():
    rng = np.random.default_rng(9)
    for V in (2, 17, 1000):
        Z = rng.standard_normal((64, V)) * rng.uniform(0.1, 20.0)
        st = oracle.row_stats(Z)
        np.testing.assert_allclose(st["conf"], np.exp(st["mx"] - st["lse"]), rtol=1e-12)
        assert np.all(st["conf"] > 0) and np.all(st["conf"] <= 1.0)
        assert np.all(st["conf"] >= 1.0 / V * (1 - 1e-12))
        assert np.all(st["lse"] >= st["mx"]) and np.all(st["lse"] <= st["mx"] + math.log(V) + 1e-12)
        assert np.all(st["gap2"] >= 0)
        assert np.all(st["margin"] >= 0) and np.all(st["margin"] <= st["conf"])
        assert np.all(st["entropy"] >= -1e-12) and np.all(st["entropy"] <= math.log(V) + 1e-9)


def test_argmax_ties_go_to_lowest_index():
    rng = np.random.default_rng(21)
    V = 97
    Z = rng.standard_normal((40, V))
    want = []
    for i in range(40):
        idx = np.sort(rng.choice(V, size=rng.integers(2, 6), replace=False))
        Z[i, idx] = Z[i].max() + 0.5
        want.append(idx[0])
    st = oracle.row_stats(Z)
    assert list(st["tok"]) == want
    assert np.all(st["gap2"] == 0.0) and np.all(st["margin"] == 0.0)


# ----------------------------------------------------------------- selection

def _linear_scan_topk(score, positions, k):
    """n rounds of 'largest score, lowest position' by linear scan."""
    left = list(zip(positions, score))
    out = []
    for _ in range(min(k, len(left))):
        best = None
        for j, (p, s) in enumerate(left):
            if best is None or s > left[best][1] or (s == left[best][1] and p < left[best][0]):
                best = j
        out.append(left.pop(best)[0])
    return out


def test_topk_matches_linear_scan_with_heavy_ties():
    rng = np.random.default_rng(4)
    for trial in range(30):
        M = int(rng.integers(0, 80))
        positions = np.sort(rng.choice(1000, size=M, replace=False))
        score = rng.integers(0, 6, size=M) / 8.0     # many exact ties
        k = int(rng.integers(0, 90))
        got = oracle.select_topk(score, positions, k)
        assert list(got) == _linear_scan_topk(list(score), list(positions), k)


def test_threshold_rule_brute_force():
    rng = np.random.default_rng(8)
    for trial in range(30):
        M = int(rng.integers(0, 50))
        positions = np.sort(rng.choice(500, size=M, replace=False))
        score = rng.integers(0, 10, size=M) / 10.0
        tau = float(rng.choice([0.25, 0.55, 0.95, 2.0]))
        cap = int(rng.integers(0, 60))
        got = oracle.select_threshold(score, positions, tau, cap)
        full = _linear_scan_topk(list(score), list(positions), M)
        n_ok = sum(1 for s in score if s >= tau)
        n = 0 if (M == 0 or cap == 0) else min(max(n_ok, 1), cap)
        assert list(got) == full[:n]


def _tiny_inputs(seed, L=48, d=16, V=40, masked_frac=0.5):
    rng = np.random.default_rng(seed)
    H = _rand_bf16(rng, (L, d))
    W = _rand_bf16(rng, (V, d), 0.3)
    mask = (rng.random(L) < masked_frac).astype(np.uint8)
    tokens = rng.integers(0, V, size=L).astype(np.int32)
    tokens[mask != 0] = V
    return H, W, mask, tokens


def test_step_against_brute_force_everything():
    """Whole step by brute force: exact logits, per-row scan, linear-scan
    selection and commit, on all rows of a tiny sequence."""
    for seed in range(6):
        H, W, mask, tokens = _tiny_inputs(seed)
        k = 5 + seed
        res = oracle.readout_step(H, W, mask, tokens, k)
        h, w = oracle.widen_bf16(H), oracle.widen_bf16(W)
        cand = [i for i in range(len(mask)) if mask[i]]
        rows = {}
        for i in cand:
            z = [math.fsum(float(h[i, j]) * float(w[v, j]) for j in range(h.shape[1]))
                 for v in range(w.shape[0])]
            rows[i] = _brute_row(z)
        sel = _linear_scan_topk([rows[i]["conf"] for i in cand], cand, k)
        assert list(res.positions) == cand
        assert list(res.sel) == sel
        for i in range(len(mask)):
            if i in sel:
                assert res.tokens[i] == rows[i]["tok"] and res.mask[i] == 0
            else:
                assert res.tokens[i] == tokens[i] and res.mask[i] == mask[i]


def test_unmasked_rows_do_not_matter():
    """Mask-only logits: changing the hidden state of unmasked rows, or rows
    outside the window, changes nothing."""
    H, W, mask, tokens = _tiny_inputs(17)
    res = oracle.readout_step(H, W, mask, tokens, 4, win_lo=8, win_hi=40)
    H2 = H.copy()
    rng = np.random.default_rng(0)
    for i in range(len(mask)):
        if mask[i] == 0 or not (8 <= i < 40):
            H2[i] = _rand_bf16(rng, H.shape[1])
    res2 = oracle.readout_step(H2, W, mask, tokens, 4, win_lo=8, win_hi=40)
    assert list(res.sel) == list(res2.sel)
    np.testing.assert_array_equal(res.tokens, res2.tokens)
    np.testing.assert_array_equal(res.mask, res2.mask)
    outside = [i for i in range(len(mask)) if not (8 <= i < 40)]
    assert np.all(res.tokens[outside] == tokens[outside]) and np.all(res.mask[outside] == mask[outside])


def test_identical_rows_select_lowest_positions():
    rng = np.random.default_rng(2)
    L, d, V = 64, 16, 50
    row = _rand_bf16(rng, d)
    H = np.tile(row, (L, 1))
    W = _rand_bf16(rng, (V, d), 0.3)
    mask = (rng.random(L) < 0.6).astype(np.uint8)
    tokens = np.full(L, V, np.int32)
    res = oracle.readout_step(H, W, mask, tokens, 7)
    assert list(res.sel) == list(np.flatnonzero(mask)[:7])


def test_special_cases_k0_kbig_m0():
    H, W, mask, tokens = _tiny_inputs(31)
    r0 = oracle.readout_step(H, W, mask, tokens, 0)
    assert len(r0.sel) == 0
    np.testing.assert_array_equal(r0.tokens, tokens)
    np.testing.assert_array_equal(r0.mask, mask)
    M = int(mask.sum())
    rb = oracle.readout_step(H, W, mask, tokens, M + 10)
    assert len(rb.sel) == M and rb.mask.sum() == 0
    assert sorted(rb.sel) == list(np.flatnonzero(mask))
    z = np.zeros_like(mask)
    rz = oracle.readout_step(H, W, z, tokens, 5)
    assert rz.M == 0 and len(rz.sel) == 0
    np.testing.assert_array_equal(rz.tokens, tokens)


def test_scatter_invariants():
    H, W, mask, tokens = _tiny_inputs(12, L=80)
    for k in (1, 3, 10, 100):
        res = oracle.readout_step(H, W, mask, tokens, k)
        flipped = np.flatnonzero(res.mask != mask)
        assert len(flipped) == min(k, int(mask.sum()))
        assert np.all(mask[flipped] == 1) and np.all(res.mask[flipped] == 0)
        changed = np.flatnonzero(res.tokens != tokens)
        assert set(changed) <= set(flipped)
        where = {int(p): i for i, p in enumerate(res.positions)}
        for p in flipped:
            assert res.tokens[p] == res.stats["tok"][where[int(p)]]


# ----------------------------------------------------------------- windows and blocks

def _brute_candidates(mask, lo, hi, block):
    masked = [i for i in range(lo, hi) if mask[i]]
    if block <= 0 or not masked:
        return masked
    b = 0
    while True:
        blo, bhi = lo + b * block, min(lo + (b + 1) * block, hi)
        inside = [i for i in masked if blo <= i < bhi]
        if inside:
            return inside
        b += 1


def test_candidate_positions_window_and_block():
    rng = np.random.default_rng(1)
    for trial in range(200):
        L = int(rng.integers(1, 200))
        mask = (rng.random(L) < rng.uniform(0, 1)).astype(np.uint8)
        lo = int(rng.integers(0, L + 1))
        hi = int(rng.integers(lo, L + 1))
        block = int(rng.choice([0, 1, 5, 32, 64]))
        got = oracle.candidate_positions(mask, lo, hi, block)
        assert list(got) == _brute_candidates(mask, lo, hi, block)


def test_multistep_fixed_hidden_block_order():
    """Fixed hidden, block 32, k 2, 32 steps over a 1024-long masked suffix:
    each block's rows are committed in the step-1 ranking, 2 per step, and
    the 32 steps cover exactly the first two blocks."""
    rng = np.random.default_rng(6)
    L, d, V, suffix, block, k = 1200, 32, 300, 1024, 32, 2
    H = _rand_bf16(rng, (L, d))
    W = _rand_bf16(rng, (V, d), 0.3)
    mask = np.zeros(L, np.uint8)
    mask[L - suffix:] = 1
    tokens = np.full(L, V, np.int32)
    lo, hi = L - suffix, L
    W64 = oracle.widen_bf16(W)
    first = oracle.readout_rows(H, W, np.arange(lo, lo + 2 * block), W64=W64)
    rank0 = list(oracle.select_topk(first["conf"][:block], np.arange(lo, lo + block), block))
    rank1 = list(oracle.select_topk(first["conf"][block:], np.arange(lo + block, lo + 2 * block), block))
    committed = []
    for t in range(32):
        res = oracle.readout_step(H, W, mask, tokens, k, lo, hi, block=block, W64=W64)
        assert res.M == block - 2 * (t % 16)
        committed += list(res.sel)
        mask, tokens = res.mask, res.tokens
    assert committed == rank0 + rank1
    assert mask[lo:lo + 2 * block].sum() == 0 and mask[lo + 2 * block:].all()


def test_step_resume_equals_straight_run():
    """The whole state of the loop is (tokens, mask): 3 + 3 steps equal 6."""
    H, W, mask, tokens = _tiny_inputs(40, L=96)
    m1, t1 = mask, tokens
    for _ in range(6):
        r = oracle.readout_step(H, W, m1, t1, 3, block=16)
        m1, t1 = r.mask, r.tokens
    m2, t2 = mask.copy(), tokens.copy()
    for _ in range(3):
        r = oracle.readout_step(H, W, m2, t2, 3, block=16)
        m2, t2 = r.mask, r.tokens
    saved = (m2.copy(), t2.copy())
    m2, t2 = saved
    for _ in range(3):
        r = oracle.readout_step(H, W, m2, t2, 3, block=16)
        m2, t2 = r.mask, r.tokens
    np.testing.assert_array_equal(m1, m2)
    np.testing.assert_array_equal(t1, t2)


# ----------------------------------------------------------------- planted tokens (independent of the oracle)

def test_planted_rows_give_planted_tokens():
    """A small copy of the high-mask long-context workload: the generator's
    plant record (not the oracle) says which token each planted row must
    read out, and planted rows must outrank the rest."""
    cfg = WL.small_config(WL.WORKLOADS["long_ctx_high_mask"], L=4096, d=512, V=4096, k=64)
    inp = WL.make(cfg)
    P = inp.plant
    assert len(P.rows) == round(0.05 * cfg.L)
    st = oracle.readout_rows(inp.H, inp.W, P.rows)
    np.testing.assert_array_equal(st["tok"], P.tokens)
    assert np.median(st["gap2"]) > 6.0
    res = oracle.readout_step(inp.H, inp.W, inp.mask, inp.tokens, cfg.k)
    assert set(res.sel) <= set(P.rows)


# ----------------------------------------------------------------- batched steps

def _brute_step(H, W, mask, tokens, k, lo, hi, block):
    """One step by brute force (exact logits, per-row scan, linear-scan
    selection, commit), windows and blocks included."""
    h, w = oracle.widen_bf16(H), oracle.widen_bf16(W)
    masked = [i for i in range(lo, hi) if mask[i]]
    if block > 0 and masked:
        b_lo = lo + ((masked[0] - lo) // block) * block
        masked = [i for i in masked if b_lo <= i < min(b_lo + block, hi)]
    rows = {}
    for i in masked:
        z = [math.fsum(float(h[i, j]) * float(w[v, j]) for j in range(h.shape[1])) for v in range(w.shape[0])]
        rows[i] = _brute_row(z)
    sel = _linear_scan_topk([rows[i]["conf"] for i in masked], masked, k)
    t2, m2 = tokens.copy(), mask.copy()
    for i in sel:
        t2[i] = rows[i]["tok"]
        m2[i] = 0
    return masked, sel, t2, m2


def test_batch_against_brute_force_per_sequence():
    """Each sequence of a batch gets exactly its own brute-force step: its own
    hidden states, mask, tokens, k and window, never another sequence's."""
    rng = np.random.default_rng(41)
    B, L, d, V = 4, 40, 12, 30
    H = _rand_bf16(rng, (B, L, d))
    W = _rand_bf16(rng, (V, d), 0.3)
    mask = (rng.random((B, L)) < 0.6).astype(np.uint8)
    mask[2] = 0                                   # a sequence with nothing to do
    tokens = rng.integers(0, V, size=(B, L)).astype(np.int32)
    tokens[mask != 0] = V
    seqs = [(3, 0, L), (5, 10, 30), (2, 0, L), (0, 0, L)]
    for block in (0, 8):
        res = oracle.readout_step_batch(H, W, mask, tokens, seqs, block)
        assert len(res) == B
        for b, (k, lo, hi) in enumerate(seqs):
            cand, sel, t2, m2 = _brute_step(H[b], W, mask[b], tokens[b], k, lo, hi, block)
            assert list(res[b].positions) == cand
            assert list(res[b].sel) == sel
            np.testing.assert_array_equal(res[b].tokens, t2)
            np.testing.assert_array_equal(res[b].mask, m2)


def test_batch_permutation_and_independence():
    """Permuting the sequences permutes the results; changing one sequence's
    inputs leaves every other sequence's result unchanged."""
    rng = np.random.default_rng(43)
    B, L, d, V = 5, 64, 16, 50
    H = _rand_bf16(rng, (B, L, d))
    W = _rand_bf16(rng, (V, d), 0.3)
    mask = (rng.random((B, L)) < 0.5).astype(np.uint8)
    tokens = np.full((B, L), V, np.int32)
    seqs = [(int(rng.integers(1, 8)), 0, L) for _ in range(B)]
    base = oracle.readout_step_batch(H, W, mask, tokens, seqs, score="margin")
    perm = rng.permutation(B)
    pr = oracle.readout_step_batch(H[perm], W, mask[perm], tokens[perm], [seqs[i] for i in perm], score="margin")
    for j, i in enumerate(perm):
        assert list(pr[j].sel) == list(base[i].sel)
        np.testing.assert_array_equal(pr[j].tokens, base[i].tokens)
    H2, m2 = H.copy(), mask.copy()
    H2[3] = _rand_bf16(rng, (L, d))
    m2[3] = 1
    ch = oracle.readout_step_batch(H2, W, m2, tokens, seqs, score="margin")
    for b in range(B):
        if b != 3:
            assert list(ch[b].sel) == list(base[b].sel)
            np.testing.assert_array_equal(ch[b].stats["margin"], base[b].stats["margin"])
    # identical sequences give identical results
    Hs = np.repeat(H[:1], B, axis=0)
    same = oracle.readout_step_batch(Hs, W, np.repeat(mask[:1], B, axis=0), np.repeat(tokens[:1], B, axis=0),
                                     [seqs[0]] * B)
    for b in range(1, B):
        assert list(same[b].sel) == list(same[0].sel)
