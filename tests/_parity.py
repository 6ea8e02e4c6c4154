"""Helpers shared by the GPU parity tests: upload, one library step, and the
comparison rules against the fp64 oracle.

Comparison rules (floating point decides integers here, so near-ties are
excluded and counted rather than compared):
  * tokens: a row's argmax must equal the oracle's wherever the oracle's gap
    between its two largest logits exceeds GAP (1e-3);
  * confidence and log-sum-exp: |gpu - oracle| <= REL * |oracle| (2e-3);
  * committed set: if the oracle's log-confidence at rank n exceeds the one
    at rank n+1 by more than GAP the sets must be equal; otherwise they must
    agree outside the band of rows whose oracle log-confidence lies within
    GAP of that boundary, and hold exactly n positions.  Sets are compared,
    rank order only where the oracle's neighbouring scores differ by > GAP.
  * margin and entropy (the other ranking scores): a relative error of REL
    on a probability is an absolute error of REL on its logarithm, so the
    entropy (an expectation of -log p) is held to REL nats absolute, and the
    margin p1 - p2 to REL * (p1 + p2).  Selections ranked by them use the
    same band rule with band widths MARGIN_GAP (probability) and
    ENTROPY_GAP (nats).
  * threshold selection: the library's n must equal the clamped count of its
    own float32 scores >= tau (the same precision decides on both sides),
    and lie between the oracle's counts at tau + gap and tau - gap.
"""
from __future__ import annotations

import numpy as np

GAP = 1e-3
REL = 2e-3
MARGIN_GAP = 2e-3
ENTROPY_GAP = 2e-3


def to_dev(W, H, mask, tokens):
    import torch
    dev = torch.device("cuda", 0)
    Wt = torch.from_numpy(np.ascontiguousarray(W).view(np.int16)).to(dev)
    Ht = torch.from_numpy(np.ascontiguousarray(H).view(np.int16)).to(dev)
    mt = torch.from_numpy(np.ascontiguousarray(mask)).to(dev)
    tt = torch.from_numpy(np.ascontiguousarray(tokens)).to(dev)
    return Wt, Ht, mt, tt


def run_step(rd, Ht, mt, tt, k, lo, hi, block=0, score="conf", tau=None, ext=False):
    """One step through the C ABI; returns host copies of every output
    (``ext``: also the per-row margin and entropy)."""
    import torch
    out = rd.outputs(ext=ext)
    rd.step(Ht, mt, tt, k, lo, hi, block, out=out, score=score, tau=tau)
    torch.cuda.synchronize()
    n = int(out["n_out"].item())
    M = int(out["m_out"].item())
    res = dict(n=n, M=M, mask=mt.cpu().numpy(), tokens=tt.cpu().numpy())
    for key in ("sel_idx", "sel_tok", "sel_conf"):
        res[key] = out[key][:n].cpu().numpy()
    for key in ("row_idx", "row_tok", "row_conf", "row_lse", "row_margin", "row_entropy"):
        if key in out:
            res[key] = out[key][:M].cpu().numpy()
    return res


def oracle_score(st, score):
    """The oracle's ranking score per row (fp64)."""
    return {"conf": st["logconf"], "margin": st["margin"], "neg_entropy": -st["entropy"]}[score]


def score_gap(score):
    """Band width of the selection rule for a score (in its own units)."""
    return {"conf": GAP, "margin": MARGIN_GAP, "neg_entropy": ENTROPY_GAP}[score]


def library_score(g, score):
    """The library's float32 ranking score per row, as its kernels rank by."""
    if score == "conf":
        return g["row_conf"].astype(np.float32)
    if score == "margin":
        return g["row_margin"].astype(np.float32)
    return -g["row_entropy"].astype(np.float32)


def check_ext_rows(g_margin, g_entropy, st, where=""):
    """Margin and entropy parity (tolerances in the module docstring)."""
    p2 = st["conf"] - st["margin"]
    for name, g, lim in (("margin", g_margin, REL * (st["conf"] + p2)),
                         ("entropy", g_entropy, np.full(len(p2), REL))):
        err = np.abs(np.asarray(g, np.float64) - st[name])
        bad = np.flatnonzero(err > lim)
        assert len(bad) == 0, f"{where}: {name} off at rows {bad[:10]}: gpu {np.asarray(g)[bad[:10]]} oracle {st[name][bad[:10]]}"


def check_self_selection(g, score, k, tau=None, where=""):
    """The commit is exactly the library's own top n by its float32 scores
    (position ascending on ties), n = min(k, M) or the threshold rule."""
    M = g["M"]
    sc = library_score(g, score)
    n = min(k, M)
    if tau is not None and n > 0:
        cnt = int(np.count_nonzero(sc >= np.float32(tau)))
        n = min(max(cnt, 1), n)
    assert g["n"] == n, f"{where}: n {g['n']} vs {n} from the library's own scores"
    order = np.lexsort((g["row_idx"], -sc.astype(np.float64)))
    np.testing.assert_array_equal(g["sel_idx"], g["row_idx"][order[:n]])
    np.testing.assert_array_equal(g["sel_tok"], g["row_tok"][order[:n]])
    np.testing.assert_array_equal(g["sel_conf"], g["row_conf"][order[:n]])
    return n


def threshold_n_bounds(score_o, tau, k, gap):
    """Range of n that the threshold rule can give when scores carry an
    error of up to ``gap``."""
    M = len(score_o)
    if M == 0 or k <= 0:
        return 0, 0
    cap = min(k, M)
    lo = min(max(int(np.count_nonzero(score_o >= tau + gap)), 1), cap)
    hi = min(max(int(np.count_nonzero(score_o >= tau - gap)), 1), cap)
    return lo, hi


def check_rows(g_tok, g_conf, g_lse, st, where=""):
    """Per-row parity; returns the number of near-tie rows excluded."""
    g_tok = np.asarray(g_tok)
    clear = st["gap2"] > GAP
    bad = np.flatnonzero(clear & (g_tok != st["tok"]))
    assert len(bad) == 0, f"{where}: token mismatch at rows {bad[:10]} (gpu {g_tok[bad[:10]]}, oracle {st['tok'][bad[:10]]})"
    for name, g in (("conf", g_conf), ("lse", g_lse)):
        o = st[name]
        err = np.abs(np.asarray(g, np.float64) - o)
        lim = REL * np.abs(o)
        badf = np.flatnonzero(err > lim)
        assert len(badf) == 0, f"{where}: {name} off at rows {badf[:10]}: gpu {np.asarray(g)[badf[:10]]} oracle {o[badf[:10]]}"
    return int(np.count_nonzero(~clear))


def oracle_rank(positions, logconf):
    """Positions sorted by score (log-confidence) descending, position ascending."""
    positions = np.asarray(positions, np.int64)
    order = np.lexsort((positions, -np.asarray(logconf, np.float64)))
    return positions[order], np.asarray(logconf, np.float64)[order]


def check_selection(sel_g, positions, logconf, n, where="", gap=GAP):
    """Committed-set parity (see module docstring); returns the band size."""
    sel_g = [int(x) for x in sel_g]
    assert len(sel_g) == n == len(set(sel_g)), f"{where}: expected {n} distinct positions, got {len(sel_g)}"
    ranked, lc = oracle_rank(positions, logconf)
    if n == 0:
        return 0
    sel_o = set(int(x) for x in ranked[:n])
    if n == len(ranked):
        assert set(sel_g) == sel_o, f"{where}: all candidates should commit"
        return 0
    c_n, c_n1 = lc[n - 1], lc[n]
    if c_n - c_n1 > gap:
        assert set(sel_g) == sel_o, f"{where}: committed sets differ: {sorted(set(sel_g) ^ sel_o)[:10]}"
        return 0
    band = set(int(p) for p, c in zip(ranked, lc) if c_n1 - gap <= c <= c_n + gap)
    assert set(sel_g) - band == sel_o - band, f"{where}: committed sets differ outside the near-tie band"
    return len(band)


def check_rank_order(sel_g, positions, logconf, where="", gap=GAP):
    """Rank order of the committed positions where the oracle separates them."""
    pos_to_lc = {int(p): float(c) for p, c in zip(positions, logconf)}
    lcs = [pos_to_lc[int(p)] for p in sel_g]
    for i in range(len(lcs) - 1):
        if lcs[i + 1] - lcs[i] > gap:
            raise AssertionError(f"{where}: rank {i} and {i + 1} out of order ({lcs[i]} < {lcs[i + 1]})")


def check_commit(before_mask, before_tok, res, lo=0, hi=None):
    """Only the committed positions changed, each to its row's token."""
    after_mask, after_tok = res["mask"], res["tokens"]
    sel = np.asarray(res["sel_idx"], np.int64)
    changed = np.flatnonzero((after_mask != before_mask) | (after_tok != before_tok))
    assert set(changed) <= set(sel.tolist())
    assert np.all(after_mask[sel] == 0) and np.all(before_mask[sel] != 0)
    np.testing.assert_array_equal(after_tok[sel], res["sel_tok"])
    if hi is not None:
        assert np.all((sel >= lo) & (sel < hi))


def run_batch(rd, Ht, mt, tt, seqs, block=0, score="conf", tau=None, ext=False):
    """One batched step through the C ABI; returns one result dict per
    sequence, shaped like run_step's."""
    import torch
    B, L = int(Ht.shape[0]), int(Ht.shape[1])
    out = rd.outputs_batch(B, L, ext=ext)
    rd.step_batch(Ht, mt, tt, seqs, block, out=out, score=score, tau=tau)
    torch.cuda.synchronize()
    host = {key: v.cpu().numpy() for key, v in out.items()}
    mask, tokens = mt.cpu().numpy(), tt.cpu().numpy()
    res = []
    for b in range(B):
        n, M = int(host["n_out"][b]), int(host["m_out"][b])
        r = dict(n=n, M=M, mask=mask[b], tokens=tokens[b])
        for key in ("sel_idx", "sel_tok", "sel_conf"):
            r[key] = host[key][b, :n]
        for key in ("row_idx", "row_tok", "row_conf", "row_lse", "row_margin", "row_entropy"):
            if key in host:
                r[key] = host[key][b, :M]
        res.append(r)
    return res
