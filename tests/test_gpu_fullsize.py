"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.

* LLaDA-like semi-AR loop (L=4096, d=4096, V=126464, k=2, blocks of 32, 32
  steps, hidden re-drawn per step): every step is checked against the oracle
  run on the same state, all rows.
* Dream-like (L=8192, d=3584, V=152064, k=64), long-context low-mask
  (L=131072, M=13107, k=256) and high-mask (M=117965, k=1024, 5% planted
  rows): the oracle cannot afford all rows, so it checks sampled rows, every
  committed row and the rows just below the commit boundary; properties
  that hold at any size check the rest (the committed set is the top n of
  the library's own confidences, and no row outside the checked set can
  reach the boundary within the tolerance).
* The batched LLaDA-like workload (16 such sequences per step, one pass over
  W_lm): two steps (512 and 480 candidate rows, the persistent GEMM); four
  of the sequences against the oracle on every row, all sixteen by the
  properties that hold at any size.
"""
import numpy as np
import pytest

import oracle
import workloads as WL
from _parity import (GAP, REL, check_commit, check_rank_order, check_rows, check_selection, check_self_selection,
                     run_batch, run_step, to_dev)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _readout(Wt, L_max, k_max):
    import masked_token_logits_amd as mtl
    return mtl.MaskedReadout(Wt, L_max, k_max)


def test_llada_semi_ar_32_steps():
    cfg = WL.WORKLOADS["llada_like_semi_ar"]
    W = WL.w_lm(cfg)
    W64 = oracle.widen_bf16(W)
    mask, tokens = WL.initial_state(cfg)
    Wt, _, mt, tt = to_dev(W, np.zeros((1, cfg.d), np.uint16), mask, tokens)
    rd = _readout(Wt, cfg.L, cfg.k)
    lo, hi = cfg.win
    total_band = total_ties = 0
    for t in range(cfg.steps):
        H, _ = WL.hidden(cfg, W, t)
        import torch
        Ht = torch.from_numpy(H.view(np.int16)).cuda()
        before_m, before_t = mt.cpu().numpy(), tt.cpu().numpy()
        g = run_step(rd, Ht, mt, tt, cfg.k, lo, hi, cfg.block)
        o = oracle.readout_step(H, W, before_m, before_t, cfg.k, lo, hi, cfg.block, W64=W64)
        where = f"llada step {t}"
        assert g["M"] == o.M == 32 - 2 * (t % 16), where
        np.testing.assert_array_equal(g["row_idx"], o.positions)
        total_ties += check_rows(g["row_tok"], g["row_conf"], g["row_lse"], o.stats, where)
        total_band += check_selection(g["sel_idx"], o.positions, o.stats["logconf"], len(o.sel), where)
        check_rank_order(g["sel_idx"], o.positions, o.stats["logconf"], where)
        check_commit(before_m, before_t, g, lo, hi)
        print(f"[llada] step {t} M={g['M']} ok", flush=True)
    final = mt.cpu().numpy()
    assert final[lo:lo + 64].sum() == 0 and final[lo + 64:hi].all() and final[:lo].sum() == 0
    print(f"llada: near-tie rows {total_ties}, band rows {total_band}")


def _sampled_case(name, n_random=384, n_boundary=256):
    import torch
    cfg = WL.WORKLOADS[name]
    print(f"[case] full-size {name}: generating", flush=True)
    inp = WL.make(cfg)
    Wt, Ht, mt, tt = to_dev(inp.W, inp.H, inp.mask, inp.tokens)
    rd = _readout(Wt, cfg.L, cfg.k)
    g = run_step(rd, Ht, mt, tt, cfg.k, 0, cfg.L)
    del Ht
    torch.cuda.empty_cache()
    M = int(inp.mask.sum())
    n = min(cfg.k, M)
    assert g["M"] == M and g["n"] == n
    np.testing.assert_array_equal(g["row_idx"], np.flatnonzero(inp.mask))
    check_commit(inp.mask, inp.tokens, g)

    # (1) the commit is the library's own top n (confidence desc, position asc), bit-exact
    keys = np.lexsort((g["row_idx"], -g["row_conf"].astype(np.float64)))
    np.testing.assert_array_equal(g["sel_idx"], g["row_idx"][keys[:n]])
    np.testing.assert_array_equal(g["sel_conf"], g["row_conf"][keys[:n]])

    # (2) oracle rows: committed, just below the boundary, and a random sample
    rng = np.random.default_rng(1000 + cfg.id)
    if n < M:
        # every row whose library confidence could, within the tolerances, still
        # reach the oracle's boundary (with a safety factor), at least n_boundary
        c_nG = float(g["row_conf"][keys[n - 1]])
        thr = c_nG * (1 - REL) ** 2 * np.exp(-GAP) * 0.995
        n_close = int(np.count_nonzero(g["row_conf"][keys[n:]] >= thr))
        n_boundary = max(n_boundary, n_close + 1)
    boundary = keys[n:n + n_boundary]
    sample = rng.choice(M, size=min(n_random, M), replace=False)
    rows = np.unique(np.concatenate([keys[:n], boundary, sample]))
    print(f"[case] {name}: oracle on {len(rows)} rows", flush=True)
    st = oracle.readout_rows(inp.H, inp.W, g["row_idx"][rows])
    ties = check_rows(g["row_tok"][rows], g["row_conf"][rows], g["row_lse"][rows], st, f"{name}")

    # (3) no unchecked row can reach the oracle's top n: every unchecked row has a
    # library confidence at or below the last boundary row's, and the sampled
    # rows bound the library's relative error by REL.
    if M > n + n_boundary:
        c_edge = float(g["row_conf"][keys[n + n_boundary - 1]])
        c_min_sel = float(st["conf"][np.searchsorted(rows, keys[:n])].min())
        assert c_edge / (1 - REL) < c_min_sel * np.exp(-GAP), \
            f"{name}: boundary set too small to exclude unchecked rows"
    band = check_selection(g["sel_idx"], g["row_idx"][rows], st["logconf"], n, f"{name}")
    check_rank_order(g["sel_idx"], g["row_idx"][rows], st["logconf"], f"{name}")
    print(f"{name}: M={M} n={n} checked rows={len(rows)} near-tie rows={ties} band rows={band}")
    return inp, g


def test_dream_like_sampled():
    _sampled_case("dream_like")


def test_long_context_low_mask_sampled():
    _sampled_case("long_ctx_low_mask")


def test_long_context_high_mask_planted():
    inp, g = _sampled_case("long_ctx_high_mask")
    P = inp.plant
    planted = dict(zip(P.rows.tolist(), P.tokens.tolist()))
    # independent of the oracle: committed rows are planted rows with their planted token
    for pos, tok in zip(g["sel_idx"], g["sel_tok"]):
        assert int(pos) in planted, f"committed position {pos} is not planted"
        assert planted[int(pos)] == int(tok)
    # every planted masked row reads out its planted token
    pos_to_row = {int(p): i for i, p in enumerate(g["row_idx"])}
    masked_planted = [p for p in P.rows.tolist() if inp.mask[p]]
    got = np.array([g["row_tok"][pos_to_row[p]] for p in masked_planted])
    want = np.array([planted[p] for p in masked_planted])
    np.testing.assert_array_equal(got, want)


def test_llada_batch16_two_steps():
    import torch
    cfg = WL.WORKLOADS["llada_like_semi_ar_batch16"]
    B, L = cfg.batch, cfg.L
    W = WL.w_lm(cfg)
    W64 = oracle.widen_bf16(W)
    states = [WL.initial_state(cfg, b) for b in range(B)]
    mask = np.stack([m for m, _ in states])
    tokens = np.stack([t for _, t in states])
    Wt, _, mt, tt = to_dev(W, np.zeros((1, cfg.d), np.uint16), mask, tokens)
    rd = _readout(Wt, B * L, cfg.k)
    lo, hi = cfg.win
    seqs = [(cfg.k, lo, hi)] * B
    for t in range(2):
        print(f"[case] llada batch16 step {t}: generating", flush=True)
        H = WL.hidden_batch(cfg, W, t)
        Ht = torch.from_numpy(H.view(np.int16)).cuda()
        before_m, before_t = mt.cpu().numpy(), tt.cpu().numpy()
        g = run_batch(rd, Ht, mt, tt, seqs, cfg.block)
        del Ht
        for b in range(B):
            where = f"batch16 step {t} seq {b}"
            assert g[b]["M"] == 32 - 2 * t, where
            check_self_selection(g[b], "conf", cfg.k, None, where)
            check_commit(before_m[b], before_t[b], g[b], lo, hi)
        for b in (0, 5, 10, 15):
            where = f"batch16 step {t} seq {b}"
            o = oracle.readout_step(H[b], W, before_m[b], before_t[b], cfg.k, lo, hi, cfg.block, W64=W64)
            np.testing.assert_array_equal(g[b]["row_idx"], o.positions)
            check_rows(g[b]["row_tok"], g[b]["row_conf"], g[b]["row_lse"], o.stats, where)
            check_selection(g[b]["sel_idx"], o.positions, o.stats["logconf"], len(o.sel), where)
            check_rank_order(g[b]["sel_idx"], o.positions, o.stats["logconf"], where)
        print(f"[llada batch16] step {t} ok", flush=True)
