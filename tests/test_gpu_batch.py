"""GPU parity of the batched readout (B sequences sharing one pass over W_lm)
against the fp64 oracle, sequence by sequence: every GEMM variant (few rows,
persistent, streaming fallback), windows, blocks, per-sequence k, empty
sequences, the scores and threshold commits, a carried semi-autoregressive
loop, the largest batch, and agreement with B single-sequence steps.  Every
call goes through the C ABI (dllm_masked_readout_step_batch)."""
import numpy as np
import pytest

import oracle
import workloads as WL
from _parity import (check_commit, check_ext_rows, check_rank_order, check_rows, check_selection,
                     check_self_selection, oracle_score, run_batch, run_step, score_gap, threshold_n_bounds,
                     to_dev)

pytestmark = pytest.mark.gpu


def _readout(Wt, L_max, k_max):
    import masked_token_logits_amd as mtl
    return mtl.MaskedReadout(Wt, L_max, k_max)


def _inputs(seed, B, L, d, V, frac, spread=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, L, d)).astype(np.float32)
    if spread:   # per-row inverse temperature, so the scores spread out
        x *= np.exp(rng.uniform(np.log(0.25), np.log(8.0), size=(B, L, 1))).astype(np.float32)
    H = WL.bf16_round(x)
    W = WL.bf16_round((rng.standard_normal((V, d)) * 0.05).astype(np.float32))
    mask = (rng.random((B, L)) < frac).astype(np.uint8)
    tokens = rng.integers(0, V, (B, L)).astype(np.int32)
    tokens[mask != 0] = V
    return H, W, mask, tokens


def _check_batch(g, H, W, mask, tokens, seqs, block, score="conf", tau=None, where=""):
    o = oracle.readout_step_batch(H, W, mask, tokens, seqs, block, score=score, tau=tau)
    for b, (k, lo, hi) in enumerate(seqs):
        gb, ob, w = g[b], o[b], f"{where} seq {b}"
        assert gb["M"] == ob.M, f"{w}: M {gb['M']} vs {ob.M}"
        np.testing.assert_array_equal(gb["row_idx"], ob.positions)
        check_rows(gb["row_tok"], gb["row_conf"], gb["row_lse"], ob.stats, w)
        if "row_margin" in gb:
            check_ext_rows(gb["row_margin"], gb["row_entropy"], ob.stats, w)
        n = check_self_selection(gb, score, k, tau, w) if ("row_margin" in gb or score == "conf") else gb["n"]
        so, gap = oracle_score(ob.stats, score), score_gap(score)
        if tau is not None:
            t_o = tau
            if score == "conf":
                t_o = np.log(tau) if tau > 0 else -np.inf
            n_lo, n_hi = threshold_n_bounds(so, t_o, k, gap)
            assert n_lo <= n <= n_hi, f"{w}: threshold n={n} outside [{n_lo}, {n_hi}]"
        else:
            assert n == len(ob.sel), f"{w}: n {n} vs {len(ob.sel)}"
        check_selection(gb["sel_idx"], ob.positions, so, n, w, gap=gap)
        check_rank_order(gb["sel_idx"], ob.positions, so, w, gap=gap)
        check_commit(mask[b], tokens[b], gb, lo, hi)
    return o


# (name, seed, B, L, d, V, frac, block, seqs)
CASES = [
    # <= 32 candidate rows in total: the few-row GEMM and one-workgroup finish
    ("few_rows", 51, 3, 400, 256, 5000, 0.7, 0, [(3, 100, 110), (5, 0, 12), (2, 390, 400)]),
    ("few_rows_blocks", 52, 4, 300, 200, 4097, 0.6, 8, [(2, 0, 300), (8, 100, 300), (0, 0, 300), (1, 40, 48)]),
    # persistent GEMM (d % 32 == 0), ragged rows and vocabulary
    ("persistent", 53, 4, 300, 256, 3001, 0.6, 0, [(40, 0, 300), (7, 50, 250), (0, 0, 300), (25, 299, 299)]),
    ("persistent_blocks", 54, 6, 256, 128, 2000, 0.8, 32,
     [(2, 128, 256), (4, 0, 256), (3, 64, 256), (32, 0, 256), (1, 200, 256), (2, 128, 160)]),
    # streaming fallback (d % 32 != 0)
    ("streaming", 55, 3, 350, 200, 2500, 0.5, 0, [(30, 0, 350), (1, 0, 350), (12, 100, 300)]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_batch_topk_confidence(case):
    name, seed, B, L, d, V, frac, block, seqs = case
    H, W, mask, tokens = _inputs(seed, B, L, d, V, frac)
    Wt, Ht, mt, tt = to_dev(W, H, mask, tokens)
    rd = _readout(Wt, B * L, max(k for k, _, _ in seqs))
    print(f"[case] batch {name} B={B} L={L} d={d} V={V} block={block}", flush=True)
    g = run_batch(rd, Ht, mt, tt, seqs, block)
    _check_batch(g, H, W, mask, tokens, seqs, block, where=name)


@pytest.mark.parametrize("case", [CASES[0], CASES[2], CASES[4]], ids=["few_rows", "persistent", "streaming"])
@pytest.mark.parametrize("score,tau", [("margin", None), ("neg_entropy", None), ("conf", 0.05),
                                       ("margin", 0.3), ("neg_entropy", -4.0)])
def test_batch_policies(case, score, tau):
    name, seed, B, L, d, V, frac, block, seqs = case
    H, W, mask, tokens = _inputs(seed + 10, B, L, d, V, frac)
    Wt, Ht, mt, tt = to_dev(W, H, mask, tokens)
    rd = _readout(Wt, B * L, max(k for k, _, _ in seqs))
    print(f"[case] batch {name} score={score} tau={tau}", flush=True)
    g = run_batch(rd, Ht, mt, tt, seqs, block, score=score, tau=tau, ext=True)
    _check_batch(g, H, W, mask, tokens, seqs, block, score=score, tau=tau, where=f"{name} {score} {tau}")


def test_batch_semi_ar_loop_carried_state():
    """8 sequences in the LLaDA-like block decoding shape (suffix masked,
    blocks of 32, k=2), each at its own stage, 20 steps with the state
    carried on the device; every step checked against the oracle run on the
    state the step started from."""
    B, L, d, V = 8, 256, 128, 3000
    H, W, _, _ = _inputs(57, B, L, d, V, 0.0, spread=False)
    mask = np.zeros((B, L), np.uint8)
    mask[:, 128:] = 1
    for b in range(B):            # stagger: sequence b has already committed 3 b positions of its first block
        mask[b, 128:128 + 3 * b] = 0
    tokens = np.full((B, L), V, np.int32)
    seqs = [(2, 128, L)] * B
    Wt, Ht, mt, tt = to_dev(W, H, mask, tokens)
    rd = _readout(Wt, B * L, 2)
    rng = np.random.default_rng(58)
    import torch
    for t in range(20):
        Hs = WL.bf16_round(rng.standard_normal((B, L, d)).astype(np.float32))
        Ht = torch.from_numpy(Hs.view(np.int16)).cuda()
        before_m, before_t = mt.cpu().numpy(), tt.cpu().numpy()
        g = run_batch(rd, Ht, mt, tt, seqs, 32)
        _check_batch(g, Hs, W, before_m, before_t, seqs, 32, where=f"semi-AR step {t}")
    final = mt.cpu().numpy()
    for b in range(B):
        # count the commits the block rule allows: min(k, masked left in the current block) per step
        left = [int(mask[b, 128 + 32 * j:160 + 32 * j].sum()) for j in range(4)]
        done = 0
        for _ in range(20):
            j = next((j for j in range(4) if left[j] > 0), None)
            if j is None:
                break
            c = min(2, left[j])
            left[j] -= c
            done += c
        assert final[b, :128].sum() == 0
        assert final[b, 128:].sum() == int(mask[b, 128:].sum()) - done


def test_batch_largest_batch_and_empty_sequences():
    """B = DLLM_BATCH_MAX sequences, most of them with nothing to commit."""
    import masked_token_logits_amd as mtl
    B, L, d, V = mtl.DLLM_BATCH_MAX, 24, 64, 700
    H, W, mask, tokens = _inputs(59, B, L, d, V, 0.3)
    seqs = [((b % 4), 0, L if b % 3 else 0) for b in range(B)]
    Wt, Ht, mt, tt = to_dev(W, H, mask, tokens)
    rd = _readout(Wt, B * L, 4)
    for block in (0, 8):
        g = run_batch(rd, Ht, mt.clone(), tt.clone(), seqs, block)
        _check_batch(g, H, W, mask, tokens, seqs, block, where=f"B={B} block={block}")


def test_batch_matches_single_sequence_steps():
    """The batched step commits what B single-sequence steps of the library
    commit, token for token where the scores are separated."""
    B, L, d, V = 5, 320, 256, 4000
    H, W, mask, tokens = _inputs(61, B, L, d, V, 0.7)
    seqs = [(8, 0, L), (3, 20, 300), (0, 0, L), (12, 0, L), (1, 310, 320)]
    Wt, Ht, mt, tt = to_dev(W, H, mask, tokens)
    rd = _readout(Wt, B * L, 12)
    g = run_batch(rd, Ht, mt, tt, seqs, 0)
    o = oracle.readout_step_batch(H, W, mask, tokens, seqs, 0)
    for b, (k, lo, hi) in enumerate(seqs):
        import torch
        rs = _readout(Wt, L, 12)
        s = run_step(rs, Ht[b].contiguous(), torch.from_numpy(mask[b]).cuda(), torch.from_numpy(tokens[b]).cuda(),
                     k, lo, hi)
        np.testing.assert_array_equal(g[b]["row_idx"], s["row_idx"])
        clear = o[b].stats["gap2"] > 1e-3
        np.testing.assert_array_equal(g[b]["row_tok"][clear], s["row_tok"][clear])
        np.testing.assert_allclose(g[b]["row_conf"], s["row_conf"], rtol=1e-5)
        lc = o[b].stats["logconf"]
        srt = np.sort(lc)[::-1]
        n = len(o[b].sel)
        if n == 0 or n == len(srt) or srt[n - 1] - srt[n] > 1e-3:
            assert set(g[b]["sel_idx"].tolist()) == set(s["sel_idx"].tolist())


def test_batch_compaction_window_lengths():
    """Windows of 1024 positions and less are compacted from one load per
    lane, longer ones by re-reading passes: block mode on both sides of the
    boundary, a long window whose first masked block lies far in, one with
    none, and an unblocked window just above the boundary."""
    B, L, d, V = 5, 3000, 64, 900
    H, W, _, _ = _inputs(63, B, L, d, V, 0.0, spread=False)
    rng = np.random.default_rng(64)
    mask = np.zeros((B, L), np.uint8)
    mask[0, 700:1024] = rng.random(324) < 0.5          # window [0, 1024): one load
    mask[1, 1010:1030] = 1                               # window [0, 1025): passes; first block at 992
    mask[2, 2601:2700] = rng.random(99) < 0.6            # window [0, 3000): first block far in
    mask[2, 2600] = 1
    mask[4, 100:1100] = rng.random(1000) < 0.03          # unblocked window [100, 1125)
    tokens = np.full((B, L), V, np.int32)
    seqs = [(3, 0, 1024), (2, 0, 1025), (4, 0, 3000), (2, 0, 3000), (40, 100, 1125)]
    Wt, Ht, mt, tt = to_dev(W, H, mask, tokens)
    rd = _readout(Wt, B * L, 40)
    for block in (32, 0):
        print(f"[case] batch compaction window lengths block={block}", flush=True)
        g = run_batch(rd, Ht, mt.clone(), tt.clone(), seqs, block)
        _check_batch(g, H, W, mask, tokens, seqs, block, where=f"window lengths block={block}")
