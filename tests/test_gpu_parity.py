"""GPU parity of the HIP readout against the fp64 oracle at sizes the oracle
finishes in seconds: the tiny workload, ragged shapes (K and vocabulary
tails, partial row tiles), both GEMM variants, windows, blocks, ties and the
degenerate cases.  Every call goes through the C ABI."""
import numpy as np
import pytest

import oracle
import workloads as WL
from _parity import check_commit, check_rank_order, check_rows, check_selection, run_step, to_dev

pytestmark = pytest.mark.gpu


def _readout(Wt, L_max, k_max):
    import masked_token_logits_amd as mtl
    return mtl.MaskedReadout(Wt, L_max, k_max)


def _rand_bf16(rng, shape, std=1.0):
    return WL.bf16_round((rng.standard_normal(shape) * std).astype(np.float32))


def _parity_case(H, W, mask, tokens, k, lo=0, hi=None, block=0, rd=None, slices=None, where=""):
    L = len(mask)
    hi = L if hi is None else hi
    Wt, Ht, mt, tt = to_dev(W, H, mask, tokens)
    if rd is None:
        rd = _readout(Wt, L, max(k, 1))
    if slices is not None:
        rd.set_slices(slices)
    print(f"[case] {where} L={L} d={H.shape[1]} V={W.shape[0]} k={k} win=({lo},{hi}) block={block}", flush=True)
    g = run_step(rd, Ht, mt, tt, k, lo, hi, block)
    o = oracle.readout_step(H, W, mask, tokens, k, lo, hi, block)
    assert g["M"] == o.M, f"{where}: M {g['M']} vs {o.M}"
    np.testing.assert_array_equal(g["row_idx"], o.positions)
    ties = check_rows(g["row_tok"], g["row_conf"], g["row_lse"], o.stats, where)
    band = check_selection(g["sel_idx"], o.positions, o.stats["logconf"], len(o.sel), where)
    check_rank_order(g["sel_idx"], o.positions, o.stats["logconf"], where)
    check_commit(mask, tokens, g, lo, hi)
    # selected confidences are the rows' confidences
    pos_to_row = {int(p): i for i, p in enumerate(g["row_idx"])}
    np.testing.assert_array_equal(g["sel_conf"], g["row_conf"][[pos_to_row[int(p)] for p in g["sel_idx"]]])
    if band == 0:
        np.testing.assert_array_equal(g["mask"], o.mask)
        clear = {int(p) for p, gp in zip(o.positions, o.stats["gap2"]) if gp > 1e-3}
        for p in o.sel:
            if int(p) in clear:
                assert g["tokens"][p] == o.tokens[p]
    return g, o, ties, band


def test_tiny_config_parity():
    inp = WL.make("tiny")
    cfg = inp.cfg
    g, o, ties, band = _parity_case(inp.H, inp.W, inp.mask, inp.tokens, cfg.k, where="tiny")
    assert g["M"] == int(inp.mask.sum()) and g["n"] == cfg.k
    print(f"tiny: M={g['M']} near-tie rows={ties} band={band}")


@pytest.mark.parametrize("seed,L,d,V,frac,k", [
    (0, 700, 200, 1000, 0.5, 17),        # K tail (d % 64 != 0), vocabulary tail, 3 row tiles
    (1, 300, 64, 256, 0.9, 40),          # exact single vocabulary tile
    (2, 1100, 136, 2999, 0.3, 100),      # odd V, several slices
    (3, 513, 512, 700, 1.0, 64),         # fully masked, ragged last row tile
    (4, 257, 8, 33, 0.5, 3),             # d = 8, V < one tile
    (5, 400, 160, 1500, 0.8, 25),        # d = 5 x 32: an odd number of 32-deep K stages
    (6, 600, 320, 1300, 0.7, 30),        # d = 10 x 32
])
def test_ragged_shapes_large_path(seed, L, d, V, frac, k):
    rng = np.random.default_rng(seed)
    H = _rand_bf16(rng, (L, d))
    W = _rand_bf16(rng, (V, d), 0.05)
    mask = (rng.random(L) < frac).astype(np.uint8)
    tokens = rng.integers(0, V, L).astype(np.int32)
    tokens[mask != 0] = V
    _parity_case(H, W, mask, tokens, k, where=f"ragged{seed}")


@pytest.mark.parametrize("seed,L,d,V,lo,hi,block,k", [
    (10, 400, 256, 5000, 100, 132, 0, 5),     # window of 32 -> small path
    (11, 400, 200, 4097, 0, 400, 32, 2),      # block mode, first block
    (12, 4096, 128, 3000, 3072, 4096, 32, 2), # semi-AR suffix window
    (13, 64, 64, 129, 10, 20, 0, 10),         # k > M inside a short window
    (14, 100, 72, 1000, 0, 100, 7, 3),        # odd block size
])
def test_windows_blocks_small_path(seed, L, d, V, lo, hi, block, k):
    rng = np.random.default_rng(seed)
    H = _rand_bf16(rng, (L, d))
    W = _rand_bf16(rng, (V, d), 0.05)
    mask = (rng.random(L) < 0.6).astype(np.uint8)
    if seed == 12:
        mask[:] = 0
        mask[3072:] = 1
        mask[3072:3080] = 0      # first block partly committed already
    tokens = rng.integers(0, V, L).astype(np.int32)
    _parity_case(H, W, mask, tokens, k, lo, hi, block, where=f"window{seed}")


def test_degenerate_cases():
    rng = np.random.default_rng(7)
    L, d, V = 300, 64, 500
    H = _rand_bf16(rng, (L, d))
    W = _rand_bf16(rng, (V, d), 0.05)
    tokens = rng.integers(0, V, L).astype(np.int32)
    mask = (rng.random(L) < 0.5).astype(np.uint8)
    Wt = to_dev(W, H, mask, tokens)[0]
    rd = _readout(Wt, L, 64)
    # M = 0
    _parity_case(H, W, np.zeros(L, np.uint8), tokens, 5, rd=rd, where="M=0")
    # k = 0
    _parity_case(H, W, mask, tokens, 0, rd=rd, where="k=0")
    # empty window
    _parity_case(H, W, mask, tokens, 5, 40, 40, rd=rd, where="empty window")
    # single candidate
    one = np.zeros(L, np.uint8)
    one[123] = 1
    _parity_case(H, W, one, tokens, 5, rd=rd, where="M=1")
    # k >= M: everything commits
    _parity_case(H, W, mask, tokens, 64, 0, 100, rd=rd, where="k>=M")
    # block mode with no masked position
    _parity_case(H, W, np.zeros(L, np.uint8), tokens, 2, 0, L, 32, rd=rd, where="block M=0")


def test_identical_rows_commit_lowest_positions():
    rng = np.random.default_rng(3)
    L, d, V = 600, 128, 1500
    row = _rand_bf16(rng, d)
    H = np.tile(row, (L, 1))
    W = _rand_bf16(rng, (V, d), 0.05)
    mask = (rng.random(L) < 0.7).astype(np.uint8)
    tokens = np.full(L, V, np.int32)
    g, o, _, _ = _parity_case(H, W, mask, tokens, 50, where="identical rows")
    assert list(g["sel_idx"]) == list(np.flatnonzero(mask)[:50])
    assert len(set(g["row_conf"].tolist())) == 1


@pytest.mark.parametrize("k", [50, 700, 1500])
def test_identical_rows_radix_select(k):
    """More than 1024 candidates (the radix-select path) in two groups of
    bit-identical rows: every key shares its score bytes with a third or two
    thirds of the others, so the selection is decided by the row bits alone.
    The commit must be the rows in (score descending, position ascending)
    order, exactly."""
    rng = np.random.default_rng(40 + k)
    L, d, V = 3000, 64, 700
    ra, rb = _rand_bf16(rng, d), _rand_bf16(rng, d)
    H = np.where((np.arange(L) % 3 == 0)[:, None], rb[None, :], ra[None, :]).astype(ra.dtype)
    W = _rand_bf16(rng, (V, d), 0.05)
    mask = (rng.random(L) < 0.7).astype(np.uint8)
    tokens = np.full(L, V, np.int32)
    print(f"[case] identical rows radix k={k} M={int(mask.sum())}", flush=True)
    g, o, _, _ = _parity_case(H, W, mask, tokens, k, where=f"identical radix k={k}")
    assert g["M"] > 1024
    pos = np.flatnonzero(mask)
    conf = g["row_conf"][: g["M"]]
    assert len(set(conf.tolist())) == 2
    order = sorted(range(len(pos)), key=lambda i: (-float(conf[i]), int(pos[i])))
    assert list(g["sel_idx"]) == [int(pos[i]) for i in order[:k]]


def test_argmax_ties_lowest_vocab_index():
    """Duplicate W_lm rows give bit-identical logits; the lowest index must win
    across lanes, tiles and slices."""
    rng = np.random.default_rng(5)
    L, d, V = 260, 64, 2000
    H = _rand_bf16(rng, (L, d))
    W = _rand_bf16(rng, (V, d), 0.05)
    mask = np.ones(L, np.uint8)
    tokens = np.full(L, V, np.int32)
    o = oracle.readout_rows(H, W, np.arange(L))
    # copy each row's argmax W row to a higher and a lower index (lower one wins)
    W2 = W.copy()
    for t in np.unique(o["tok"])[:40]:
        for dst in (int(t) // 3, min(V - 1, int(t) + 700)):
            if dst != t:
                W2[dst] = W[t]
    Wt, Ht, mt, tt = to_dev(W2, H, mask, tokens)
    o2 = oracle.readout_rows(H, W2, np.arange(L))
    exact_tie = o2["gap2"] == 0.0
    decided = exact_tie | (o2["gap2"] > 1e-3)
    assert exact_tie.sum() >= 20
    for slices in (1, 3, 8):
        rd = _readout(Wt, L, 8)
        rd.set_slices(slices)
        g = run_step(rd, Ht, mt.clone(), tt.clone(), 8, 0, L)
        np.testing.assert_array_equal(g["row_tok"][decided], o2["tok"][decided])


def test_slice_count_invariance_and_repeats():
    rng = np.random.default_rng(9)
    L, d, V = 900, 256, 6000
    H = _rand_bf16(rng, (L, d))
    W = _rand_bf16(rng, (V, d), 0.05)
    mask = (rng.random(L) < 0.8).astype(np.uint8)
    tokens = np.full(L, V, np.int32)
    Wt, Ht, mt, tt = to_dev(W, H, mask, tokens)
    rd = _readout(Wt, L, 32)
    ref = None
    for slices in (1, 2, 7, 23, 0):
        rd.set_slices(slices)
        g = run_step(rd, Ht, mt.clone(), tt.clone(), 32, 0, L)
        if ref is None:
            ref = g
            continue
        np.testing.assert_array_equal(g["row_tok"], ref["row_tok"])
        np.testing.assert_allclose(g["row_conf"], ref["row_conf"], rtol=1e-5)
        np.testing.assert_allclose(g["row_lse"], ref["row_lse"], rtol=1e-6)
    rd.set_slices(0)
    first = run_step(rd, Ht, mt.clone(), tt.clone(), 32, 0, L)
    for _ in range(9):
        g = run_step(rd, Ht, mt.clone(), tt.clone(), 32, 0, L)
        for key in ("sel_idx", "sel_tok", "sel_conf", "row_tok", "row_conf", "row_lse", "mask", "tokens"):
            np.testing.assert_array_equal(g[key], first[key])


@pytest.mark.parametrize("M", [33, 63, 64, 65, 96, 127, 128, 129, 160, 200, 255, 256, 257, 300, 383, 385, 511, 513])
def test_persistent_partial_row_tiles(M):
    """Candidate counts around every 32-row block boundary of the 256-row
    tile: waves whose rows are partly or wholly padding skip those blocks."""
    rng = np.random.default_rng(100 + M)
    L, d, V = 600, 128, 1100
    H = _rand_bf16(rng, (L, d))
    W = _rand_bf16(rng, (V, d), 0.05)
    mask = np.zeros(L, np.uint8)
    mask[rng.choice(L, size=M, replace=False)] = 1
    tokens = np.full(L, V, np.int32)
    for slices in (0, 3):
        _parity_case(H, W, mask, tokens, min(M, 20), slices=slices, where=f"M={M} slices={slices}")


def test_few_row_steps_back_to_back():
    """Consecutive single-sequence block steps on one handle (the GEMM finds
    each step's rows itself): a ragged vocabulary of 40 slices, an empty
    step (M = 0) in between, each step checked against the oracle with the
    state carried on the device."""
    import torch
    rng = np.random.default_rng(21)
    L, d, V, block, k = 160, 192, 40 * 128 - 37, 32, 3
    H = _rand_bf16(rng, (L, d))
    W = _rand_bf16(rng, (V, d), 0.05)
    tokens = np.full(L, V, np.int32)
    mask = np.zeros(L, np.uint8)
    mask[64:] = 1
    Wt, Ht, mt, tt = to_dev(W, H, mask, tokens)
    rd = _readout(Wt, L, k)
    for t in range(8):
        lo, hi = (0, 64) if t == 3 else (64, L)  # step 3: nothing masked in the window
        before_m, before_t = mt.cpu().numpy(), tt.cpu().numpy()
        print(f"[case] few-row step {t} win=({lo},{hi})", flush=True)
        g = run_step(rd, Ht, mt, tt, k, lo, hi, block)
        o = oracle.readout_step(H, W, before_m, before_t, k, lo, hi, block)
        where = f"few-row step {t}"
        assert g["M"] == o.M and g["n"] == len(o.sel), where
        np.testing.assert_array_equal(g["row_idx"], o.positions)
        check_rows(g["row_tok"], g["row_conf"], g["row_lse"], o.stats, where)
        band = check_selection(g["sel_idx"], o.positions, o.stats["logconf"], len(o.sel), where)
        check_commit(before_m, before_t, g, lo, hi)
        if band == 0:
            np.testing.assert_array_equal(mt.cpu().numpy(), o.mask)
        else:  # continue from the oracle's state so later steps stay comparable
            mt.copy_(torch.from_numpy(o.mask))
            tt.copy_(torch.from_numpy(o.tokens))
    assert t == 7


@pytest.mark.parametrize("first", [63, 1023, 1024, 4095, 5119, 13007, 19990])
def test_few_row_block_search_long_window(first):
    """Block mode over a long window whose first masked position lies
    anywhere (several search iterations, any lane and any 16-byte group of a
    lane's 64 positions); later masked positions must not be candidates."""
    rng = np.random.default_rng(first)
    L, d, V, block, k = 20000, 64, 700, 32, 3
    H = _rand_bf16(rng, (L, d))
    W = _rand_bf16(rng, (V, d), 0.05)
    tokens = np.full(L, V, np.int32)
    mask = np.zeros(L, np.uint8)
    mask[first] = 1
    mask[first + 1:first + 40:3] = 1   # more in (and past) its block
    mask[min(L - 1, first + 100)] = 1
    _parity_case(H, W, mask, tokens, k, 0, L, block, where=f"long window, first={first}")


@pytest.mark.parametrize("first", [65535, 131000])
def test_few_row_block_search_longest_context(first):
    """The in-GEMM block search over a 131072-position window (the
    long-context length), with the first masked position mid-window or near
    its end."""
    rng = np.random.default_rng(first)
    L, d, V, block, k = 131072, 32, 300, 32, 2
    H = _rand_bf16(rng, (L, d))
    W = _rand_bf16(rng, (V, d), 0.05)
    tokens = np.full(L, V, np.int32)
    mask = np.zeros(L, np.uint8)
    mask[first] = 1
    mask[first + 2:min(L, first + 60):5] = 1
    _parity_case(H, W, mask, tokens, k, 0, L, block, where=f"longest window, first={first}")
