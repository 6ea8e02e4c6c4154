"""State carried across denoising steps on the GPU (the sequence goes from
fully masked to unmasked over T steps: Sparse-dLLM, Method "Inference
background").

* Resume: the loop's whole state is (mask, tokens) in the caller's arrays.
  16 LLaDA-like steps, destroy the handle, create a new one on a workspace
  filled with 0xFF bytes, 16 more steps: every step's commit and the final
  state equal the straight 32-step run bit for bit -- no step reads
  workspace contents an earlier step left behind.  The same holds for a
  persistent-GEMM step (compaction plan, partials, radix select).
* Fixed hidden states: with the same H at every step, block decoding with
  k = 2 commits each 32-position block's rows in the order of the first
  step's confidences, 2 per step, and 32 steps cover exactly the first two
  blocks (the closed form the oracle is pinned to).
"""
import numpy as np
import pytest

import oracle
import workloads as WL
from _parity import GAP, check_rank_order, check_rows, run_step, to_dev

pytestmark = pytest.mark.gpu


def _readout(Wt, L_max, k_max, fill):
    import masked_token_logits_amd as mtl
    rd = mtl.MaskedReadout(Wt, L_max, k_max)
    rd.workspace.fill_(fill)
    return rd


def test_resume_on_dirty_workspace_equals_straight_run():
    import torch
    cfg = WL.WORKLOADS["llada_like_semi_ar"]
    W = WL.w_lm(cfg)
    mask0, tok0 = WL.initial_state(cfg)
    Wt = torch.from_numpy(W.view(np.int16)).cuda()
    Hts = [torch.from_numpy(WL.hidden(cfg, W, t)[0].view(np.int16)).cuda() for t in range(cfg.steps)]
    lo, hi = cfg.win

    def loop(rd, mt, tt, steps):
        out = []
        for t in steps:
            g = run_step(rd, Hts[t], mt, tt, cfg.k, lo, hi, cfg.block)
            out.append((g["sel_idx"].copy(), g["sel_tok"].copy(), g["row_conf"].copy()))
        return out

    print("[case] straight 32-step run on a zeroed workspace", flush=True)
    mt, tt = torch.from_numpy(mask0).cuda(), torch.from_numpy(tok0).cuda()
    rd = _readout(Wt, cfg.L, cfg.k, 0)
    straight = loop(rd, mt, tt, range(32))
    final = (mt.cpu().numpy(), tt.cpu().numpy())
    rd.close()

    print("[case] 16 + 16 steps, each half on a fresh handle over a 0xFF workspace", flush=True)
    mt, tt = torch.from_numpy(mask0).cuda(), torch.from_numpy(tok0).cuda()
    rd1 = _readout(Wt, cfg.L, cfg.k, 0xFF)
    first = loop(rd1, mt, tt, range(16))
    rd1.close()
    del rd1
    rd2 = _readout(Wt, cfg.L, cfg.k, 0xFF)
    second = loop(rd2, mt, tt, range(16, 32))
    rd2.close()
    for t, (a, b) in enumerate(zip(straight, first + second)):
        for x, y, what in zip(a, b, ("sel_idx", "sel_tok", "row_conf")):
            np.testing.assert_array_equal(x, y, err_msg=f"step {t}: {what}")
    np.testing.assert_array_equal(mt.cpu().numpy(), final[0])
    np.testing.assert_array_equal(tt.cpu().numpy(), final[1])


def test_dirty_workspace_persistent_step():
    import torch
    inp = WL.make("tiny")
    cfg = inp.cfg
    res = []
    for fill in (0, 0xFF, 0x7F):
        print(f"[case] tiny whole window, workspace filled with {fill:#x}", flush=True)
        Wt, Ht, mt, tt = to_dev(inp.W, inp.H, inp.mask, inp.tokens)
        rd = _readout(Wt, cfg.L, cfg.k, fill)
        res.append(run_step(rd, Ht, mt, tt, cfg.k, 0, cfg.L))
        rd.close()
        torch.cuda.synchronize()
    for r in res[1:]:
        for key in ("sel_idx", "sel_tok", "row_idx", "row_tok", "row_conf", "row_lse", "mask", "tokens"):
            np.testing.assert_array_equal(r[key], res[0][key], err_msg=key)


def test_fixed_hidden_32_steps_block_order():
    import torch
    cfg = WL.WORKLOADS["llada_like_semi_ar"]
    W = WL.w_lm(cfg)
    H, _ = WL.hidden(cfg, W, 0)
    mask0, tok0 = WL.initial_state(cfg)
    lo, hi, block, k = cfg.win[0], cfg.win[1], cfg.block, cfg.k
    Wt, Ht, mt, tt = to_dev(W, H, mask0, tok0)
    rd = _readout(Wt, cfg.L, k, 0)
    print("[case] fixed hidden states, 32 block steps", flush=True)
    order, toks = [], []
    for t in range(32):
        g = run_step(rd, Ht, mt, tt, k, lo, hi, block)
        assert g["M"] == block - 2 * (t % 16), t
        assert g["n"] == 2
        order += g["sel_idx"].tolist()
        toks += g["sel_tok"].tolist()
    rd.close()
    m = mt.cpu().numpy()
    # exactly the first two blocks are committed, each position once
    assert sorted(order) == list(range(lo, lo + 2 * block))
    assert m[lo:lo + 2 * block].sum() == 0 and m[lo + 2 * block:hi].all() and m[:lo].sum() == 0
    # within each block, the commit order is the first step's ranking (conf
    # descending, position ascending) wherever the oracle separates the rows
    st = oracle.readout_rows(H, W, np.arange(lo, lo + 2 * block))
    pos = np.arange(lo, lo + 2 * block)
    for b in range(2):
        blk = order[b * block:(b + 1) * block]
        assert sorted(blk) == list(range(lo + b * block, lo + (b + 1) * block))
        check_rank_order(np.array(blk), pos, st["logconf"], f"block {b}", gap=GAP)
    # committed tokens are the rows' argmax tokens
    where = {int(p): i for i, p in enumerate(pos)}
    idx = np.array([where[p] for p in order])
    sub = {key: v[idx] for key, v in st.items()}
    check_rows(np.array(toks), sub["conf"], sub["lse"], sub, "fixed hidden tokens")
