"""A hidden tensor larger than 4 GiB on the persistent GEMM (its whole-line
main loop addresses gathered hidden rows with 64-bit offsets): L = 540000
positions of d = 4096 (4.4 GB), 600 candidates, half of them beyond byte
offset 2^32 of the tensor, checked row by row against the oracle.  The rows
that are not candidates are never read, so they stay zero; the candidate
rows, W_lm (V = 700, a ragged vocabulary tile) and the mask come from the
seeded generators."""
import numpy as np
import pytest

import oracle
import workloads as WL
from _parity import check_rank_order, check_rows, check_selection

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def test_hidden_over_4gib():
    import torch

    import masked_token_logits_amd as mtl
    L, d, V, k, M = 540000, 4096, 700, 20, 600
    assert L * d * 2 > (1 << 32)
    rng = np.random.default_rng(4242)
    edge = (1 << 32) // (d * 2)                          # first row at or past byte offset 2^32
    pos = np.sort(np.concatenate([rng.choice(edge, M // 2, replace=False),
                                  edge + rng.choice(L - edge, M // 2, replace=False)])).astype(np.int64)
    rows = WL.random_rows(M, d, 1.0, 90, 1)
    W = WL.random_rows(V, d, WL.W_STD, 90, 0)
    mask = np.zeros(L, np.uint8)
    mask[pos] = 1
    tokens = np.full(L, V, np.int32)
    print(f"[case] hidden {L} x {d} ({L * d * 2 / 2**30:.2f} GiB), {M} candidates, {int((pos >= edge).sum())} "
          f"past 4 GiB", flush=True)
    dev = torch.device("cuda", 0)
    Ht = torch.zeros((L, d), dtype=torch.int16, device=dev)
    Ht[torch.from_numpy(pos).to(dev)] = torch.from_numpy(rows.view(np.int16)).to(dev)
    Wt = torch.from_numpy(W.view(np.int16)).to(dev)
    mt = torch.from_numpy(mask).to(dev)
    tt = torch.from_numpy(tokens).to(dev)
    rd = mtl.MaskedReadout(Wt, L, k)
    out = rd.outputs()
    rd.step(Ht, mt, tt, k, 0, L, 0, out=out)
    torch.cuda.synchronize()
    n, Mg = int(out["n_out"].item()), int(out["m_out"].item())
    assert Mg == M and n == k
    np.testing.assert_array_equal(out["row_idx"][:M].cpu().numpy(), pos)
    st = oracle.readout_rows(rows, W, np.arange(M))
    check_rows(out["row_tok"][:M].cpu().numpy(), out["row_conf"][:M].cpu().numpy(),
               out["row_lse"][:M].cpu().numpy(), st, "hidden > 4 GiB")
    sel = out["sel_idx"][:n].cpu().numpy()
    check_selection(sel, pos, st["logconf"], n, "hidden > 4 GiB")
    check_rank_order(sel, pos, st["logconf"], "hidden > 4 GiB")
    m2, t2 = mt.cpu().numpy(), tt.cpu().numpy()
    assert m2[sel].sum() == 0 and int(m2.sum()) == M - n
    np.testing.assert_array_equal(t2[sel], out["sel_tok"][:n].cpu().numpy())
    rd.close()
