"""The handle-free step on the library's static device scratch
(dllm_masked_readout_step_noalloc) against the handle step on a caller
workspace: two calls in a row, the second with a smaller input on another
GEMM variant and policy, each compared with the workspace step on the same
inputs (indices, tokens, committed set and state bit for bit; confidence
and log-sum-exp within the relative tolerance of the parity tests)."""
import numpy as np
import pytest

import workloads as WL
from _parity import REL, to_dev

pytestmark = pytest.mark.gpu


def _outputs(L, k, ext):
    import torch
    dev = torch.device("cuda", 0)
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    o = dict(n_out=torch.zeros(1, **i32), m_out=torch.zeros(1, **i32), sel_idx=torch.full((max(k, 1),), -1, **i32),
             sel_tok=torch.full((max(k, 1),), -1, **i32), sel_conf=torch.zeros(max(k, 1), **f32),
             row_idx=torch.full((L,), -1, **i32), row_tok=torch.full((L,), -1, **i32), row_conf=torch.zeros(L, **f32),
             row_lse=torch.zeros(L, **f32))
    if ext:
        o["row_margin"] = torch.zeros(L, **f32)
        o["row_entropy"] = torch.zeros(L, **f32)
    return o


def _host(o, mt, tt):
    import torch
    torch.cuda.synchronize()
    n, M = int(o["n_out"].item()), int(o["m_out"].item())
    r = dict(n=n, M=M, mask=mt.cpu().numpy(), tokens=tt.cpu().numpy())
    for key in ("sel_idx", "sel_tok", "sel_conf"):
        r[key] = o[key][:n].cpu().numpy()
    for key in ("row_idx", "row_tok", "row_conf", "row_lse", "row_margin", "row_entropy"):
        if key in o:
            r[key] = o[key][:M].cpu().numpy()
    return r


def _compare(a, b, where):
    assert a["M"] == b["M"] and a["n"] == b["n"], where
    for key in ("row_idx", "row_tok", "sel_idx", "sel_tok", "mask", "tokens"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=f"{where}: {key}")
    for key in ("row_conf", "row_lse", "sel_conf"):
        x, y = a[key].astype(np.float64), b[key].astype(np.float64)
        assert np.all(np.abs(x - y) <= REL * np.abs(y)), f"{where}: {key}"
    for key in ("row_margin", "row_entropy"):
        if key in b:
            x, y = a[key].astype(np.float64), b[key].astype(np.float64)
            assert np.all(np.abs(x - y) <= REL * (np.abs(y) + 1.0)), f"{where}: {key}"


def _one(inp, k, lo, hi, block, score, tau):
    import torch

    import masked_token_logits_amd as mtl
    cfg = inp.cfg
    ext = score != "conf"
    Wt, Ht, mt, tt = to_dev(inp.W, inp.H, inp.mask, inp.tokens)
    # the workspace step (handle + caller workspace), on its own copies of the state
    rd = mtl.MaskedReadout(Wt, cfg.L, k)
    m1, t1 = mt.clone(), tt.clone()
    o1 = _outputs(cfg.L, k, ext)
    rd.step(Ht, m1, t1, k, lo, hi, block, out=o1, score=score, tau=tau)
    want = _host(o1, m1, t1)
    rd.close()
    # the handle-free step on the static scratch
    o2 = _outputs(cfg.L, k, ext)
    stream = torch.cuda.current_stream()
    pol = mtl.make_policy(score, tau)
    st = mtl.dllm_masked_readout_step_noalloc(Wt, cfg.V, cfg.d, Ht, cfg.L, mt, tt, k, lo, hi, block, pol, o2,
                                              stream)
    assert st == mtl.DLLM_OK, mtl.dllm_status_string(st)
    got = _host(o2, mt, tt)
    return got, want


def test_noalloc_matches_workspace_step_twice():
    # 1: Dream-like step at full size (L = 8192, d = 3584, V = 152064, 7373
    #    candidates, k = 64): compaction, persistent GEMM, merge, radix select
    print("[case] noalloc call 1: dream_like full size, top-k by confidence", flush=True)
    inp = WL.make("dream_like")
    got, want = _one(inp, inp.cfg.k, 0, inp.cfg.L, 0, "conf", None)
    assert want["M"] == 7373 and want["n"] == 64
    _compare(got, want, "dream_like")
    # 2: a smaller input right after: the tiny head, block-mode window (the
    #    few-row GEMM that finds its own rows), margin score with a threshold
    print("[case] noalloc call 2: tiny, block window, margin + threshold", flush=True)
    tiny = WL.make("tiny")
    got, want = _one(tiny, 8, 128, 512, 32, "margin", 0.05)
    assert 0 < want["M"] <= 32
    _compare(got, want, "tiny block")
    # 3: the whole tiny window (persistent GEMM with one row tile), conf
    print("[case] noalloc call 3: tiny, whole window", flush=True)
    got, want = _one(tiny, tiny.cfg.k, 0, tiny.cfg.L, 0, "conf", None)
    assert want["M"] > 32
    _compare(got, want, "tiny whole")
