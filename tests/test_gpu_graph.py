"""A readout step captured in a HIP graph (torch.cuda.CUDAGraph) and replayed:
a step queues kernels and nothing else (no memset, copy, allocation or
synchronisation), so replaying it must reproduce eager steps exactly.
Every replay is checked bit for bit against the same step run eagerly from
the same state, with unrelated eager work and synchronisations between the
replays.  The oracle parity of these steps is covered elsewhere; this file
checks that capture changes nothing."""
import numpy as np
import pytest

import workloads as WL
from _parity import to_dev

pytestmark = pytest.mark.gpu


def _rand_bf16(rng, shape, std=1.0):
    return WL.bf16_round((rng.standard_normal(shape) * std).astype(np.float32))


def _snapshot(out, mt, tt):
    return {k: v.cpu().numpy().copy() for k, v in list(out.items()) + [("mask", mt), ("tokens", tt)]}


@pytest.mark.parametrize("case", ["few_rows_block", "persistent_window", "margin_threshold"])
def test_graph_replay_matches_eager(case):
    import torch

    import masked_token_logits_amd as mtl
    rng = np.random.default_rng({"few_rows_block": 31, "persistent_window": 32, "margin_threshold": 33}[case])
    L, d, V = 2048, 256, 3000
    H = _rand_bf16(rng, (L, d))
    W = _rand_bf16(rng, (V, d), 0.05)
    tokens = np.full(L, V, np.int32)
    mask = np.zeros(L, np.uint8)
    mask[1024:] = 1
    if case == "few_rows_block":
        k, lo, hi, block, score, tau = 2, 1024, L, 32, "conf", None    # <= 32 rows: the few-row GEMM
    elif case == "persistent_window":
        k, lo, hi, block, score, tau = 24, 1024, 1536, 0, "conf", None  # up to 512 rows: persistent GEMM
    else:
        k, lo, hi, block, score, tau = 3, 1024, L, 32, "margin", 1e-4
    Wt, Ht, mt0, tt0 = to_dev(W, H, mask, tokens)
    steps = 5
    print(f"[case] graph {case} k={k} win=({lo},{hi}) block={block} score={score} tau={tau}", flush=True)

    # eager reference: `steps` consecutive steps from the initial state
    s = torch.cuda.Stream()
    ref = []
    with torch.cuda.stream(s):
        rd = mtl.MaskedReadout(Wt, L, k, stream=s)
        out = rd.outputs()
        init = {key: v.clone() for key, v in out.items()}
        mt, tt = mt0.clone(), tt0.clone()
        for _ in range(steps):
            rd.step(Ht, mt, tt, k, lo, hi, block, out=out, score=score, tau=tau)
            s.synchronize()
            ref.append(_snapshot(out, mt, tt))

        # the same handle, buffers reset, one step captured
        mt.copy_(mt0)
        tt.copy_(tt0)
        for key, v in out.items():
            v.copy_(init[key])
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            rd.step(Ht, mt, tt, k, lo, hi, block, out=out, score=score, tau=tau)
        # capture queued nothing: the state is still the initial one
        s.synchronize()
        assert torch.equal(mt, mt0) and torch.equal(tt, tt0)
        junk = torch.randn(1 << 20, device=mt.device)
        for i in range(steps):
            g.replay()
            s.synchronize()
            got = _snapshot(out, mt, tt)
            for key, want in ref[i].items():
                np.testing.assert_array_equal(got[key], want, err_msg=f"{case} replay {i} {key}")
            junk = torch.tanh(junk * 1.0001)  # unrelated eager work between replays
            torch.cuda.synchronize()
    assert int(ref[-1]["m_out"][0]) >= 0
    print(f"graph {case}: {steps} replays identical to eager steps", flush=True)


@pytest.mark.parametrize("case", ["batch_persistent", "batch_few_rows"])
def test_graph_replay_batched_matches_eager(case):
    """The batched step under capture: B sequences, per-sequence windows and
    k, in block mode (persistent GEMM for up to 128 rows; the few-row GEMM
    when at most 32 rows can come out)."""
    import torch

    import masked_token_logits_amd as mtl
    rng = np.random.default_rng({"batch_persistent": 34, "batch_few_rows": 35}[case])
    if case == "batch_persistent":
        B, L, block = 4, 1024, 32
        seqs = [(2, 512, 1024), (3, 600, 1024), (1, 512, 900), (2, 0, 1024)]
    else:
        B, L, block = 2, 1024, 16
        seqs = [(2, 512, 1024), (1, 700, 1024)]
    d, V = 256, 3000
    H = _rand_bf16(rng, (B, L, d))
    W = _rand_bf16(rng, (V, d), 0.05)
    tokens = np.full((B, L), V, np.int32)
    mask = np.zeros((B, L), np.uint8)
    mask[:, 512:] = 1
    dev = torch.device("cuda", 0)
    Wt = torch.from_numpy(W.view(np.int16)).to(dev)
    Ht = torch.from_numpy(H.view(np.int16)).to(dev)
    mt0 = torch.from_numpy(mask).to(dev)
    tt0 = torch.from_numpy(tokens).to(dev)
    k_max = max(k for k, _, _ in seqs)
    steps = 5
    print(f"[case] graph {case} B={B} L={L} block={block}", flush=True)

    s = torch.cuda.Stream()
    ref = []
    with torch.cuda.stream(s):
        rd = mtl.MaskedReadout(Wt, B * L, k_max, stream=s)
        out = rd.outputs_batch(B, L)
        init = {key: v.clone() for key, v in out.items()}
        mt, tt = mt0.clone(), tt0.clone()
        for _ in range(steps):
            rd.step_batch(Ht, mt, tt, seqs, block, out=out)
            s.synchronize()
            ref.append(_snapshot(out, mt, tt))

        mt.copy_(mt0)
        tt.copy_(tt0)
        for key, v in out.items():
            v.copy_(init[key])
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            rd.step_batch(Ht, mt, tt, seqs, block, out=out)
        s.synchronize()
        assert torch.equal(mt, mt0) and torch.equal(tt, tt0)
        junk = torch.randn(1 << 20, device=mt.device)
        for i in range(steps):
            g.replay()
            s.synchronize()
            got = _snapshot(out, mt, tt)
            for key, want in ref[i].items():
                np.testing.assert_array_equal(got[key], want, err_msg=f"{case} replay {i} {key}")
            junk = torch.tanh(junk * 1.0001)
            torch.cuda.synchronize()
    assert int(ref[-1]["m_out"].sum()) > 0
    print(f"graph {case}: {steps} replays identical to eager steps", flush=True)
