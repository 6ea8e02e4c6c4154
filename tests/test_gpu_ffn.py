"""GPU parity of the sequence-chunked SwiGLU FFN against the fp64 oracle.

Tolerance, derived from the arithmetic: the GPU rounds the activation
A = SiLU(x W_gate^T) * (x W_up^T) and the output to bfloat16 (relative error
at most 2^-8 per value) and accumulates in fp32.  With B = sum_f |A_f Wd_jf|
and Q = sum_f (A_f Wd_jf)^2 from the oracle, every output must satisfy
  * |dY| <= 2^-7 (B + |Y|)                 (worst case, twice the rounding bound)
  * |dY| <= 6 2^-8 sqrt(Q) + 2^-7 |Y|      (the activation roundings are
    independent, so their sum is within 6 standard deviations),
the second being tight enough that a dropped or misplaced K chunk fails.
Over all outputs, the rms error relative to the rms output must stay below
RMS_REL = sqrt(2) 2^-8 / sqrt(3) (two independent roundings, each with a
standard deviation of at most 2^-8 / sqrt(3) relative), plus 10%.
Chunking must not change any bit of the result.  Every call goes through
the C ABI (dllm_ffn_pack_gate_up, dllm_ffn_swiglu_chunked)."""
import numpy as np
import pytest

import oracle
import workloads as WL

pytestmark = pytest.mark.gpu

RMS_REL = 1.1 * np.sqrt(2.0) * 2.0 ** -8 / np.sqrt(3.0)    # 3.6e-3


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _bf(rng, shape, std):
    return WL.bf16_round((rng.standard_normal(shape) * std).astype(np.float32))


def _check(Yg_bits, X, Wg, Wu, Wd, rows=None, where=""):
    Xr = X if rows is None else X[rows]
    Y, A, B, Q = oracle.ffn_rows(Xr, Wg, Wu, Wd, want_bound=True)
    Yg = WL.bf16_to_f32(np.asarray(Yg_bits).view(np.uint16)).astype(np.float64)
    if rows is not None:
        Yg = Yg[rows]
    err = np.abs(Yg - Y)
    hard = 2.0 ** -7 * (B + np.abs(Y))
    stat = 6 * 2.0 ** -8 * np.sqrt(Q) + 2.0 ** -7 * np.abs(Y)
    bad = np.argwhere(err > np.minimum(hard, stat))
    assert len(bad) == 0, f"{where}: {len(bad)} outputs off, first {bad[:5].tolist()}: gpu {Yg[tuple(bad[0])]} oracle {Y[tuple(bad[0])]}"
    rel = np.sqrt(np.mean(err ** 2)) / np.sqrt(np.mean(Y ** 2))
    print(f"{where}: rms error / rms output = {rel:.2e}", flush=True)
    return rel


def _run(X, Wg, Wu, Wd, chunk, Y=None):
    import torch
    import masked_token_logits_amd as mtl
    ffn = mtl.SwiGLUFFN(_dev(Wg), _dev(Wu), _dev(Wd), chunk)
    Xt = _dev(X)
    out = ffn(Xt, Xt if Y == "inplace" else None)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16), ffn


def test_pack_gate_up_layout():
    import torch
    import masked_token_logits_amd as mtl
    rng = np.random.default_rng(80)
    F, d = 256, 64
    Wg, Wu = _bf(rng, (F, d), 1.0), _bf(rng, (F, d), 1.0)
    out = torch.empty((2 * F, d), dtype=torch.int16, device="cuda")
    assert mtl.dllm_ffn_pack_gate_up(_dev(Wg), _dev(Wu), F, d, out) == mtl.DLLM_OK
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    want = np.empty_like(got)
    for u in range(2 * F // 64):
        want[64 * u:64 * u + 32] = Wg[32 * u:32 * u + 32]
        want[64 * u + 32:64 * u + 64] = Wu[32 * u:32 * u + 32]
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("L,d,F,chunk", [
    (600, 256, 384, 256),     # the tiny FFN workload: ragged last chunk (88 rows)
    (1, 256, 128, 256),       # one row
    (257, 512, 640, 100),     # chunks not a multiple of the row tile
    (300, 256, 1024, 1000),   # chunk larger than L
    (513, 768, 256, 513),     # partial last row tile, d = 3 output tiles
])
def test_ffn_parity(L, d, F, chunk):
    rng = np.random.default_rng(L + d + F)
    X = WL.bf16_round(rng.standard_normal((L, d)).astype(np.float32))
    Wg, Wu, Wd = _bf(rng, (F, d), 0.05), _bf(rng, (F, d), 0.05), _bf(rng, (d, F), 0.05)
    print(f"[case] ffn L={L} d={d} F={F} chunk={chunk}", flush=True)
    Yg, _ = _run(X, Wg, Wu, Wd, chunk)
    rel = _check(Yg, X, Wg, Wu, Wd, where=f"L={L} d={d} F={F} chunk={chunk}")
    assert rel < RMS_REL


def test_ffn_tiny_workload_and_chunk_invariance():
    cfg = WL.FFN_WORKLOADS["ffn_tiny"]
    Wg, Wu, Wd = WL.ffn_weights(cfg)
    X = WL.ffn_input(cfg)
    ref = None
    for chunk in (cfg.chunk, cfg.L, 1000, 100, 37):
        Yg, _ = _run(X, Wg, Wu, Wd, chunk)
        if ref is None:
            ref = Yg
            _check(Yg, X, Wg, Wu, Wd, where="ffn_tiny")
        else:
            np.testing.assert_array_equal(Yg, ref)      # rows never depend on the chunking
    Yi, _ = _run(X, Wg, Wu, Wd, cfg.chunk, Y="inplace")
    np.testing.assert_array_equal(Yi, ref)


def test_ffn_zero_cases():
    rng = np.random.default_rng(81)
    L, d, F = 300, 256, 384
    X = WL.bf16_round(rng.standard_normal((L, d)).astype(np.float32))
    Wg, Wu, Wd = _bf(rng, (F, d), 0.05), _bf(rng, (F, d), 0.05), _bf(rng, (d, F), 0.05)
    Yg, _ = _run(np.zeros_like(X), Wg, Wu, Wd, 128)
    assert np.all((Yg & 0x7FFF) == 0)                    # +-0 everywhere
    Yg, _ = _run(X, Wg, np.zeros_like(Wu), Wd, 128)
    assert np.all((Yg & 0x7FFF) == 0)


@pytest.mark.slow
def test_ffn_long_context_sampled_rows():
    """The 128k-context LLaDA-like FFN in the benchmark's configuration
    (chunks of 8192 rows); the oracle checks 384 sampled rows and the first
    and last row of every chunk."""
    cfg = WL.FFN_WORKLOADS["ffn_long_ctx_low_mask"]
    print("[case] ffn long context: generating", flush=True)
    Wg, Wu, Wd = WL.ffn_weights(cfg)
    X = WL.ffn_input(cfg)
    Yg, ffn = _run(X, Wg, Wu, Wd, cfg.chunk)
    assert ffn.workspace.numel() == cfg.chunk * cfg.F * 2
    rng = np.random.default_rng(82)
    edges = np.concatenate([np.arange(0, cfg.L, cfg.chunk), np.arange(cfg.chunk - 1, cfg.L, cfg.chunk)])
    rows = np.unique(np.concatenate([rng.choice(cfg.L, 384, replace=False), edges]))
    print(f"[case] ffn long context: oracle on {len(rows)} rows", flush=True)
    rel = _check(Yg, X, Wg, Wu, Wd, rows=rows, where="ffn long context")
    assert rel < RMS_REL
