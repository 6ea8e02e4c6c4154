"""The seeded input generator: determinism, documented counts, bf16 rounding."""
import numpy as np
import pytest
import torch

import workloads as WL


def test_bf16_round_matches_torch_rne():
    """Round-to-nearest-even against torch's float32 -> bfloat16 cast."""
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10,
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -1e-40, 1e-45], np.float32),
        # exact ties: low half 0x8000 with even and odd kept bits
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x3F80C000], np.uint32).view(np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(WL.bf16_round(x), want)


def test_same_seed_same_bytes_and_thread_independence(monkeypatch):
    cfg = WL.small_config(WL.WORKLOADS["dream_like"], L=300, d=64, V=20000, k=8)
    a = WL.w_lm(cfg)
    monkeypatch.setattr(WL, "_threads", lambda: 1)
    b = WL.w_lm(cfg)
    assert WL.sha256(a) == WL.sha256(b)
    h1, _ = WL.hidden(cfg)
    h2, _ = WL.hidden(cfg)
    assert WL.sha256(h1) == WL.sha256(h2)
    other = WL.small_config(cfg, id=4)
    assert WL.sha256(WL.w_lm(other)) != WL.sha256(a)


@pytest.mark.parametrize("name,M", [("dream_like", 7373), ("long_ctx_low_mask", 13107),
                                    ("long_ctx_high_mask", 117965)])
def test_documented_mask_counts(name, M):
    cfg = WL.WORKLOADS[name]
    mask, tokens = WL.initial_state(cfg)
    assert mask.shape == (cfg.L,) and mask.dtype == np.uint8
    assert int(mask.sum()) == M
    assert np.all(tokens[mask != 0] == cfg.V)
    assert np.all((tokens[mask == 0] >= 0) & (tokens[mask == 0] < cfg.V))


def test_tiny_and_semi_ar_masks():
    m1, _ = WL.initial_state(WL.WORKLOADS["tiny"])
    assert 200 < int(m1.sum()) < 312          # Bernoulli(0.5) over 512
    m2, _ = WL.initial_state(WL.WORKLOADS["llada_like_semi_ar"])
    assert m2[:3072].sum() == 0 and m2[3072:].all()
    assert WL.WORKLOADS["llada_like_semi_ar"].win == (3072, 4096)


def test_distributions_and_rms_norm():
    cfg = WL.small_config(WL.WORKLOADS["llada_like_semi_ar"], L=64, d=4096, V=512)
    H, _ = WL.hidden(cfg, step=3)
    h = WL.bf16_to_f32(H).astype(np.float64)
    rms = np.sqrt((h ** 2).mean(axis=1))
    np.testing.assert_allclose(rms, 1.0, atol=5e-3)
    H2, _ = WL.hidden(cfg, step=4)
    assert WL.sha256(H) != WL.sha256(H2)          # re-drawn every step
    W = WL.bf16_to_f32(WL.w_lm(cfg)).astype(np.float64)
    assert abs(W.std() - 0.02) < 2e-4 and abs(W.mean()) < 2e-4


def test_plant_record():
    cfg = WL.small_config(WL.WORKLOADS["long_ctx_high_mask"], L=2000, d=128, V=1000)
    W = WL.w_lm(cfg)
    H, P = WL.hidden(cfg, W)
    assert len(P.rows) == 100 and np.all(np.diff(P.rows) > 0)
    assert np.all((P.tokens >= 0) & (P.tokens < cfg.V))
    H0, _ = WL.hidden(WL.small_config(cfg, plant_frac=0.0))
    changed = np.flatnonzero(np.any(H != H0, axis=1))
    assert set(changed) <= set(P.rows)


def test_batch_sequences_draw_their_own_bytes():
    """Sequence 0 of a batch draws the bytes of the unbatched seeds; the other
    sequences draw different, reproducible bytes."""
    base = WL.WORKLOADS["llada_like_semi_ar_batch16"]
    assert base.batch == 16 and base.win == (3072, 4096)
    cfg = WL.small_config(base, L=64, d=128, V=300, batch=3, suffix=32)
    H0 = WL.hidden(cfg, step=2)[0]
    Hb = WL.hidden_batch(cfg, step=2)
    assert Hb.shape == (3, 64, 128)
    np.testing.assert_array_equal(Hb[0], H0)
    assert WL.sha256(Hb[1]) != WL.sha256(Hb[0]) and WL.sha256(Hb[2]) != WL.sha256(Hb[1])
    np.testing.assert_array_equal(WL.hidden_batch(cfg, step=2), Hb)
    inp = WL.make_batch(cfg)
    assert inp.mask.shape == (3, 64) and np.all(inp.mask[:, 32:] == 1) and np.all(inp.mask[:, :32] == 0)
    assert WL.sha256(inp.tokens[1]) != WL.sha256(inp.tokens[0])


def test_ffn_inputs():
    cfg = WL.FFN_WORKLOADS["ffn_tiny"]
    Wg, Wu, Wd = WL.ffn_weights(cfg)
    assert Wg.shape == Wu.shape == (cfg.F, cfg.d) and Wd.shape == (cfg.d, cfg.F)
    assert len({WL.sha256(Wg), WL.sha256(Wu), WL.sha256(Wd)}) == 3
    X = WL.ffn_input(cfg)
    assert X.shape == (cfg.L, cfg.d)
    rms = np.sqrt((WL.bf16_to_f32(X).astype(np.float64) ** 2).mean(axis=1))
    np.testing.assert_allclose(rms, 1.0, atol=5e-3)
    np.testing.assert_array_equal(WL.ffn_input(cfg), X)
    big = WL.FFN_WORKLOADS["ffn_long_ctx_low_mask"]
    assert (big.L, big.d, big.F) == (131072, 4096, 12288) and big.F % 128 == 0 and big.d % 256 == 0
