"""Seeded synthetic inputs for the masked-token readout.

This module makes the bytes that both the CPU oracle and the HIP library
read: the LM head W_lm, the final hidden states, the mask flags and the
token array of one denoising step.  It holds none of the readout's own
arithmetic (no logits, no softmax, no selection): it draws random numbers,
rounds them to bfloat16 and places the mask.

Workloads follow the masked diffusion LLM setting of the pages:
  * Mosaic (Unlocking Long-Context Inference for Diffusion LLMs via Global
    Memory Planning and Dynamic Peak Taming), Abstract and Fig. 3: logits
    are needed only at masked positions; at 128k context the mask ratio r_m
    decides whether logits or the FFN hold the memory peak.
  * Sparse-dLLM (Accelerating Diffusion LLMs with Dynamic Cache Eviction),
    Experiment / More Results: block-wise decoding with 32-token blocks
    needs logits only for the current block.

  * Serving many requests at once (Accelerating Masked Diffusion Large
    Language Models: A Survey of Efficient Inference Techniques, Main
    Findings: microbatching; throughput-bound serving): a batch of B
    sequences decoded together, sharing the LM head.

Seeding: every tensor comes from
``np.random.Generator(PCG64(SeedSequence([0xD11A, config, stream, step, chunk])))``
with streams 0 = W_lm, 1 = hidden, 2 = mask/tokens, 3 = plant; sequence
b > 0 of a batch appends b to that list (sequence 0 draws exactly the bytes of
an unbatched workload).  Large tensors are drawn in fixed chunks of
``CHUNK`` elements, each with its own seed, so the bytes do not depend on how
many threads draw them.
"""
from __future__ import annotations

import concurrent.futures as _cf
import hashlib
import math
import os
from dataclasses import dataclass, field

import numpy as np

SEED_ROOT = 0xD11A
STREAM_W, STREAM_HIDDEN, STREAM_MASK, STREAM_PLANT = 0, 1, 2, 3
STREAM_FFN_GATE, STREAM_FFN_UP, STREAM_FFN_DOWN = 4, 5, 6
CHUNK = 1 << 22          # elements per independently seeded chunk
W_STD = 0.02             # W_lm ~ N(0, 0.02): 0.02 is the standard deviation
RMS_EPS = 1e-6           # RMS normalisation of the LLaDA-like hidden states


@dataclass(frozen=True)
class Config:
    """One synthetic workload (``id`` only selects its random streams).

    ``mask_kind``: "bernoulli" (each position masked with prob ``mask_ratio``),
    "exact" (exactly round(mask_ratio * L) positions, uniform without
    replacement) or "suffix" (the last ``suffix`` positions masked).
    ``block``: 0 = candidates are all masked rows of the window; >0 = only the
    masked rows of the lowest ``block``-aligned block that still holds one.
    ``plant_frac``: fraction of all L rows that carry a planted dominant token.
    ``batch``: number of sequences decoded together (each of length L).
    """
    id: int
    name: str
    L: int
    d: int
    V: int
    k: int
    steps: int = 1
    mask_kind: str = "exact"
    mask_ratio: float = 0.0
    suffix: int = 0
    block: int = 0
    rms_norm: bool = False
    plant_frac: float = 0.0
    plant_margin: float = 8.0
    batch: int = 1

    @property
    def win(self) -> tuple[int, int]:
        """Window the readout is called on ([lo, hi) positions)."""
        if self.mask_kind == "suffix":
            return (self.L - self.suffix, self.L)
        return (0, self.L)


WORKLOADS: dict[str, Config] = {c.name: c for c in (
    Config(1, "tiny", L=512, d=256, V=4096, k=32,
              mask_kind="bernoulli", mask_ratio=0.5),
    Config(2, "llada_like_semi_ar", L=4096, d=4096, V=126464, k=2, steps=32,
              mask_kind="suffix", suffix=1024, block=32, rms_norm=True),
    Config(3, "dream_like", L=8192, d=3584, V=152064, k=64,
              mask_kind="exact", mask_ratio=0.9),
    Config(4, "long_ctx_low_mask", L=131072, d=4096, V=126464, k=256,
              mask_kind="exact", mask_ratio=0.1),
    Config(5, "long_ctx_high_mask", L=131072, d=4096, V=126464, k=1024,
           mask_kind="exact", mask_ratio=0.9, plant_frac=0.05),
    Config(6, "llada_like_semi_ar_batch16", L=4096, d=4096, V=126464, k=2, steps=32,
           mask_kind="suffix", suffix=1024, block=32, rms_norm=True, batch=16),
)}

MASK_TOKEN_OFFSET = 0   # masked positions hold token id V + this (outside the vocabulary)


def _rng(config_id: int, stream: int, step: int = 0, chunk: int = 0, seq: int = 0) -> np.random.Generator:
    key = [SEED_ROOT, int(config_id), int(stream), int(step), int(chunk)]
    if seq:
        key.append(int(seq))
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (round to nearest, ties to even).

    Returns the bfloat16 bit patterns as uint16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (used to build inputs)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(n_rows: int, n_cols: int, std: float, config_id: int, stream: int,
                 step: int = 0, rms_norm: bool = False, seq: int = 0) -> np.ndarray:
    """[n_rows, n_cols] uint16 bf16 bits of N(0, std) draws, chunk-seeded.

    With ``rms_norm`` each row is scaled by 1/sqrt(mean(row**2) + RMS_EPS) in
    float32 before rounding (chunks then hold whole rows)."""
    out = np.empty((n_rows, n_cols), dtype=np.uint16)
    flat = out.reshape(-1)
    total = n_rows * n_cols
    if rms_norm:
        rows_per_chunk = max(1, CHUNK // n_cols)
        spans = [(c, r0 * n_cols, min(n_rows, r0 + rows_per_chunk) * n_cols)
                 for c, r0 in enumerate(range(0, n_rows, rows_per_chunk))]
    else:
        spans = [(c, a, min(total, a + CHUNK)) for c, a in enumerate(range(0, total, CHUNK))]

    def work(span):
        c, a, b = span
        x = _rng(config_id, stream, step, c, seq).standard_normal(b - a, dtype=np.float32)
        if rms_norm:
            x = x.reshape(-1, n_cols)
            ms = np.mean(x.astype(np.float64) ** 2, axis=1, keepdims=True).astype(np.float32)
            x = (x / np.sqrt(ms + np.float32(RMS_EPS))).reshape(-1)
        elif std != 1.0:
            x *= np.float32(std)
        flat[a:b] = bf16_round(x)

    if len(spans) == 1:
        work(spans[0])
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, spans))
    return out


def random_rows(n_rows: int, n_cols: int, std: float, config_id: int, stream: int) -> np.ndarray:
    """[n_rows, n_cols] bf16 bits of seeded N(0, std) draws (tests that place a
    few rows inside a large, otherwise unread tensor)."""
    return _normal_bf16(n_rows, n_cols, std, config_id, stream)


def w_lm(cfg: Config) -> np.ndarray:
    """LM head W_lm [V, d], bf16 bits, N(0, 0.02)."""
    return _normal_bf16(cfg.V, cfg.d, W_STD, cfg.id, STREAM_W)


def initial_state(cfg: Config, seq: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """(mask u8 [L], tokens i32 [L]) of sequence ``seq`` before the first step.

    Masked positions hold token id V (outside the vocabulary); the others hold
    uniform draws from [0, V)."""
    g = _rng(cfg.id, STREAM_MASK, seq=seq)
    L = cfg.L
    mask = np.zeros(L, dtype=np.uint8)
    if cfg.mask_kind == "bernoulli":
        mask[:] = (g.random(L) < cfg.mask_ratio).astype(np.uint8)
    elif cfg.mask_kind == "exact":
        m = int(round(cfg.mask_ratio * L))
        mask[g.choice(L, size=m, replace=False)] = 1
    elif cfg.mask_kind == "suffix":
        mask[L - cfg.suffix:] = 1
    else:
        raise ValueError(cfg.mask_kind)
    tokens = g.integers(0, cfg.V, size=L, dtype=np.int64).astype(np.int32)
    tokens[mask != 0] = cfg.V + MASK_TOKEN_OFFSET
    return mask, tokens


def _expected_max_std_normal(n: int) -> float:
    """Expected maximum of n iid N(0,1) draws (extreme-value approximation)."""
    a = math.sqrt(2.0 * math.log(n))
    return a - (math.log(math.log(n)) + math.log(4.0 * math.pi)) / (2.0 * a) + 0.5772156649015329 / a


@dataclass
class Plant:
    rows: np.ndarray      # int64 [P] planted positions (ascending)
    tokens: np.ndarray    # int32 [P] planted token per row


def hidden(cfg: Config, W_bits: np.ndarray | None = None, step: int = 0, seq: int = 0
           ) -> tuple[np.ndarray, Plant | None]:
    """Final hidden states [L, d] (bf16 bits) for one step, plus the plant record.

    Planted rows (``plant_frac`` > 0) form the second component of the
    mixture: the N(0,1) row r is moved along w_t / |w_t|^2 so that its logit
    for the planted token t lands ``plant_margin`` above the expected maximum
    of its other V-1 logits, sigma * E[max of V-1 N(0,1)] with
    sigma = |r| * 0.02 (the spread of r . w_v under W_lm's distribution).
    This needs one d-long dot product per planted row, no logits."""
    H = _normal_bf16(cfg.L, cfg.d, 1.0, cfg.id, STREAM_HIDDEN, step, rms_norm=cfg.rms_norm, seq=seq)
    if cfg.plant_frac <= 0.0:
        return H, None
    if W_bits is None:
        raise ValueError("planting needs W_lm")
    g = _rng(cfg.id, STREAM_PLANT, step, seq=seq)
    P = int(round(cfg.plant_frac * cfg.L))
    rows = np.sort(g.choice(cfg.L, size=P, replace=False)).astype(np.int64)
    toks = g.integers(0, cfg.V, size=P, dtype=np.int64).astype(np.int32)
    emax = _expected_max_std_normal(cfg.V - 1)
    for a in range(0, P, 1024):
        rr, tt = rows[a:a + 1024], toks[a:a + 1024]
        r = bf16_to_f32(H[rr]).astype(np.float64)
        w = bf16_to_f32(W_bits[tt]).astype(np.float64)
        wn2 = np.einsum("ij,ij->i", w, w)
        target = cfg.plant_margin + np.linalg.norm(r, axis=1) * W_STD * emax
        beta = target - np.einsum("ij,ij->i", r, w)
        H[rr] = bf16_round((r + (beta / wn2)[:, None] * w).astype(np.float32))
    return H, Plant(rows, toks)


@dataclass
class StepInputs:
    cfg: Config
    W: np.ndarray
    H: np.ndarray
    mask: np.ndarray
    tokens: np.ndarray
    plant: Plant | None = None
    meta: dict = field(default_factory=dict)


def make(cfg_or_name, W_bits: np.ndarray | None = None) -> StepInputs:
    """All inputs of the first step of a workload (a Config or its name)."""
    cfg = WORKLOADS[cfg_or_name] if isinstance(cfg_or_name, str) else cfg_or_name
    W = w_lm(cfg) if W_bits is None else W_bits
    H, plant = hidden(cfg, W, 0)
    mask, tokens = initial_state(cfg)
    return StepInputs(cfg, W, H, mask, tokens, plant)


@dataclass
class BatchInputs:
    cfg: Config
    W: np.ndarray
    H: np.ndarray         # [B, L, d] bf16 bits
    mask: np.ndarray      # [B, L]
    tokens: np.ndarray    # [B, L]


def hidden_batch(cfg: Config, W_bits: np.ndarray | None = None, step: int = 0) -> np.ndarray:
    """[B, L, d] hidden states of every sequence of a batch at one step."""
    return np.stack([hidden(cfg, W_bits, step, seq=b)[0] for b in range(cfg.batch)])


def make_batch(cfg_or_name, W_bits: np.ndarray | None = None) -> BatchInputs:
    """All inputs of the first step of a batched workload."""
    cfg = WORKLOADS[cfg_or_name] if isinstance(cfg_or_name, str) else cfg_or_name
    W = w_lm(cfg) if W_bits is None else W_bits
    states = [initial_state(cfg, b) for b in range(cfg.batch)]
    return BatchInputs(cfg, W, hidden_batch(cfg, W, 0), np.stack([m for m, _ in states]),
                       np.stack([t for _, t in states]))


@dataclass(frozen=True)
class FFNConfig:
    """A SwiGLU FFN over all L positions of one step, run ``chunk`` rows at a
    time (the FFN memory peak at low mask ratio: Mosaic, Abstract and
    Fig. 3).  Weights N(0, 0.02); inputs are RMS-normalised N(0, 1) rows,
    drawn like the LLaDA-like hidden states."""
    id: int
    name: str
    L: int
    d: int
    F: int
    chunk: int
    rms_norm: bool = True


FFN_WORKLOADS: dict[str, FFNConfig] = {c.name: c for c in (
    FFNConfig(7, "ffn_tiny", L=600, d=256, F=384, chunk=256),
    FFNConfig(8, "ffn_long_ctx_low_mask", L=131072, d=4096, F=12288, chunk=8192),
)}


def ffn_weights(cfg: FFNConfig) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(W_gate [F, d], W_up [F, d], W_down [d, F]) bf16 bits, N(0, 0.02)."""
    return (_normal_bf16(cfg.F, cfg.d, W_STD, cfg.id, STREAM_FFN_GATE),
            _normal_bf16(cfg.F, cfg.d, W_STD, cfg.id, STREAM_FFN_UP),
            _normal_bf16(cfg.d, cfg.F, W_STD, cfg.id, STREAM_FFN_DOWN))


def ffn_input(cfg: FFNConfig) -> np.ndarray:
    """FFN input rows X [L, d] (bf16 bits)."""
    return _normal_bf16(cfg.L, cfg.d, 1.0, cfg.id, STREAM_HIDDEN, 0, rms_norm=cfg.rms_norm)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def small_config(base: Config, **kw) -> Config:
    """A config of the same structure with other sizes (tests)."""
    d = dict(base.__dict__)
    d.update(kw)
    return Config(**d)
