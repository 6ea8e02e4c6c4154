"""fp64 CPU oracle of one denoising readout step (test infrastructure only).

What it computes, in the pages' terms:

* Mosaic (Unlocking Long-Context Inference for Diffusion LLMs via Global
  Memory Planning and Dynamic Peak Taming), TL;DR and Abstract: the LM-head
  logits are computed only for positions that still hold the mask token
  ("mask-only logits"), and the full L x V logits tensor is the memory peak
  at high mask ratio (Fig. 3).
* Sparse-dLLM (Accelerating Diffusion LLMs with Dynamic Cache Eviction),
  Method "Inference background": the sequence goes from fully masked to
  unmasked over T steps, so each step commits some masked positions;
  Experiment "Memory" and More Results: block-wise decoding with 32-token
  blocks needs logits only for the current block.
* Accelerating Masked Diffusion Large Language Models: A Survey of Efficient
  Inference Techniques, Main Findings: confidence-driven unmasking picks the
  positions to commit; the update set Delta_t is the set of positions whose
  token changes in a step; notation M_t (masked set) and U_t (unmasked set).
* Dynamic-dLLM (fourth abstract on the last page): adaptive parallel decoding
  commits every position whose confidence clears a calibrated threshold.

The pages print no formula for the confidence or the selection.  This
oracle reads them as: confidence = the largest softmax probability of the
row at temperature 1 (greedy argmax token), the k most confident masked rows
are committed, argmax ties go to the lowest vocabulary index and selection
ties to the lowest position.

Everything here is plain fp64 NumPy: a full logits matrix per chunk of
masked rows (BLAS dgemm), a materialised naive softmax and a stable sort.
Rows are processed in chunks of at most ``row_chunk`` rows only so that
long-context inputs fit in host memory; every row still sees all V logits.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64, exactly (a bf16 value is the top 16
    bits of a float32, and every float32 is a float64)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def candidate_positions(mask: np.ndarray, win_lo: int, win_hi: int, block: int = 0) -> np.ndarray:
    """Positions whose logits are needed this step, ascending.

    Mask-only logits (Mosaic, Abstract): only positions still masked are
    candidates.  The window [win_lo, win_hi) restricts them to a part of the
    sequence.  With ``block`` > 0 (block-wise / semi-autoregressive decoding,
    Sparse-dLLM Experiment "Memory": logits only for the current block), the
    window is cut into consecutive blocks of ``block`` positions starting at
    win_lo, and only the first block that still holds a masked position
    contributes."""
    mask = np.asarray(mask)
    lo, hi = int(win_lo), int(win_hi)
    masked = [i for i in range(lo, hi) if mask[i] != 0]
    if block <= 0 or not masked:
        return np.asarray(masked, dtype=np.int64)
    first = masked[0]
    b_lo = lo + ((first - lo) // block) * block
    b_hi = min(b_lo + block, hi)
    return np.asarray([i for i in masked if b_lo <= i < b_hi], dtype=np.int64)


def logits(H_rows: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Z = H_rows . W^T in fp64: one row per candidate position, one column per
    vocabulary entry (the LM-head projection, Mosaic Abstract)."""
    return np.asarray(H_rows, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def row_stats(Z: np.ndarray) -> dict:
    """Per-row readout of a full logits matrix Z [M, V] (fp64).

    tok      argmax over the vocabulary, lowest index on ties
    mx       the largest logit
    gap2     mx minus the largest logit at any other index (0 on a tie)
    conf     softmax probability of tok (the row's confidence)
    lse      log-sum-exp of the row (natural log)
    logconf  log(conf) = mx - lse
    margin   conf minus the second-largest softmax probability
    entropy  -sum_v p_v log p_v of the softmax
    The softmax is materialised: P = exp(Z - mx) / sum(exp(Z - mx))."""
    Z = np.asarray(Z, dtype=np.float64)
    M, V = Z.shape
    if M == 0:
        e = np.zeros(0)
        return dict(tok=np.zeros(0, np.int64), mx=e, gap2=e, conf=e, lse=e,
                    logconf=e, margin=e, entropy=e)
    tok = np.argmax(Z, axis=1)
    r = np.arange(M)
    mx = Z[r, tok]
    Zo = Z.copy()
    Zo[r, tok] = -np.inf
    second = Zo.max(axis=1) if V > 1 else np.full(M, -np.inf)
    gap2 = mx - second
    E = np.exp(Z - mx[:, None])
    S = E.sum(axis=1)
    P = E / S[:, None]
    conf = P[r, tok]
    lse = mx + np.log(S)
    Po = P.copy()
    Po[r, tok] = -np.inf
    p2 = Po.max(axis=1) if V > 1 else np.zeros(M)
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(P > 0.0, P * np.log(P), 0.0)
    entropy = -plogp.sum(axis=1)
    return dict(tok=tok.astype(np.int64), mx=mx, gap2=gap2, conf=conf, lse=lse,
                logconf=mx - lse, margin=conf - p2, entropy=entropy)


def select_topk(score: np.ndarray, positions: np.ndarray, k: int) -> np.ndarray:
    """The n = min(k, M) candidates with the largest score, in rank order
    (score descending, position ascending on ties).

    Confidence-driven unmasking (survey, Main Findings).  ``positions`` is
    ascending, so a stable sort of -score keeps equal scores in position
    order."""
    n = min(max(int(k), 0), len(positions))
    order = np.argsort(-np.asarray(score, dtype=np.float64), kind="stable")
    return np.asarray(positions, dtype=np.int64)[order[:n]]


def select_threshold(score: np.ndarray, positions: np.ndarray, tau: float, k_cap: int) -> np.ndarray:
    """Threshold unmasking (Dynamic-dLLM, adaptive parallel decoding): every
    candidate with score >= tau, at least one (the best) when any candidate
    exists, at most k_cap; rank order as in select_topk."""
    score = np.asarray(score, dtype=np.float64)
    M = len(positions)
    if M == 0 or k_cap <= 0:
        return np.zeros(0, dtype=np.int64)
    n = int(np.count_nonzero(score >= tau))
    n = min(max(n, 1), int(k_cap), M)
    order = np.argsort(-score, kind="stable")
    return np.asarray(positions, dtype=np.int64)[order[:n]]


def apply_updates(tokens: np.ndarray, mask: np.ndarray, sel: np.ndarray, sel_tok: np.ndarray):
    """Commit the selected positions (Sparse-dLLM, Method: masked positions
    become tokens step by step; survey: Delta_t = the positions that change).
    Returns new (tokens, mask); nothing else changes."""
    t = np.array(tokens, dtype=np.int32, copy=True)
    m = np.array(mask, dtype=np.uint8, copy=True)
    sel = np.asarray(sel, dtype=np.int64)
    t[sel] = np.asarray(sel_tok, dtype=np.int32)
    m[sel] = 0
    return t, m


@dataclass
class StepResult:
    positions: np.ndarray   # candidate positions C (ascending)
    stats: dict             # row_stats over C
    sel: np.ndarray         # committed positions, rank order
    sel_tok: np.ndarray     # their tokens
    tokens: np.ndarray      # tokens after the step
    mask: np.ndarray        # mask after the step

    @property
    def M(self) -> int:
        return len(self.positions)


def _score(stats: dict, kind: str) -> np.ndarray:
    if kind == "conf":
        return stats["conf"]
    if kind == "margin":
        return stats["margin"]
    if kind == "neg_entropy":
        return -stats["entropy"]
    raise ValueError(kind)


def readout_rows(H_bits: np.ndarray, W_bits: np.ndarray, positions, row_chunk: int = 2048,
                 W64: np.ndarray | None = None) -> dict:
    """row_stats for the given positions of the hidden states, full vocabulary
    per row, computed ``row_chunk`` rows at a time."""
    positions = np.asarray(positions, dtype=np.int64)
    if W64 is None:
        W64 = widen_bf16(W_bits)
    parts = []
    for a in range(0, len(positions), row_chunk):
        Hc = widen_bf16(H_bits[positions[a:a + row_chunk]])
        parts.append(row_stats(logits(Hc, W64)))
    if not parts:
        return row_stats(np.zeros((0, W64.shape[0])))
    return {key: np.concatenate([p[key] for p in parts]) for key in parts[0]}


def readout_step(H_bits: np.ndarray, W_bits: np.ndarray, mask: np.ndarray, tokens: np.ndarray,
                 k: int, win_lo: int = 0, win_hi: int | None = None, block: int = 0,
                 score: str = "conf", tau: float | None = None, row_chunk: int = 2048,
                 W64: np.ndarray | None = None) -> StepResult:
    """One readout step: candidates -> full fp64 logits -> softmax statistics
    -> select -> commit.  ``tau`` None selects the top k; otherwise the
    threshold rule with cap k."""
    if win_hi is None:
        win_hi = len(mask)
    C = candidate_positions(mask, win_lo, win_hi, block)
    st = readout_rows(H_bits, W_bits, C, row_chunk=row_chunk, W64=W64)
    sc = _score(st, score)
    if tau is None:
        sel = select_topk(sc, C, k)
    else:
        sel = select_threshold(sc, C, tau, k)
    where = {int(p): i for i, p in enumerate(C)}
    sel_tok = np.asarray([st["tok"][where[int(p)]] for p in sel], dtype=np.int32)
    t2, m2 = apply_updates(tokens, mask, sel, sel_tok)
    return StepResult(C, st, sel, sel_tok, t2, m2)


def readout_step_batch(H_bits: np.ndarray, W_bits: np.ndarray, mask: np.ndarray, tokens: np.ndarray,
                       seqs, block: int = 0, score: str = "conf", tau: float | None = None,
                       row_chunk: int = 2048, W64: np.ndarray | None = None) -> list:
    """B independent readout steps that share one LM head: sequence b has
    hidden states H_bits[b] [L, d], mask[b], tokens[b] and its own
    (k, win_lo, win_hi) = seqs[b]; ``block``, ``score`` and ``tau`` are common.

    Serving many requests at once (Survey, Main Findings: microbatching;
    "Real-world applications": high-throughput serving of concurrent
    requests) changes how the work is scheduled, not what a step computes,
    so each sequence's result is exactly readout_step on that sequence
    alone.  Returns one StepResult per sequence."""
    H_bits = np.asarray(H_bits)
    if W64 is None:
        W64 = widen_bf16(W_bits)
    out = []
    for b, (k, lo, hi) in enumerate(seqs):
        out.append(readout_step(H_bits[b], W_bits, mask[b], tokens[b], int(k), int(lo), int(hi), block,
                                score=score, tau=tau, row_chunk=row_chunk, W64=W64))
    return out
