"""fp64 CPU oracle of the sequence-chunked SwiGLU FFN (test infrastructure only).

Mosaic (Unlocking Long-Context Inference for Diffusion LLMs via Global Memory
Planning and Dynamic Peak Taming), Abstract and Fig. 3: a dLLM recomputes
its transient activations at every step, and at low mask ratio the memory
peak is the FFN's rather than the logits'; lazy chunking tames such peaks.
The pages give no FFN formula; this oracle reads it as the SwiGLU MLP of
LLaMA-family models (LLaDA is one):

    FFN(x) = W_down (SiLU(W_gate x) * (W_up x)),   SiLU(g) = g / (1 + e^-g),

applied to every position, and chunking as running it on consecutive
blocks of rows: a row's output depends on that row only, so the chunk size
changes the memory peak and never the result.  Everything is plain fp64
NumPy on the exact bf16 inputs; no intermediate is rounded.
"""
from __future__ import annotations

import numpy as np

from .readout import widen_bf16


def silu(g: np.ndarray) -> np.ndarray:
    """SiLU(g) = g * sigmoid(g) = g / (1 + exp(-g)), fp64."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def ffn_rows(X_bits: np.ndarray, Wg_bits: np.ndarray, Wu_bits: np.ndarray, Wd_bits: np.ndarray,
             want_bound: bool = False):
    """SwiGLU FFN of the given rows in fp64.

    X [n, d], W_gate / W_up [F, d], W_down [d, F] (bf16 bits).  Returns
    (Y [n, d], A [n, F]) and, with ``want_bound``, also the sums over f of
    |A_f W_down[j, f]| and of (A_f W_down[j, f])^2 for every output (the
    scales of rounding errors in its terms)."""
    X = widen_bf16(X_bits)
    Wg, Wu, Wd = widen_bf16(Wg_bits), widen_bf16(Wu_bits), widen_bf16(Wd_bits)
    A = silu(X @ Wg.T) * (X @ Wu.T)
    Y = A @ Wd.T
    if want_bound:
        return Y, A, np.abs(A) @ np.abs(Wd).T, (A * A) @ (Wd * Wd).T
    return Y, A


def ffn_chunked(X_bits, Wg_bits, Wu_bits, Wd_bits, chunk: int) -> np.ndarray:
    """The FFN over all L rows, ``chunk`` rows at a time (Y [L, d], fp64)."""
    L = X_bits.shape[0]
    out = np.empty((L, Wd_bits.shape[0]), dtype=np.float64)
    for a in range(0, L, max(1, int(chunk))):
        out[a:a + chunk] = ffn_rows(X_bits[a:a + chunk], Wg_bits, Wu_bits, Wd_bits)[0]
    return out
