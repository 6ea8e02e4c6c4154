"""Masked-token readout of a masked diffusion LLM on MI355X (gfx950).

One step gathers the hidden states of still-masked positions, projects them
through the LM head with a bf16 MFMA GEMM whose epilogue streams the
vocabulary (running max / argmax / sum of exponentials, so no L x V logits
tensor exists), and commits the k best positions by confidence, top-2
margin or negative entropy (top-k, or every position above a threshold).  The work runs
in hand-written HIP kernels behind the C ABI in include/dllm_readout.h;
this package is its thin Python binding.  PyTorch only provides device
memory and streams.
"""
from __future__ import annotations

from ._abi import (  # noqa: F401
    DLLM_BATCH_MAX,
    DLLM_ERR_HIP,
    DLLM_ERR_INVALID_ARG,
    DLLM_ERR_UNSUPPORTED,
    DLLM_ERR_WORKSPACE,
    DLLM_K_MAX_LIMIT,
    DLLM_NOALLOC_SCRATCH_BYTES,
    DLLM_OK,
    DLLM_SCORE_CONF,
    DLLM_SCORE_MARGIN,
    DLLM_SCORE_NEG_ENTROPY,
    EXPORTED,
    LIB_PATH,
    DllmError,
    dllm_ffn_pack_gate_up,
    dllm_ffn_swiglu_chunked,
    dllm_ffn_workspace_bytes,
    dllm_masked_readout_create,
    dllm_masked_readout_destroy,
    dllm_masked_readout_set_gemm_events,
    dllm_masked_readout_set_slices,
    dllm_masked_readout_step,
    dllm_masked_readout_step_batch,
    dllm_masked_readout_step_ex,
    dllm_masked_readout_step_noalloc,
    dllm_masked_readout_workspace_bytes,
    dllm_probe_gemm_mix,
    dllm_probe_source_bytes,
    dllm_probe_wall_clock_khz,
    dllm_policy,
    dllm_seq,
    dllm_status_string,
    load,
    make_policy,
)


_BF16_DTYPES = ("bfloat16", "int16", "uint16")   # bf16 data or its bit pattern
_OUT_INT = ("n_out", "m_out", "sel_idx", "sel_tok", "row_idx", "row_tok")
_OUT_FLOAT = ("sel_conf", "row_conf", "row_lse", "row_margin", "row_entropy")


def _check(t, name: str, dtypes, shape=None, min_numel=None, device=None):
    """Host-side guard before a raw pointer crosses the C ABI: the kernels
    read and write exactly the documented extents, so a wrong dtype, shape,
    stride or device would be an out-of-bounds access on the GPU.  Raw
    integers (device addresses) are passed through unchecked."""
    if isinstance(t, int):
        return
    if str(t.dtype).replace("torch.", "") not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} is not one of {', '.join(dtypes)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name}: {t.numel()} elements, at least {min_numel} needed")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def _check_out(out, n_scalar: int, n_sel: int, n_rows: int, device) -> None:
    for key, v in (out or {}).items():
        if key not in _OUT_INT and key not in _OUT_FLOAT:
            raise KeyError(f"unknown output {key!r}")
        need = n_scalar if key in ("n_out", "m_out") else n_sel if key.startswith("sel_") else n_rows
        _check(v, key, ("int32",) if key in _OUT_INT else ("float32",), min_numel=need, device=device)


class SwiGLUFFN:
    """The sequence-chunked SwiGLU FFN: packed gate/up weights, W_down and
    a torch-allocated [chunk, F] activation workspace.

    ``W_gate``/``W_up`` [F, d] and ``W_down`` [d, F] are bf16 (or int16 bit
    pattern) CUDA tensors; W_down must stay alive as long as this object."""

    def __init__(self, W_gate, W_up, W_down, chunk: int, stream=None):
        import torch
        F, d = W_gate.shape
        dev = W_gate.device
        _check(W_gate, "W_gate", _BF16_DTYPES, shape=(F, d))
        _check(W_up, "W_up", _BF16_DTYPES, shape=(F, d), device=dev)
        _check(W_down, "W_down", _BF16_DTYPES, shape=(d, F), device=dev)
        if not W_gate.is_cuda:
            raise ValueError("W_gate must be a device tensor")
        self.F, self.d, self.chunk = int(F), int(d), int(chunk)
        self.stream = stream if stream is not None else torch.cuda.current_stream(W_gate.device)
        self.W_gu = torch.empty((2 * self.F, self.d), dtype=W_gate.dtype, device=W_gate.device)
        st = dllm_ffn_pack_gate_up(W_gate, W_up, self.F, self.d, self.W_gu, self.stream)
        if st != DLLM_OK:
            raise DllmError(st, "dllm_ffn_pack_gate_up")
        self.W_down = W_down
        nbytes = dllm_ffn_workspace_bytes(self.chunk, self.F)
        if nbytes == 0:
            raise DllmError(DLLM_ERR_INVALID_ARG, "dllm_ffn_workspace_bytes")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=W_gate.device)

    def __call__(self, X, Y=None):
        """Queue Y = FFN(X) (X [L, d]); returns Y (new unless given; may be X)."""
        import torch
        dev = self.W_gu.device
        _check(X, "X", _BF16_DTYPES, shape=(X.shape[0], self.d), device=dev)
        if Y is None:
            Y = torch.empty_like(X)
        _check(Y, "Y", _BF16_DTYPES, shape=tuple(X.shape), device=dev)
        st = dllm_ffn_swiglu_chunked(X, int(X.shape[0]), self.d, self.W_gu, self.W_down, self.F, self.chunk, Y,
                                     self.workspace, int(self.workspace.numel()), self.stream)
        if st != DLLM_OK:
            raise DllmError(st, "dllm_ffn_swiglu_chunked")
        return Y


class MaskedReadout:
    """A handle plus its torch-allocated workspace.

    ``W_lm`` is a [V, d] torch.bfloat16 (or int16 bit-pattern) CUDA tensor
    that must stay alive as long as this object."""

    def __init__(self, W_lm, L_max: int, k_max: int, stream=None):
        import torch
        if W_lm.dim() != 2:
            raise ValueError("W_lm must be [V, d]")
        _check(W_lm, "W_lm", _BF16_DTYPES)
        if not W_lm.is_cuda:
            raise ValueError("W_lm must be a device tensor")
        V, d = W_lm.shape
        self.V, self.d, self.L_max, self.k_max = int(V), int(d), int(L_max), int(k_max)
        nbytes = dllm_masked_readout_workspace_bytes(L_max, d, V, k_max)
        if nbytes == 0:
            raise DllmError(DLLM_ERR_INVALID_ARG, "dllm_masked_readout_workspace_bytes")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=W_lm.device)
        self.W_lm = W_lm
        self.stream = stream if stream is not None else torch.cuda.current_stream(W_lm.device)
        st, h = dllm_masked_readout_create(W_lm, self.V, self.d, L_max, k_max, self.workspace, nbytes,
                                           self.stream)
        if st != DLLM_OK:
            raise DllmError(st, "dllm_masked_readout_create")
        self.handle = h

    def set_slices(self, slices: int) -> None:
        st = dllm_masked_readout_set_slices(self.handle, slices)
        if st != DLLM_OK:
            raise DllmError(st, "dllm_masked_readout_set_slices")

    def outputs(self, ext: bool = False):
        """Freshly allocated output buffers for step(); ``ext`` adds the
        per-row margin and entropy."""
        import torch
        dev = self.W_lm.device
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        K, L = max(self.k_max, 1), self.L_max
        o = dict(n_out=torch.zeros(1, **i32), m_out=torch.zeros(1, **i32),
                 sel_idx=torch.full((K,), -1, **i32), sel_tok=torch.full((K,), -1, **i32),
                 sel_conf=torch.zeros(K, **f32), row_idx=torch.full((L,), -1, **i32),
                 row_tok=torch.full((L,), -1, **i32), row_conf=torch.zeros(L, **f32),
                 row_lse=torch.zeros(L, **f32))
        if ext:
            o["row_margin"] = torch.zeros(L, **f32)
            o["row_entropy"] = torch.zeros(L, **f32)
        return o

    def step(self, hidden, mask, tokens, k: int, win_lo: int = 0, win_hi: int | None = None,
             block: int = 0, out: dict | None = None, score="conf", tau: float | None = None) -> None:
        """Queue one readout step on the handle's stream (asynchronous).

        ``score`` ranks the candidates ("conf", "margin", "neg_entropy");
        ``tau`` None commits the top k, otherwise every candidate whose score
        is >= tau (at least one, at most k)."""
        L = int(hidden.shape[0])
        if win_hi is None:
            win_hi = L
        dev = self.W_lm.device
        _check(hidden, "hidden", _BF16_DTYPES, shape=(L, self.d), device=dev)
        _check(mask, "mask", ("uint8", "bool"), shape=(L,), device=dev)
        _check(tokens, "tokens", ("int32",), shape=(L,), device=dev)
        _check_out(out, 1, int(k), max(int(win_hi) - int(win_lo), 0), dev)
        if score == "conf" and tau is None:
            st = dllm_masked_readout_step(self.handle, hidden, L, mask, tokens, int(k), int(win_lo),
                                          int(win_hi), int(block), out)
        else:
            st = dllm_masked_readout_step_ex(self.handle, hidden, L, mask, tokens, int(k), int(win_lo),
                                             int(win_hi), int(block), make_policy(score, tau), out)
        if st != DLLM_OK:
            raise DllmError(st, "dllm_masked_readout_step")

    def outputs_batch(self, B: int, L: int, ext: bool = False):
        """Freshly allocated per-sequence output buffers for step_batch()."""
        import torch
        dev = self.W_lm.device
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        K = max(self.k_max, 1)
        o = dict(n_out=torch.zeros(B, **i32), m_out=torch.zeros(B, **i32),
                 sel_idx=torch.full((B, K), -1, **i32), sel_tok=torch.full((B, K), -1, **i32),
                 sel_conf=torch.zeros((B, K), **f32), row_idx=torch.full((B, L), -1, **i32),
                 row_tok=torch.full((B, L), -1, **i32), row_conf=torch.zeros((B, L), **f32),
                 row_lse=torch.zeros((B, L), **f32))
        if ext:
            o["row_margin"] = torch.zeros((B, L), **f32)
            o["row_entropy"] = torch.zeros((B, L), **f32)
        return o

    def step_batch(self, hidden, mask, tokens, seqs, block: int = 0, out: dict | None = None, score="conf",
                   tau: float | None = None) -> None:
        """Queue one batched step: ``hidden`` [B, L, d], ``mask``/``tokens``
        [B, L], ``seqs`` B (k, win_lo, win_hi) triples.  Outputs (outputs_batch)
        are per sequence; sel_* have a row stride of max(k_max, 1), which is
        k_max for any handle that can commit."""
        B, L = int(hidden.shape[0]), int(hidden.shape[1])
        if len(seqs) != B:
            raise ValueError("one (k, win_lo, win_hi) per sequence")
        dev = self.W_lm.device
        _check(hidden, "hidden", _BF16_DTYPES, shape=(B, L, self.d), device=dev)
        _check(mask, "mask", ("uint8", "bool"), shape=(B, L), device=dev)
        _check(tokens, "tokens", ("int32",), shape=(B, L), device=dev)
        _check_out(out, B, B * max(self.k_max, 1), B * L, dev)
        pol = None if (score == "conf" and tau is None) else make_policy(score, tau)
        st = dllm_masked_readout_step_batch(self.handle, B, hidden, L, mask, tokens, seqs, int(block), pol, out)
        if st != DLLM_OK:
            raise DllmError(st, "dllm_masked_readout_step_batch")

    def close(self) -> None:
        if getattr(self, "handle", None):
            dllm_masked_readout_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
