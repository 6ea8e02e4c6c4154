"""ctypes binding of libdllm_readout.so (argument marshalling only).

The functions carry the C names and C argument order; device buffers may be
given as torch tensors (their data pointers are passed) or plain integers.
Every step of the readout runs in the library's HIP kernels; there is no
Python or CPU fallback, and loading fails loudly when the library is absent.
"""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdllm_readout.so")

DLLM_OK = 0
DLLM_ERR_INVALID_ARG = 1
DLLM_ERR_UNSUPPORTED = 2
DLLM_ERR_WORKSPACE = 3
DLLM_ERR_HIP = 4
DLLM_K_MAX_LIMIT = 4096
DLLM_BATCH_MAX = 128
DLLM_NOALLOC_SCRATCH_BYTES = 32 << 20

DLLM_SCORE_CONF = 0
DLLM_SCORE_MARGIN = 1
DLLM_SCORE_NEG_ENTROPY = 2
SCORES = {"conf": DLLM_SCORE_CONF, "margin": DLLM_SCORE_MARGIN, "neg_entropy": DLLM_SCORE_NEG_ENTROPY}

EXPORTED = (
    "dllm_masked_readout_workspace_bytes",
    "dllm_masked_readout_create",
    "dllm_masked_readout_step",
    "dllm_masked_readout_step_ex",
    "dllm_masked_readout_step_batch",
    "dllm_masked_readout_destroy",
    "dllm_status_string",
    "dllm_masked_readout_set_slices",
    "dllm_masked_readout_set_gemm_events",
    "dllm_masked_readout_step_noalloc",
    "dllm_ffn_workspace_bytes",
    "dllm_ffn_pack_gate_up",
    "dllm_ffn_swiglu_chunked",
    "dllm_probe_source_bytes",
    "dllm_probe_wall_clock_khz",
    "dllm_probe_gemm_mix",
)


class dllm_step_out(C.Structure):
    _fields_ = [
        ("n_out", C.c_void_p),
        ("m_out", C.c_void_p),
        ("sel_idx", C.c_void_p),
        ("sel_tok", C.c_void_p),
        ("sel_conf", C.c_void_p),
        ("row_idx", C.c_void_p),
        ("row_tok", C.c_void_p),
        ("row_conf", C.c_void_p),
        ("row_lse", C.c_void_p),
        ("row_margin", C.c_void_p),
        ("row_entropy", C.c_void_p),
    ]


class dllm_seq(C.Structure):
    _fields_ = [
        ("k", C.c_int32),
        ("win_lo", C.c_int32),
        ("win_hi", C.c_int32),
    ]


class dllm_policy(C.Structure):
    _fields_ = [
        ("score", C.c_int32),
        ("use_threshold", C.c_int32),
        ("tau", C.c_float),
    ]


_lib = None


def load(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m masked_token_logits_amd.build`")
    # The library must share the process's HIP runtime with PyTorch, which
    # allocates the buffers: with torch loaded first, the dynamic linker
    # resolves the library's libamdhip64 to torch's copy.  Loaded the other
    # way round, the process holds two runtimes and the library's sees no
    # device.
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover - the library still loads (host-only uses)
        pass
    lib = C.CDLL(path)
    lib.dllm_masked_readout_workspace_bytes.restype = C.c_size_t
    lib.dllm_masked_readout_workspace_bytes.argtypes = [C.c_int64, C.c_int64, C.c_int64, C.c_int32]
    lib.dllm_masked_readout_create.restype = C.c_int
    lib.dllm_masked_readout_create.argtypes = [C.POINTER(C.c_void_p), C.c_void_p, C.c_int64, C.c_int64,
                                               C.c_int64, C.c_int32, C.c_void_p, C.c_size_t, C.c_void_p]
    lib.dllm_masked_readout_step.restype = C.c_int
    lib.dllm_masked_readout_step.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p,
                                             C.c_int32, C.c_int64, C.c_int64, C.c_int64,
                                             C.POINTER(dllm_step_out)]
    lib.dllm_masked_readout_step_ex.restype = C.c_int
    lib.dllm_masked_readout_step_ex.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p,
                                                C.c_int32, C.c_int64, C.c_int64, C.c_int64,
                                                C.POINTER(dllm_policy), C.POINTER(dllm_step_out)]
    lib.dllm_masked_readout_step_batch.restype = C.c_int
    lib.dllm_masked_readout_step_batch.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_int64, C.c_void_p,
                                                   C.c_void_p, C.POINTER(dllm_seq), C.c_int64,
                                                   C.POINTER(dllm_policy), C.POINTER(dllm_step_out)]
    lib.dllm_masked_readout_destroy.restype = C.c_int
    lib.dllm_masked_readout_destroy.argtypes = [C.c_void_p]
    lib.dllm_status_string.restype = C.c_char_p
    lib.dllm_status_string.argtypes = [C.c_int]
    lib.dllm_masked_readout_set_slices.restype = C.c_int
    lib.dllm_masked_readout_set_slices.argtypes = [C.c_void_p, C.c_int32]
    lib.dllm_masked_readout_set_gemm_events.restype = C.c_int
    lib.dllm_masked_readout_set_gemm_events.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p]
    lib.dllm_masked_readout_step_noalloc.restype = C.c_int
    lib.dllm_masked_readout_step_noalloc.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_int64,
                                                     C.c_void_p, C.c_void_p, C.c_int32, C.c_int64, C.c_int64,
                                                     C.c_int64, C.POINTER(dllm_policy), C.POINTER(dllm_step_out),
                                                     C.c_void_p]
    lib.dllm_probe_source_bytes.restype = C.c_size_t
    lib.dllm_probe_source_bytes.argtypes = []
    lib.dllm_probe_wall_clock_khz.restype = C.c_int64
    lib.dllm_probe_wall_clock_khz.argtypes = []
    lib.dllm_probe_gemm_mix.restype = C.c_int
    lib.dllm_probe_gemm_mix.argtypes = [C.c_int32, C.c_void_p, C.c_int32, C.c_void_p, C.c_int32, C.c_void_p,
                                        C.c_void_p]
    lib.dllm_ffn_workspace_bytes.restype = C.c_size_t
    lib.dllm_ffn_workspace_bytes.argtypes = [C.c_int64, C.c_int64]
    lib.dllm_ffn_pack_gate_up.restype = C.c_int
    lib.dllm_ffn_pack_gate_up.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p]
    lib.dllm_ffn_swiglu_chunked.restype = C.c_int
    lib.dllm_ffn_swiglu_chunked.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p, C.c_int64,
                                            C.c_int64, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    _lib = lib
    return lib


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class DllmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {dllm_status_string(status)} (status {status})")


def dllm_status_string(status: int) -> str:
    return load().dllm_status_string(int(status)).decode()


def dllm_masked_readout_workspace_bytes(L_max: int, d: int, V: int, k_max: int) -> int:
    return int(load().dllm_masked_readout_workspace_bytes(L_max, d, V, k_max))


def dllm_masked_readout_create(W_lm, V: int, d: int, L_max: int, k_max: int, workspace,
                               workspace_bytes: int, stream=None) -> tuple[int, int | None]:
    """Returns (status, handle)."""
    h = C.c_void_p()
    st = load().dllm_masked_readout_create(C.byref(h), _ptr(W_lm), V, d, L_max, k_max, _ptr(workspace),
                                           workspace_bytes, _stream(stream))
    return st, h.value


def dllm_masked_readout_step(handle, hidden, L: int, mask, tokens, k: int, win_lo: int, win_hi: int,
                             block: int = 0, out: dict | None = None) -> int:
    """``out`` maps dllm_step_out field names to device buffers (optional)."""
    so = None
    if out:
        so = dllm_step_out(**{key: _ptr(v) for key, v in out.items()})
    return load().dllm_masked_readout_step(handle, _ptr(hidden), L, _ptr(mask), _ptr(tokens), k, win_lo, win_hi,
                                           block, C.byref(so) if so is not None else None)


def make_policy(score="conf", tau: float | None = None) -> dllm_policy:
    """dllm_policy for a score name ("conf", "margin", "neg_entropy") or
    dllm_score value; ``tau`` None = top-k, otherwise the threshold rule."""
    sc = SCORES[score] if isinstance(score, str) else int(score)
    if tau is None:
        return dllm_policy(sc, 0, 0.0)
    return dllm_policy(sc, 1, float(tau))


def dllm_masked_readout_step_ex(handle, hidden, L: int, mask, tokens, k: int, win_lo: int, win_hi: int,
                                block: int = 0, policy: dllm_policy | None = None,
                                out: dict | None = None) -> int:
    so = None
    if out:
        so = dllm_step_out(**{key: _ptr(v) for key, v in out.items()})
    return load().dllm_masked_readout_step_ex(handle, _ptr(hidden), L, _ptr(mask), _ptr(tokens), k, win_lo,
                                              win_hi, block, C.byref(policy) if policy is not None else None,
                                              C.byref(so) if so is not None else None)


def dllm_masked_readout_step_noalloc(W_lm, V: int, d: int, hidden, L: int, mask, tokens, k: int, win_lo: int,
                                     win_hi: int, block: int = 0, policy: dllm_policy | None = None,
                                     out: dict | None = None, stream=None) -> int:
    """The handle-free step on the library's static device scratch."""
    so = None
    if out:
        so = dllm_step_out(**{key: _ptr(v) for key, v in out.items()})
    return load().dllm_masked_readout_step_noalloc(_ptr(W_lm), V, d, _ptr(hidden), L, _ptr(mask), _ptr(tokens), k,
                                                   win_lo, win_hi, block,
                                                   C.byref(policy) if policy is not None else None,
                                                   C.byref(so) if so is not None else None, _stream(stream))


def dllm_probe_source_bytes() -> int:
    return int(load().dllm_probe_source_bytes())


def dllm_probe_wall_clock_khz() -> int:
    return int(load().dllm_probe_wall_clock_khz())


def dllm_probe_gemm_mix(mode: int, src, stages: int, sink, grid: int, clocks=None, stream=None) -> int:
    return load().dllm_probe_gemm_mix(int(mode), _ptr(src), int(stages), _ptr(sink), int(grid), _ptr(clocks),
                                      _stream(stream))


def dllm_masked_readout_step_batch(handle, B: int, hidden, L: int, mask, tokens, seqs, block: int = 0,
                                   policy: dllm_policy | None = None, out: dict | None = None) -> int:
    """``seqs``: B (k, win_lo, win_hi) triples (or a dllm_seq array)."""
    if not isinstance(seqs, C.Array):
        arr = (dllm_seq * max(len(seqs), 1))()
        for i, (k, lo, hi) in enumerate(seqs):
            arr[i] = dllm_seq(int(k), int(lo), int(hi))
        seqs = arr
    so = None
    if out:
        so = dllm_step_out(**{key: _ptr(v) for key, v in out.items()})
    return load().dllm_masked_readout_step_batch(handle, int(B), _ptr(hidden), int(L), _ptr(mask), _ptr(tokens),
                                                 seqs, int(block),
                                                 C.byref(policy) if policy is not None else None,
                                                 C.byref(so) if so is not None else None)


def dllm_ffn_workspace_bytes(chunk: int, F: int) -> int:
    return int(load().dllm_ffn_workspace_bytes(chunk, F))


def dllm_ffn_pack_gate_up(W_gate, W_up, F: int, d: int, W_gu, stream=None) -> int:
    return load().dllm_ffn_pack_gate_up(_ptr(W_gate), _ptr(W_up), F, d, _ptr(W_gu), _stream(stream))


def dllm_ffn_swiglu_chunked(X, L: int, d: int, W_gu, W_down, F: int, chunk: int, Y, workspace,
                            workspace_bytes: int, stream=None) -> int:
    return load().dllm_ffn_swiglu_chunked(_ptr(X), L, d, _ptr(W_gu), _ptr(W_down), F, chunk, _ptr(Y),
                                          _ptr(workspace), workspace_bytes, _stream(stream))


def dllm_masked_readout_destroy(handle) -> int:
    return load().dllm_masked_readout_destroy(handle)


def dllm_masked_readout_set_slices(handle, slices: int) -> int:
    return load().dllm_masked_readout_set_slices(handle, slices)


def dllm_masked_readout_set_gemm_events(handle, ev_before, ev_after) -> int:
    return load().dllm_masked_readout_set_gemm_events(handle, ev_before, ev_after)
