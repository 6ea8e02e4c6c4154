"""The Python binding's host-side guards: a tensor whose dtype, shape,
stride or size does not match what the kernels will read or write is
rejected before its pointer reaches the C ABI.  CPU tensors only: the
checks run before any device work, and a valid call goes on to the library,
which returns an error without a GPU."""
import pytest
import torch

import masked_token_logits_amd as mtl
from masked_token_logits_amd import MaskedReadout, SwiGLUFFN, _check, _check_out


def _readout(V=64, d=16, L_max=32, k_max=4):
    """A MaskedReadout whose checks can run on the CPU (no device handle)."""
    rd = object.__new__(MaskedReadout)
    rd.V, rd.d, rd.L_max, rd.k_max = V, d, L_max, k_max
    rd.W_lm = torch.zeros((V, d), dtype=torch.bfloat16)
    rd.handle = None
    return rd


def _inputs(L=32, d=16, B=None):
    lead = (L,) if B is None else (B, L)
    return (torch.zeros(lead + (d,), dtype=torch.bfloat16), torch.zeros(lead, dtype=torch.uint8),
            torch.zeros(lead, dtype=torch.int32))


def test_check_accepts_bf16_bit_patterns_and_raw_addresses():
    _check(torch.zeros(4, dtype=torch.int16), "x", ("bfloat16", "int16"))
    _check(torch.zeros(4, dtype=torch.bfloat16), "x", ("bfloat16", "int16"))
    _check(12345678, "x", ("int32",), shape=(3,))  # a device address: not checkable, passed through


def test_check_rejects_dtype_shape_size_and_strides():
    with pytest.raises(TypeError):
        _check(torch.zeros(4, dtype=torch.float32), "x", ("bfloat16",))
    with pytest.raises(ValueError):
        _check(torch.zeros(4, dtype=torch.int32), "x", ("int32",), shape=(5,))
    with pytest.raises(ValueError):
        _check(torch.zeros(4, dtype=torch.int32), "x", ("int32",), min_numel=5)
    with pytest.raises(ValueError):
        _check(torch.zeros((4, 4), dtype=torch.int32).t(), "x", ("int32",))


def test_step_validates_every_tensor_before_the_library():
    rd = _readout()
    H, m, t = _inputs()
    bad = [
        (H.float(), m, t),                     # hidden not bf16
        (H[:, :8], m, t),                      # hidden: wrong d
        (torch.zeros((16, 32), dtype=torch.bfloat16).t(), m, t),  # hidden: transposed view
        (H, m.to(torch.int32), t),             # mask dtype
        (H, m[:31], t),                        # mask length
        (H, m, t.to(torch.int64)),             # tokens dtype
        (H, m, t[:31]),                        # tokens length
    ]
    for args in bad:
        with pytest.raises((TypeError, ValueError)):
            rd.step(*args, k=2)
    # outputs: sizes follow k and the window, dtypes follow the header
    with pytest.raises(ValueError):
        rd.step(H, m, t, k=4, out={"sel_idx": torch.zeros(3, dtype=torch.int32)})
    with pytest.raises(ValueError):
        rd.step(H, m, t, k=2, win_lo=0, win_hi=32, out={"row_conf": torch.zeros(31, dtype=torch.float32)})
    with pytest.raises(TypeError):
        rd.step(H, m, t, k=2, out={"row_conf": torch.zeros(32, dtype=torch.float64)})
    with pytest.raises(KeyError):
        rd.step(H, m, t, k=2, out={"rows": torch.zeros(32, dtype=torch.int32)})
    # a valid call passes the guards and reaches the library (no handle here)
    with pytest.raises(mtl.DllmError):
        rd.step(H, m, t, k=2, win_lo=8, win_hi=16, out={"row_idx": torch.zeros(8, dtype=torch.int32),
                                                        "sel_conf": torch.zeros(2, dtype=torch.float32)})


def test_step_batch_validates_shapes_and_per_sequence_outputs():
    rd = _readout()
    B = 3
    H, m, t = _inputs(B=B)
    seqs = [(2, 0, 32)] * B
    with pytest.raises(ValueError):
        rd.step_batch(H, m[:2], t, seqs)
    with pytest.raises(ValueError):
        rd.step_batch(H, m, t, seqs[:2])
    with pytest.raises(ValueError):
        rd.step_batch(H, m, t, seqs, out={"sel_idx": torch.zeros((B, 3), dtype=torch.int32)})  # stride k_max = 4
    with pytest.raises(ValueError):
        rd.step_batch(H, m, t, seqs, out={"row_tok": torch.zeros((B, 31), dtype=torch.int32)})
    with pytest.raises(mtl.DllmError):
        rd.step_batch(H, m, t, seqs, out={"sel_idx": torch.zeros((B, 4), dtype=torch.int32),
                                          "m_out": torch.zeros(B, dtype=torch.int32)})


def test_ffn_checks_weight_and_activation_shapes():
    F, d = 64, 16
    g = torch.zeros((F, d), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        SwiGLUFFN(g, torch.zeros((F, d + 8), dtype=torch.bfloat16), torch.zeros((d, F), dtype=torch.bfloat16), 8)
    with pytest.raises(ValueError):
        SwiGLUFFN(g, g, torch.zeros((F, d), dtype=torch.bfloat16), 8)   # W_down must be [d, F]
    with pytest.raises(ValueError):
        SwiGLUFFN(g, g, torch.zeros((d, F), dtype=torch.bfloat16), 8)   # host tensors: no device
    ffn = object.__new__(SwiGLUFFN)
    ffn.F, ffn.d, ffn.chunk = F, d, 8
    ffn.W_gu = torch.zeros((2 * F, d), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ffn(torch.zeros((10, d + 1), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        ffn(torch.zeros((10, d), dtype=torch.bfloat16), torch.zeros((9, d), dtype=torch.bfloat16))


def test_check_out_counts_per_field():
    _check_out({"n_out": torch.zeros(1, dtype=torch.int32), "sel_tok": torch.zeros(5, dtype=torch.int32),
                "row_lse": torch.zeros(7, dtype=torch.float32)}, 1, 5, 7, torch.device("cpu"))
    with pytest.raises(ValueError):
        _check_out({"m_out": torch.zeros(2, dtype=torch.int32)}, 3, 1, 1, torch.device("cpu"))
