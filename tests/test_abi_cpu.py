"""The C-ABI library on the host: it loads, exports every declared symbol, and
rejects bad arguments before touching the GPU.  No compute is launched."""
import ctypes as C
import os
import re

import pytest

import masked_token_logits_amd as mtl
from masked_token_logits_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dllm_readout.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

# Fake but 256-byte aligned device addresses: validation never dereferences them.
FAKE = 0x7F0000000000


@pytest.fixture(scope="module")
def lib():
    return mtl.load()


def declared_functions():
    """Every dllm_* function declared in include/*.h."""
    names = set()
    for h in HEADERS:
        names |= set(re.findall(r"\b(dllm_\w+)\s*\(", open(h).read()))
    return sorted(names)


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("dllm_masked_readout_create", "dllm_masked_readout_step", "dllm_masked_readout_destroy"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert sorted(_abi.EXPORTED) == declared_functions()


def test_status_strings(lib):
    for s in range(5):
        assert mtl.dllm_status_string(s)
    assert mtl.dllm_status_string(99) == "unknown status"


def test_workspace_bytes():
    b = mtl.dllm_masked_readout_workspace_bytes(131072, 4096, 126464, 1024)
    # O(L_max * slices) partials of 5 fields (m, a, s, m2, t) + O(L_max) row
    # arrays; never O(L * V)
    assert 0 < b < 131072 * 64 * 20 + 131072 * 40 + (1 << 20)
    assert mtl.dllm_masked_readout_workspace_bytes(0, 4096, 126464, 8) == 0
    assert mtl.dllm_masked_readout_workspace_bytes(10, 4096, 126464, -1) == 0
    assert mtl.dllm_masked_readout_workspace_bytes(10, 4096, 0, 8) == 0
    assert mtl.dllm_masked_readout_workspace_bytes(10, 4096, 126464, mtl.DLLM_K_MAX_LIMIT + 1) == 0
    small = mtl.dllm_masked_readout_workspace_bytes(64, 4096, 126464, 8)
    assert small >= 32 * ((126464 + 127) // 128) * 12


def _create(**kw):
    a = dict(W_lm=FAKE, V=1000, d=64, L_max=512, k_max=16, workspace=FAKE + 0x100000,
             workspace_bytes=1 << 30, stream=None)
    a.update(kw)
    return mtl.dllm_masked_readout_create(**a)


def test_create_validation():
    E = mtl
    assert _create(W_lm=None)[0] == E.DLLM_ERR_INVALID_ARG
    assert _create(V=0)[0] == E.DLLM_ERR_INVALID_ARG
    assert _create(d=0)[0] == E.DLLM_ERR_INVALID_ARG
    assert _create(L_max=0)[0] == E.DLLM_ERR_INVALID_ARG
    assert _create(k_max=-1)[0] == E.DLLM_ERR_INVALID_ARG
    assert _create(k_max=E.DLLM_K_MAX_LIMIT + 1)[0] == E.DLLM_ERR_UNSUPPORTED
    assert _create(d=12)[0] == E.DLLM_ERR_UNSUPPORTED
    assert _create(W_lm=FAKE + 8)[0] == E.DLLM_ERR_UNSUPPORTED
    assert _create(workspace=None)[0] == E.DLLM_ERR_WORKSPACE
    assert _create(workspace_bytes=100)[0] == E.DLLM_ERR_WORKSPACE
    assert _create(workspace=FAKE + 0x100010)[0] == E.DLLM_ERR_WORKSPACE
    st, h = _create()
    assert st == E.DLLM_OK and h
    assert mtl.dllm_masked_readout_destroy(h) == E.DLLM_OK


def test_create_null_out(lib):
    assert lib.dllm_masked_readout_create(None, FAKE, 10, 8, 10, 1, FAKE, 1 << 30, None) == mtl.DLLM_ERR_INVALID_ARG


def test_step_validation_before_any_hip_call():
    st, h = _create()
    assert st == mtl.DLLM_OK
    E = mtl
    H, Mk, T = FAKE + 0x200000, FAKE + 0x300000, FAKE + 0x400000

    def step(**kw):
        a = dict(handle=h, hidden=H, L=256, mask=Mk, tokens=T, k=4, win_lo=0, win_hi=256, block=0)
        a.update(kw)
        return mtl.dllm_masked_readout_step(**a)

    assert step(handle=None) == E.DLLM_ERR_INVALID_ARG
    assert step(hidden=None) == E.DLLM_ERR_INVALID_ARG
    assert step(mask=None) == E.DLLM_ERR_INVALID_ARG
    assert step(tokens=None) == E.DLLM_ERR_INVALID_ARG
    assert step(L=0) == E.DLLM_ERR_INVALID_ARG
    assert step(L=513) == E.DLLM_ERR_INVALID_ARG
    assert step(k=-1) == E.DLLM_ERR_INVALID_ARG
    assert step(k=17) == E.DLLM_ERR_INVALID_ARG
    assert step(win_lo=-1) == E.DLLM_ERR_INVALID_ARG
    assert step(win_lo=10, win_hi=5) == E.DLLM_ERR_INVALID_ARG
    assert step(win_hi=257) == E.DLLM_ERR_INVALID_ARG
    assert step(block=-1) == E.DLLM_ERR_INVALID_ARG
    assert step(hidden=H + 2) == E.DLLM_ERR_UNSUPPORTED
    assert mtl.dllm_masked_readout_set_slices(h, -1) == E.DLLM_ERR_INVALID_ARG
    assert mtl.dllm_masked_readout_set_slices(h, 65) == E.DLLM_ERR_INVALID_ARG
    assert mtl.dllm_masked_readout_set_slices(h, 7) == E.DLLM_OK
    assert mtl.dllm_masked_readout_set_slices(None, 1) == E.DLLM_ERR_INVALID_ARG
    mtl.dllm_masked_readout_destroy(h)


def test_step_ex_policy_validation_before_any_hip_call():
    st, h = _create()
    assert st == mtl.DLLM_OK
    E = mtl
    H, Mk, T = FAKE + 0x200000, FAKE + 0x300000, FAKE + 0x400000

    def step(policy):
        return mtl.dllm_masked_readout_step_ex(h, H, 256, Mk, T, 4, 0, 256, 0, policy)

    assert step(_abi.dllm_policy(3, 0, 0.0)) == E.DLLM_ERR_INVALID_ARG       # unknown score
    assert step(_abi.dllm_policy(-1, 0, 0.0)) == E.DLLM_ERR_INVALID_ARG
    assert step(_abi.dllm_policy(0, 2, 0.0)) == E.DLLM_ERR_INVALID_ARG       # use_threshold not 0/1
    assert step(_abi.dllm_policy(1, 1, float("nan"))) == E.DLLM_ERR_INVALID_ARG
    # argument checks come first, also for step_ex
    assert mtl.dllm_masked_readout_step_ex(h, H, 0, Mk, T, 4, 0, 256, 0, None) == E.DLLM_ERR_INVALID_ARG
    assert mtl.dllm_masked_readout_step_ex(None, H, 256, Mk, T, 4, 0, 256, 0,
                                           mtl.make_policy("margin", 0.5)) == E.DLLM_ERR_INVALID_ARG
    p = mtl.make_policy("neg_entropy", -1.5)
    assert (p.score, p.use_threshold) == (mtl.DLLM_SCORE_NEG_ENTROPY, 1) and abs(p.tau + 1.5) < 1e-7
    assert (mtl.make_policy("conf").use_threshold, mtl.make_policy(1).score) == (0, 1)
    mtl.dllm_masked_readout_destroy(h)


def test_step_batch_validation_before_any_hip_call():
    st, h = _create()            # L_max = 512, k_max = 16
    assert st == mtl.DLLM_OK
    E = mtl
    H, Mk, T = FAKE + 0x200000, FAKE + 0x300000, FAKE + 0x400000

    def step(B=2, L=200, seqs=((4, 0, 200), (2, 10, 50)), block=0, hidden=H, policy=None):
        return mtl.dllm_masked_readout_step_batch(h, B, hidden, L, Mk, T, list(seqs), block, policy)

    assert step(B=0, seqs=()) == E.DLLM_ERR_INVALID_ARG
    assert step(B=E.DLLM_BATCH_MAX + 1, L=1, seqs=[(0, 0, 1)] * (E.DLLM_BATCH_MAX + 1)) == E.DLLM_ERR_INVALID_ARG
    assert step(L=0, seqs=((0, 0, 0), (0, 0, 0))) == E.DLLM_ERR_INVALID_ARG
    assert step(B=3, L=200, seqs=((1, 0, 1),) * 3) == E.DLLM_ERR_INVALID_ARG     # 3 * 200 > L_max
    assert step(seqs=((17, 0, 200), (1, 0, 1))) == E.DLLM_ERR_INVALID_ARG        # k > k_max
    assert step(seqs=((-1, 0, 200), (1, 0, 1))) == E.DLLM_ERR_INVALID_ARG
    assert step(seqs=((1, 0, 201), (1, 0, 1))) == E.DLLM_ERR_INVALID_ARG         # window past L
    assert step(seqs=((1, 5, 4), (1, 0, 1))) == E.DLLM_ERR_INVALID_ARG
    assert step(seqs=((1, 0, 10), (1, -1, 1))) == E.DLLM_ERR_INVALID_ARG
    assert step(block=-1) == E.DLLM_ERR_INVALID_ARG
    assert step(hidden=H + 2) == E.DLLM_ERR_UNSUPPORTED
    assert step(policy=_abi.dllm_policy(7, 0, 0.0)) == E.DLLM_ERR_INVALID_ARG
    assert mtl.dllm_masked_readout_step_batch(None, 1, H, 10, Mk, T, [(1, 0, 10)]) == E.DLLM_ERR_INVALID_ARG
    assert mtl.dllm_masked_readout_step_batch(h, 1, None, 10, Mk, T, [(1, 0, 10)]) == E.DLLM_ERR_INVALID_ARG
    import torch
    if not torch.cuda.is_available():
        # valid arguments reach the device query and report the missing GPU
        assert step(B=2, L=256, seqs=((4, 0, 256), (16, 0, 256))) == E.DLLM_ERR_HIP
    mtl.dllm_masked_readout_destroy(h)


def test_step_out_struct_matches_header():
    """The ctypes struct lists the header's dllm_step_out fields in order."""
    text = open(HEADER).read()
    body = re.search(r"typedef struct \{([^}]*)\} dllm_step_out;", text).group(1)
    fields = re.findall(r"\*\s*(\w+);", body)
    assert fields == [f[0] for f in _abi.dllm_step_out._fields_]
    body = re.search(r"typedef struct \{([^}]*)\} dllm_policy;", text).group(1)
    assert re.findall(r"(\w+);", body) == [f[0] for f in _abi.dllm_policy._fields_]
    body = re.search(r"typedef struct \{([^}]*)\} dllm_seq;", text).group(1)
    assert re.findall(r"(\w+);", body) == [f[0] for f in _abi.dllm_seq._fields_]
    assert int(re.search(r"#define DLLM_BATCH_MAX (\d+)", text).group(1)) == _abi.DLLM_BATCH_MAX


def test_step_without_device_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    st, h = _create()
    r = mtl.dllm_masked_readout_step(h, FAKE + 0x200000, 256, FAKE + 0x300000, FAKE + 0x400000, 4, 0, 256, 0)
    assert r == mtl.DLLM_ERR_HIP
    mtl.dllm_masked_readout_destroy(h)


def test_destroy_null():
    assert mtl.dllm_masked_readout_destroy(None) == mtl.DLLM_OK


def test_ffn_validation_before_any_hip_call():
    E = mtl
    assert mtl.dllm_ffn_workspace_bytes(8192, 12288) == 8192 * 12288 * 2
    assert mtl.dllm_ffn_workspace_bytes(0, 128) == 0 and mtl.dllm_ffn_workspace_bytes(8, 0) == 0
    X, Wgu, Wd, Y, ws = FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, FAKE + 0x400000

    def ffn(X=X, L=1000, d=256, Wgu=Wgu, Wd=Wd, F=384, chunk=256, Y=Y, ws=ws, nbytes=1 << 30):
        return mtl.dllm_ffn_swiglu_chunked(X, L, d, Wgu, Wd, F, chunk, Y, ws, nbytes)

    assert ffn(X=None) == E.DLLM_ERR_INVALID_ARG
    assert ffn(Y=None) == E.DLLM_ERR_INVALID_ARG
    assert ffn(L=-1) == E.DLLM_ERR_INVALID_ARG
    assert ffn(chunk=0) == E.DLLM_ERR_INVALID_ARG
    assert ffn(d=200) == E.DLLM_ERR_UNSUPPORTED            # d % 256
    assert ffn(F=200) == E.DLLM_ERR_UNSUPPORTED            # F % 128
    assert ffn(chunk=1 << 20, F=4096, d=4096) == E.DLLM_ERR_UNSUPPORTED   # 32-bit row offsets
    assert ffn(X=X + 8) == E.DLLM_ERR_UNSUPPORTED
    assert ffn(ws=None) == E.DLLM_ERR_WORKSPACE
    assert ffn(nbytes=100) == E.DLLM_ERR_WORKSPACE
    assert ffn(L=0) == E.DLLM_OK                           # nothing to queue
    assert mtl.dllm_ffn_pack_gate_up(None, FAKE, 128, 64, FAKE) == E.DLLM_ERR_INVALID_ARG
    assert mtl.dllm_ffn_pack_gate_up(FAKE, FAKE, 100, 64, FAKE) == E.DLLM_ERR_UNSUPPORTED
    assert mtl.dllm_ffn_pack_gate_up(FAKE, FAKE, 128, 12, FAKE) == E.DLLM_ERR_UNSUPPORTED
    import torch
    if not torch.cuda.is_available():
        assert ffn() == E.DLLM_ERR_HIP


def test_step_noalloc_validation_before_any_hip_call():
    E = mtl
    W, H, Mk, T = FAKE, FAKE + 0x200000, FAKE + 0x300000, FAKE + 0x400000

    def step(**kw):
        a = dict(W_lm=W, V=1000, d=64, hidden=H, L=256, mask=Mk, tokens=T, k=4, win_lo=0, win_hi=256, block=0)
        a.update(kw)
        return mtl.dllm_masked_readout_step_noalloc(**a)

    assert step(W_lm=None) == E.DLLM_ERR_INVALID_ARG
    assert step(hidden=None) == E.DLLM_ERR_INVALID_ARG
    assert step(mask=None) == E.DLLM_ERR_INVALID_ARG
    assert step(tokens=None) == E.DLLM_ERR_INVALID_ARG
    assert step(L=0) == E.DLLM_ERR_INVALID_ARG
    assert step(V=0) == E.DLLM_ERR_INVALID_ARG
    assert step(k=-1) == E.DLLM_ERR_INVALID_ARG
    assert step(k=E.DLLM_K_MAX_LIMIT + 1) == E.DLLM_ERR_UNSUPPORTED
    assert step(d=60) == E.DLLM_ERR_UNSUPPORTED
    assert step(W_lm=W + 8) == E.DLLM_ERR_UNSUPPORTED
    assert step(hidden=H + 2) == E.DLLM_ERR_UNSUPPORTED
    assert step(win_lo=-1) == E.DLLM_ERR_INVALID_ARG
    assert step(win_lo=10, win_hi=5) == E.DLLM_ERR_INVALID_ARG
    assert step(win_hi=257) == E.DLLM_ERR_INVALID_ARG
    assert step(block=-1) == E.DLLM_ERR_INVALID_ARG
    bad = mtl.dllm_policy(7, 0, 0.0)
    assert step(policy=bad) == E.DLLM_ERR_INVALID_ARG
    # sizes whose workspace exceeds the static scratch: rejected, nothing queued
    big = 200000
    assert mtl.dllm_masked_readout_workspace_bytes(big, 64, 1000, 4) > E.DLLM_NOALLOC_SCRATCH_BYTES
    assert step(L=big, win_hi=big) == E.DLLM_ERR_WORKSPACE
    # the largest L that fits, at the LLaDA-like vocabulary
    fits = [L for L in (4096, 8192, 16384) if
            mtl.dllm_masked_readout_workspace_bytes(L, 4096, 126464, 1024) <= E.DLLM_NOALLOC_SCRATCH_BYTES]
    assert fits == [4096, 8192, 16384]


def test_noalloc_scratch_size_matches_header():
    text = open(os.path.join(ROOT, "include", "dllm_readout.h")).read()
    m = re.search(r"#define DLLM_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _abi.DLLM_NOALLOC_SCRATCH_BYTES


def test_step_noalloc_without_device_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    r = mtl.dllm_masked_readout_step_noalloc(FAKE, 1000, 64, FAKE + 0x200000, 256, FAKE + 0x300000,
                                             FAKE + 0x400000, 4, 0, 256, 0)
    assert r == mtl.DLLM_ERR_HIP


def test_probe_validation_before_any_hip_call():
    E = mtl
    assert mtl.dllm_probe_source_bytes() == 32 << 20
    S, K = FAKE, FAKE + 0x4000000
    assert mtl.dllm_probe_gemm_mix(2, S, 10, K, 256) == E.DLLM_ERR_INVALID_ARG
    assert mtl.dllm_probe_gemm_mix(0, None, 10, K, 256) == E.DLLM_ERR_INVALID_ARG
    assert mtl.dllm_probe_gemm_mix(0, S, 0, K, 256) == E.DLLM_ERR_INVALID_ARG
    assert mtl.dllm_probe_gemm_mix(1, S, 10, None, 256) == E.DLLM_ERR_INVALID_ARG
    assert mtl.dllm_probe_gemm_mix(1, S, 10, K, 0) == E.DLLM_ERR_INVALID_ARG
    assert mtl.dllm_probe_gemm_mix(1, S + 2, 10, K, 256) == E.DLLM_ERR_UNSUPPORTED


def test_probe_wall_clock_without_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert mtl.dllm_probe_wall_clock_khz() == 0
