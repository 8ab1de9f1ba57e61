"""The C-ABI library loads, exports every symbol its header declares, and
rejects bad configurations before touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

import token_decode_llama_amd as lm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lmdecode.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lm_[a-z_0-9]+)\s*\(", text)))


def test_header_declarations_match_binding_list():
    assert _declared_functions() == sorted(lm.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = lm.load()
    for name in _declared_functions():
        assert hasattr(L, name), name


def _good():
    return dict(vocab=512, hidden=256, n_layers=2, n_heads=4, n_kv_heads=2, head_dim=64,
                ffn=704, rms_eps=1e-5, rope_theta=5e5, max_ctx=20, max_seqs=1, qtype=8)


@pytest.mark.parametrize("field,value,needle", [
    ("qtype", 3, "qtype"),
    ("vocab", 511, "vocab"),
    ("hidden", 100, "hidden"),
    ("n_layers", 0, "n_layers"),
    ("n_kv_heads", 3, "n_kv_heads"),
    ("head_dim", 96, "head_dim"),
    ("ffn", 30, "ffn"),
    ("max_ctx", 0, "max_ctx"),
    ("max_seqs", 5, "max_seqs"),
    ("rope_theta", 0.0, "rope_theta"),
    ("rms_eps", float("nan"), "rms_eps"),
    ("ffn", 64 * 1024, "LDS"),
])
def test_create_rejects_bad_config_before_any_device_call(field, value, needle):
    L = lm.load()
    d = _good()
    d[field] = value
    c = lm.Config(**d)
    h = ctypes.c_void_p(123)
    st = L.lm_model_create(ctypes.byref(c), None, ctypes.byref(h))
    assert st == lm.LM_E_ARG
    assert not h.value
    msg = L.lm_last_error(None).decode()
    assert needle in msg and "expected" in msg


@pytest.mark.parametrize("hidden", [6176, 8192])
def test_create_rejects_wide_hidden_for_several_sequences(hidden):
    """2..4 sequences: each GEMV workgroup stages the digits of an
    RMSNorm-gained input (K = hidden) in LDS, at most 6144 columns, so hidden
    is at most 6144 there (one sequence: no limit)."""
    L = lm.load()
    d = _good()
    d.update(hidden=hidden, max_seqs=2)
    c = lm.Config(**d)
    h = ctypes.c_void_p(123)
    assert L.lm_model_create(ctypes.byref(c), None, ctypes.byref(h)) == lm.LM_E_ARG
    assert not h.value
    msg = L.lm_last_error(None).decode()
    assert "hidden" in msg and "6144" in msg


def test_null_arguments():
    L = lm.load()
    assert L.lm_model_create(None, None, None) == lm.LM_E_ARG
    h = ctypes.c_void_p()
    assert L.lm_model_create(None, None, ctypes.byref(h)) == lm.LM_E_ARG
    L.lm_model_destroy(None)   # no-op
    assert L.lm_last_error(None) is not None


# The tier sizing rule of the C/CUDA Llama engine page (section 4.1, compute_tier_sizes):
# tier A = floor(0.9 * free GPU memory / layer bytes), tier B = floor(0.7 *
# available host memory / layer bytes), clamped to the layers left.  Expected
# values worked by hand.
@pytest.mark.parametrize("args,expect", [
    ((80, 10**9, 40 * 10**9, 100 * 10**9), (36, 44, True)),     # 36 of 80 in HBM, the rest fits in host memory
    ((80, 10**9, 40 * 10**9, 50 * 10**9), (36, 35, False)),     # 9 layers would need the disk tier
    ((80, 10**9, 10**12, 0), (80, 0, True)),                    # everything resident
    ((80, 10**9, 0, 200 * 10**9), (0, 80, True)),               # everything streamed
    ((32, 3, 10, 100), (3, 23, False)),                         # 0.9 * 10 / 3 = 3 exactly; 0.7 * 100 / 3 = 23.3
    ((32, 7, 69, 10), (8, 1, False)),                           # 62.1 / 7 = 8.87; 7 / 7 = 1
    ((4, 2**40, 2**62, 2**62), (4, 0, True)),                   # no overflow at large sizes
])
def test_tier_sizes(args, expect):
    assert lm.tier_sizes(*args) == expect


def test_tier_sizes_rejects_bad_arguments():
    L = lm.load()
    a, b = ctypes.c_int32(), ctypes.c_int32()
    assert L.lm_tier_sizes(80, 0, 10, 10, ctypes.byref(a), ctypes.byref(b)) == lm.LM_E_ARG
    assert L.lm_tier_sizes(0, 10, 10, 10, ctypes.byref(a), ctypes.byref(b)) == lm.LM_E_ARG
    assert L.lm_tier_sizes(80, 10, -1, 10, ctypes.byref(a), ctypes.byref(b)) == lm.LM_E_ARG
    assert L.lm_tier_sizes(80, 10, 10, 10, None, ctypes.byref(b)) == lm.LM_E_ARG


@pytest.mark.parametrize("changes,needle", [
    (dict(ffn=704), "ffn"),                               # 704 = 2.75 super-blocks
    (dict(hidden=288, n_heads=4, head_dim=64), "hidden"),
    (dict(n_heads=2, n_kv_heads=2, head_dim=64, hidden=256), "n_heads * head_dim"),
    (dict(max_seqs=2), "max_seqs"),
])
@pytest.mark.parametrize("qtype", [lm.LM_Q4_K, lm.LM_Q5_K, lm.LM_Q6_K])
def test_create_rejects_k_formats_outside_their_shapes(qtype, changes, needle):
    """Q4_K / Q6_K: 256-weight super-blocks along every GEMV input, one
    sequence per step; checked before any device call."""
    L = lm.load()
    d = _good()
    d.update(ffn=768, qtype=qtype)
    d.update(changes)
    c = lm.Config(**d)
    h = ctypes.c_void_p(123)
    assert L.lm_model_create(ctypes.byref(c), None, ctypes.byref(h)) == lm.LM_E_ARG
    assert not h.value
    msg = L.lm_last_error(None).decode()
    assert needle in msg and "expected" in msg
