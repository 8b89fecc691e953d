"""Host-side checks of the C-ABI library (no GPU work is launched): the library loads,
exports every function the header declares, validates configs with the documented error
codes, sizes workspaces, and links nothing beyond the HIP runtime and system libraries."""
import ctypes as C
import os
import re
import subprocess

import pytest

from dense_transformer_prefill_amd import _abi as A
from workloads import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tf_prefill.h")


def _lib():
    if not os.path.exists(A.LIB_PATH):
        pytest.skip("library not built")
    return A.load()


def test_header_exports_match_library():
    lib = _lib()
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:tf_status|void|const char\*)\s+(tf_\w+)\s*\(", text, re.M))
    assert declared == set(A.EXPORTS), declared ^ set(A.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", A.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r" T (tf_\w+)$", out, re.M))
    assert declared <= exported, declared - exported
    for name in declared:
        assert getattr(lib, name) is not None


def test_linkage_hip_runtime_and_system_only():
    """The library links the HIP runtime and the C/C++ runtime only -- no vendor BLAS/DNN."""
    out = subprocess.run(["readelf", "-d", A.LIB_PATH], capture_output=True, text=True).stdout
    needed = re.findall(r"\(NEEDED\)\s+Shared library: \[(.+?)\]", out)
    allowed = re.compile(r"^(libamdhip64\.so.*|libstdc\+\+\.so.*|libm\.so.*|libgcc_s\.so.*|"
                         r"libc\.so.*|ld-linux.*|libdl\.so.*|libpthread\.so.*|librt\.so.*)$")
    assert needed, out
    bad = [n for n in needed if not allowed.match(n)]
    assert not bad, bad
    for forbidden in ("rocblas", "hipblas", "miopen", "mkl", "cublas"):
        assert not any(forbidden in n.lower() for n in needed)


def _cfg(name="c2_stablelm2_b8s2048", **kw):
    cfg = CONFIGS[name].with_(**kw) if kw else CONFIGS[name]
    return A.config_to_c(cfg)


def _validate(c):
    return _lib().tf_config_validate(C.byref(c))


def test_validate_accepts_all_named_configs():
    for name in CONFIGS:
        assert _validate(_cfg(name)) == A.TF_OK, (name, _lib().tf_last_error())


@pytest.mark.parametrize("field,value,code", [
    ("rot_dim", 15, A.TF_ERR_INVALID_ARG),        # odd
    ("rot_dim", 66, A.TF_ERR_INVALID_ARG),        # beyond head_dim
    ("rot_dim", 24, A.TF_ERR_UNSUPPORTED),        # half 12 is not a fused-epilogue span
    ("hidden", 2050, A.TF_ERR_INVALID_ARG),       # heads * head_dim != hidden
    ("n_layers", 0, A.TF_ERR_INVALID_ARG),
    ("vocab", -1, A.TF_ERR_INVALID_ARG),
    ("inter", 100, A.TF_ERR_UNSUPPORTED),
    ("abi_version", 99, A.TF_ERR_INVALID_ARG),
    ("norm_kind", 7, A.TF_ERR_INVALID_ARG),
])
def test_validate_rejects(field, value, code):
    c = _cfg()
    setattr(c, field, value)
    assert _validate(c) == code
    assert _lib().tf_last_error().decode()


def test_validate_alibi_with_rotary_rejected():
    c = _cfg("c3_bloom560m")
    c.rot_dim = 16
    assert _validate(c) == A.TF_ERR_INVALID_ARG
    assert b"alibi" in _lib().tf_last_error()


def test_validate_head_dim_and_post_norm_envelope():
    c = _cfg(n_heads=64, head_dim=32)
    assert _validate(c) == A.TF_ERR_UNSUPPORTED
    c = _cfg(norm_place="post")          # post-norm with LayerNorm
    assert _validate(c) == A.TF_ERR_UNSUPPORTED
    assert _lib().tf_config_validate(None) == A.TF_ERR_INVALID_ARG


def test_workspace_size_monotonic():
    lib = _lib()
    c = _cfg()
    sizes = []
    for b, s in [(1, 1), (1, 512), (8, 2048)]:
        n = C.c_size_t()
        assert lib.tf_workspace_size(C.byref(c), b, s, C.byref(n)) == A.TF_OK
        sizes.append(n.value)
    assert sizes[0] < sizes[1] < sizes[2]
    # C2: fp32 residual, five fp16 [T, h] activations (normed x, q, k, v, attention out)
    # and the fp16 MLP activation [T, I]
    T, h, I = 16384, 2048, 5632
    assert sizes[2] >= T * h * 4 + 5 * T * h * 2 + T * I * 2
    n = C.c_size_t()
    assert lib.tf_workspace_size(C.byref(c), -1, 4, C.byref(n)) == A.TF_ERR_INVALID_ARG


def test_pack_and_prefill_reject_null_arguments():
    lib = _lib()
    c = _cfg("c0_tiny")
    h = C.c_void_p()
    assert lib.tf_weights_pack(C.byref(c), None, None, C.byref(h)) == A.TF_ERR_INVALID_ARG
    assert not h.value
    raw = A.TfRawWeights()          # every slot NULL
    assert lib.tf_weights_pack(C.byref(c), C.byref(raw), None, C.byref(h)) == A.TF_ERR_INVALID_ARG
    assert b"missing weight slot" in lib.tf_last_error()
    assert lib.tf_prefill(C.byref(c), None, None, 1, 1, None, None) == A.TF_ERR_INVALID_ARG
    lib.tf_weights_free(None)
