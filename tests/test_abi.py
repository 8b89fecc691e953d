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


def test_validate_stablelm12b_block_options():
    """The 12B block options: grouped key/value heads must divide the query heads, the
    per-head interleaved fused QKV layout has no grouped form, and the parallel block is a
    pre-norm block."""
    assert _validate(_cfg("c5_slm12b_block_b8s2048")) == A.TF_OK
    c = _cfg(n_kv_heads=8)
    assert _validate(c) == A.TF_OK and c.n_kv_heads == 8
    for kv in (3, 40, -1):
        c = _cfg()
        c.n_kv_heads = kv
        assert _validate(c) == A.TF_ERR_INVALID_ARG, kv
    c = _cfg("c3_bloom560m")
    c.n_kv_heads = 4
    assert _validate(c) == A.TF_ERR_UNSUPPORTED
    assert b"fused" in _lib().tf_last_error()
    c = _cfg("c4_olmo2_1b")
    c.parallel_residual = 1
    assert _validate(c) == A.TF_ERR_UNSUPPORTED
    c = _cfg()
    c.parallel_residual = 2
    assert _validate(c) == A.TF_ERR_INVALID_ARG
    c = _cfg()
    c.qk_norm = 3
    assert _validate(c) == A.TF_ERR_INVALID_ARG


def test_workspace_shrinks_with_grouped_heads():
    """Q | K | V activations take (H + 2 Hkv) d columns per token."""
    lib = _lib()
    n1, n2 = C.c_size_t(), C.c_size_t()
    c1, c2 = _cfg(), _cfg(n_kv_heads=8)
    assert lib.tf_workspace_size(C.byref(c1), 8, 2048, C.byref(n1)) == A.TF_OK
    assert lib.tf_workspace_size(C.byref(c2), 8, 2048, C.byref(n2)) == A.TF_OK
    T, d = 8 * 2048, 64
    assert n1.value - n2.value == T * 2 * (32 - 8) * d * 2


def test_pack_parallel_block_needs_no_mlp_norm():
    """Host-side slot check of the parallel block: with the MLP norm slots left NULL and
    k_norm_w dropped, the error names k_norm_w, which is checked after the MLP norm, so the
    parallel block does not ask for an MLP norm. No device work is reached."""
    lib = _lib()
    cfg = CONFIGS["c5_slm12b_block_b8s2048"].with_(n_layers=1)
    c = A.config_to_c(cfg)
    raw = A.TfRawWeights()
    fake = C.c_void_p(16)
    for f in ("embed", "lm_head", "final_norm_w", "final_norm_b"):
        setattr(raw, f, fake)
    layers = (A.TfRawLayer * 1)()
    for f in ("attn_norm_w", "attn_norm_b", "q_w", "k_w", "v_w", "q_norm_w", "k_norm_w",
              "o_w", "gate_w", "up_w", "down_w"):
        setattr(layers[0], f, fake)
    raw.layers = layers
    layers[0].k_norm_w = None
    h = C.c_void_p()
    assert lib.tf_weights_pack(C.byref(c), C.byref(raw), None, C.byref(h)) == A.TF_ERR_INVALID_ARG
    assert b"k_norm_w" in lib.tf_last_error()


def test_validate_learned_positions():
    """Learned absolute positions are the model's one positional scheme."""
    assert _validate(_cfg("c6_learned_pos_b4s1024")) == A.TF_OK
    c = _cfg("c6_learned_pos_b4s1024")
    c.rot_dim = 16
    assert _validate(c) == A.TF_ERR_UNSUPPORTED
    c = _cfg("c6_learned_pos_b4s1024")
    c.alibi = 1
    assert _validate(c) == A.TF_ERR_UNSUPPORTED
    c = _cfg("c6_learned_pos_b4s1024")
    c.learned_pos = 2
    assert _validate(c) == A.TF_ERR_INVALID_ARG


def test_pack_learned_positions_needs_the_position_table():
    lib = _lib()
    c = A.config_to_c(CONFIGS["c6_learned_pos_b4s1024"].with_(n_layers=1))
    raw = A.TfRawWeights()
    fake = C.c_void_p(16)
    for f in ("embed", "lm_head", "final_norm_w", "final_norm_b"):
        setattr(raw, f, fake)
    layers = (A.TfRawLayer * 1)()
    raw.layers = layers
    h = C.c_void_p()
    assert lib.tf_weights_pack(C.byref(c), C.byref(raw), None, C.byref(h)) == A.TF_ERR_INVALID_ARG
    assert b"pos_embed" in lib.tf_last_error()


def test_validate_weight_format_and_quantizer_arguments():
    assert _validate(_cfg("c7_stablelm2_q8_b8s2048")) == A.TF_OK
    c = _cfg()
    c.weight_format = 5
    assert _validate(c) == A.TF_ERR_INVALID_ARG
    lib = _lib()
    fake = C.c_void_p(16)
    assert lib.tf_quantize_q8_0(None, 4, 32, fake, fake, None) == A.TF_ERR_INVALID_ARG
    assert lib.tf_quantize_q8_0(fake, 4, 48, fake, fake, None) == A.TF_ERR_INVALID_ARG
    assert b"cols" in lib.tf_last_error()
    assert lib.tf_quantize_q8_0(fake, -1, 32, fake, fake, None) == A.TF_ERR_INVALID_ARG


def test_q8_workspace_holds_the_largest_decoded_matrix():
    lib = _lib()
    n16, n8 = C.c_size_t(), C.c_size_t()
    assert lib.tf_workspace_size(C.byref(_cfg()), 8, 2048, C.byref(n16)) == A.TF_OK
    assert lib.tf_workspace_size(C.byref(_cfg("c7_stablelm2_q8_b8s2048")), 8, 2048,
                                 C.byref(n8)) == A.TF_OK
    assert n8.value - n16.value == 100352 * 2048 * 2   # the lm_head, the largest matrix


def test_build_info_names_the_sources_it_was_built_from():
    """tf_build_info() carries the sha256 of the source files the library was compiled
    from; a library built from the sources in this tree reports their current hash."""
    from dense_transformer_prefill_amd import build as B
    info = _lib().tf_build_info().decode()
    m = re.fullmatch(r"sources ([0-9a-f]{64}) git (\S+)", info)
    assert m, info
    assert m.group(1) == B.sources_sha256(), "library is older than its sources: rebuild"
