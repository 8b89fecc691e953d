"""ctypes declarations of the C ABI in include/tf_prefill.h (argument marshalling only).

Loading fails loudly if the HIP library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtf_prefill.so")

TF_ABI_VERSION = 5
TF_OK, TF_ERR_INVALID_ARG, TF_ERR_UNSUPPORTED, TF_ERR_OUT_OF_MEMORY, TF_ERR_HIP = 0, 1, 2, 3, 4
TF_NORM_LAYERNORM, TF_NORM_RMS = 0, 1
TF_NORM_PRE, TF_NORM_POST = 0, 1
TF_QK_NORM_NONE, TF_QK_NORM_FULL_RMS, TF_QK_NORM_HEAD_LN = 0, 1, 2
TF_QKV_SEPARATE, TF_QKV_FUSED = 0, 1
TF_MLP_SWIGLU, TF_MLP_GELU_TANH = 0, 1
TF_LOGITS_F32, TF_LOGITS_F16 = 0, 1
TF_WEIGHTS_F16, TF_WEIGHTS_Q8_0 = 0, 1
(TF_KT_NONE, TF_KT_GEMM_QKV, TF_KT_ATTENTION, TF_KT_GEMM_O, TF_KT_GEMM_MLP_UP,
 TF_KT_GEMM_MLP_DOWN, TF_KT_GEMM_LM_HEAD, TF_KT_NORM) = range(8)
KERNEL_CLASSES = {"gemm_qkv": TF_KT_GEMM_QKV, "attention": TF_KT_ATTENTION,
                  "gemm_o": TF_KT_GEMM_O, "gemm_mlp_up": TF_KT_GEMM_MLP_UP,
                  "gemm_mlp_down": TF_KT_GEMM_MLP_DOWN, "gemm_lm_head": TF_KT_GEMM_LM_HEAD,
                  "norm": TF_KT_NORM}


class TfConfig(C.Structure):
    _fields_ = [("abi_version", C.c_int32), ("n_layers", C.c_int32), ("hidden", C.c_int32),
                ("n_heads", C.c_int32), ("head_dim", C.c_int32), ("inter", C.c_int32),
                ("vocab", C.c_int32), ("max_seq", C.c_int32), ("norm_kind", C.c_int32),
                ("norm_place", C.c_int32), ("embed_norm", C.c_int32), ("rot_dim", C.c_int32),
                ("rope_theta", C.c_double), ("alibi", C.c_int32), ("qk_norm", C.c_int32),
                ("qkv_bias", C.c_int32), ("o_bias", C.c_int32), ("mlp_bias", C.c_int32),
                ("qkv_layout", C.c_int32), ("mlp_kind", C.c_int32), ("norm_eps", C.c_float),
                ("qk_norm_eps", C.c_float), ("logits_dtype", C.c_int32),
                ("n_kv_heads", C.c_int32), ("parallel_residual", C.c_int32),
                ("learned_pos", C.c_int32), ("weight_format", C.c_int32)]


RAW_LAYER_SLOTS = ["attn_norm_w", "attn_norm_b", "q_w", "k_w", "v_w", "q_b", "k_b", "v_b",
                   "qkv_fused_w", "qkv_fused_b", "q_norm_w", "k_norm_w", "o_w", "o_b",
                   "mlp_norm_w", "mlp_norm_b", "post_attn_norm_w", "post_ff_norm_w",
                   "gate_w", "up_w", "fc1_w", "fc1_b", "down_w", "down_b"]


class TfRawLayer(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in RAW_LAYER_SLOTS]


class TfRawWeights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("embed_norm_w", C.c_void_p),
                ("embed_norm_b", C.c_void_p), ("layers", C.POINTER(TfRawLayer)),
                ("final_norm_w", C.c_void_p), ("final_norm_b", C.c_void_p),
                ("lm_head", C.c_void_p), ("pos_embed", C.c_void_p)]


class TfPrefillOpts(C.Structure):
    _fields_ = [("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
                ("residual_dump", C.c_void_p), ("timed_kernel", C.c_int32),
                ("attention_mask", C.c_void_p), ("next_token_probs", C.c_void_p)]


EXPORTS = ["tf_config_validate", "tf_weights_pack", "tf_weights_free", "tf_workspace_size",
           "tf_prefill", "tf_prefill_ex", "tf_timing_read", "tf_quantize_q8_0", "tf_last_error",
           "tf_build_info", "tf_prefill_noalloc"]
NOALLOC_SCRATCH_BYTES = 96 << 20

_lib = None


class TfError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"tf_prefill error {code}: {msg}")
        self.code = code


def load(path: str = LIB_PATH):
    """Load the HIP library (once). Raises if it is missing: nothing runs without it."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"HIP library not built: {path} is missing "
                          "(run __graft_entry__.build() or python -m "
                          "dense_transformer_prefill_amd.build)")
    lib = C.CDLL(path)
    P, I32, SZ = C.c_void_p, C.c_int32, C.c_size_t
    lib.tf_config_validate.argtypes = [C.POINTER(TfConfig)]
    lib.tf_weights_pack.argtypes = [C.POINTER(TfConfig), C.POINTER(TfRawWeights), P,
                                    C.POINTER(P)]
    lib.tf_weights_free.argtypes = [P]
    lib.tf_weights_free.restype = None
    lib.tf_workspace_size.argtypes = [C.POINTER(TfConfig), I32, I32, C.POINTER(SZ)]
    lib.tf_prefill.argtypes = [C.POINTER(TfConfig), P, P, I32, I32, P, P]
    lib.tf_prefill_ex.argtypes = [C.POINTER(TfConfig), P, P, I32, I32, P, P,
                                  C.POINTER(TfPrefillOpts)]
    lib.tf_prefill_noalloc.argtypes = [C.POINTER(TfConfig), P, P, I32, I32, P, P]
    lib.tf_timing_read.argtypes = [P, I32, C.POINTER(C.c_double), C.POINTER(I32)]
    lib.tf_quantize_q8_0.argtypes = [P, C.c_int64, C.c_int64, P, P, P]
    lib.tf_last_error.argtypes = []
    lib.tf_last_error.restype = C.c_char_p
    lib.tf_build_info.argtypes = []
    lib.tf_build_info.restype = C.c_char_p
    for f in EXPORTS:
        if f not in ("tf_weights_free", "tf_last_error", "tf_build_info"):
            getattr(lib, f).restype = I32
    _lib = lib
    return lib


def check(status: int):
    if status != TF_OK:
        raise TfError(status, load().tf_last_error().decode())


def config_to_c(cfg, logits_dtype: int = TF_LOGITS_F32) -> TfConfig:
    """Fill a tf_config from any object with the ModelConfig attribute names."""
    c = TfConfig()
    c.abi_version = TF_ABI_VERSION
    for f in ("n_layers", "hidden", "n_heads", "head_dim", "inter", "vocab", "max_seq",
              "rot_dim"):
        setattr(c, f, int(getattr(cfg, f)))
    c.norm_kind = TF_NORM_LAYERNORM if cfg.norm_kind == "layernorm" else TF_NORM_RMS
    c.norm_place = TF_NORM_PRE if cfg.norm_place == "pre" else TF_NORM_POST
    c.embed_norm = int(bool(cfg.embed_norm))
    c.rope_theta = float(cfg.rope_theta)
    c.alibi = int(bool(cfg.alibi))
    c.qk_norm = {"none": TF_QK_NORM_NONE, "full_rms": TF_QK_NORM_FULL_RMS,
                 "head_ln": TF_QK_NORM_HEAD_LN}[cfg.qk_norm]
    c.qkv_bias, c.o_bias, c.mlp_bias = (int(bool(cfg.qkv_bias)), int(bool(cfg.o_bias)),
                                        int(bool(cfg.mlp_bias)))
    c.qkv_layout = TF_QKV_FUSED if cfg.qkv_layout == "fused" else TF_QKV_SEPARATE
    c.mlp_kind = TF_MLP_SWIGLU if cfg.mlp_kind == "swiglu" else TF_MLP_GELU_TANH
    c.norm_eps = float(cfg.norm_eps)
    c.qk_norm_eps = float(cfg.qk_norm_eps)
    c.logits_dtype = logits_dtype
    c.n_kv_heads = int(getattr(cfg, "n_kv_heads", 0) or 0)
    c.parallel_residual = int(bool(getattr(cfg, "parallel_residual", False)))
    c.learned_pos = int(bool(getattr(cfg, "learned_pos", False)))
    c.weight_format = {"f16": TF_WEIGHTS_F16, "q8_0": TF_WEIGHTS_Q8_0}[
        getattr(cfg, "weight_format", "f16")]
    return c
