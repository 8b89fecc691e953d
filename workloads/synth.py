"""Seeded synthetic weights and token ids.

Every named weight tensor draws from its own numpy stream,
`default_rng([seed, layer_slot, slot_id])`, so a tensor's values do not depend on the order
in which tensors are generated and no two slots share values. Distributions:

  projection / embedding / lm_head matrices   N(0, 0.02)
  norm gains                                  1 + N(0, 0.02)
  biases                                      N(0, 0.02)

all rounded once to float16 (round-to-nearest-even). Token ids are uniform in
[0, vocab) from `default_rng([seed, 10**6])`.

Tensors use the nn.Linear layout [out_features, in_features], row-major. Only draws
happen here; no part of the forward pass is computed.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import ModelConfig

# Stable slot ids: a tensor's stream depends on its name, never on generation order.
_SLOT_IDS = {
    "embed": 1, "embed_norm_w": 2, "embed_norm_b": 3, "final_norm_w": 4, "final_norm_b": 5,
    "lm_head": 6, "pos_embed": 7,
    "attn_norm_w": 10, "attn_norm_b": 11, "q_w": 12, "k_w": 13, "v_w": 14, "q_b": 15,
    "k_b": 16, "v_b": 17, "qkv_fused_w": 18, "qkv_fused_b": 19, "q_norm_w": 20,
    "k_norm_w": 21, "o_w": 22, "o_b": 23, "mlp_norm_w": 24, "mlp_norm_b": 25,
    "post_attn_norm_w": 26, "post_ff_norm_w": 27, "gate_w": 28, "up_w": 29, "fc1_w": 30,
    "fc1_b": 31, "down_w": 32, "down_b": 33,
}


def weight_slots(cfg: ModelConfig):
    """Yield (name, shape, kind) for every raw tensor the config uses.

    kind is "matrix", "gain" or "bias". Per-layer names are prefixed "layers.{l}.".
    """
    h, I, V, L = cfg.hidden, cfg.inter, cfg.vocab, cfg.n_layers
    hd = cfg.n_heads * cfg.head_dim
    kvd = cfg.kv_heads * cfg.head_dim
    ln = cfg.norm_kind == "layernorm"
    yield "embed", (V, h), "matrix"
    if cfg.learned_pos:
        yield "pos_embed", (cfg.max_seq, h), "matrix"
    if cfg.embed_norm:
        yield "embed_norm_w", (h,), "gain"
        yield "embed_norm_b", (h,), "bias"
    for l in range(L):
        p = f"layers.{l}."
        if cfg.norm_place == "pre":
            yield p + "attn_norm_w", (h,), "gain"
            if ln:
                yield p + "attn_norm_b", (h,), "bias"
        if cfg.qkv_layout == "fused":
            yield p + "qkv_fused_w", (3 * hd, h), "matrix"
            if cfg.qkv_bias:
                yield p + "qkv_fused_b", (3 * hd,), "bias"
        else:
            for c, n in (("q", hd), ("k", kvd), ("v", kvd)):
                yield p + f"{c}_w", (n, h), "matrix"
            if cfg.qkv_bias:
                for c, n in (("q", hd), ("k", kvd), ("v", kvd)):
                    yield p + f"{c}_b", (n,), "bias"
        if cfg.qk_norm in ("full_rms", "head_ln"):
            yield p + "q_norm_w", (hd,), "gain"
            yield p + "k_norm_w", (kvd,), "gain"
        yield p + "o_w", (h, hd), "matrix"
        if cfg.o_bias:
            yield p + "o_b", (h,), "bias"
        if cfg.parallel_residual:
            pass  # both sublayers read the one input norm
        elif cfg.norm_place == "pre":
            yield p + "mlp_norm_w", (h,), "gain"
            if ln:
                yield p + "mlp_norm_b", (h,), "bias"
        else:
            yield p + "post_attn_norm_w", (h,), "gain"
            yield p + "post_ff_norm_w", (h,), "gain"
        if cfg.mlp_kind == "swiglu":
            yield p + "gate_w", (I, h), "matrix"
            yield p + "up_w", (I, h), "matrix"
        else:
            yield p + "fc1_w", (I, h), "matrix"
            if cfg.mlp_bias:
                yield p + "fc1_b", (I,), "bias"
        yield p + "down_w", (h, I), "matrix"
        if cfg.mlp_bias:
            yield p + "down_b", (h,), "bias"
    yield "final_norm_w", (h,), "gain"
    if ln:
        yield "final_norm_b", (h,), "bias"
    yield "lm_head", (V, h), "matrix"


def _draw(seed: int, name: str, shape, kind: str) -> np.ndarray:
    if name.startswith("layers."):
        _, l, base = name.split(".", 2)
        layer_slot = int(l) + 1
    else:
        layer_slot, base = 0, name
    rng = np.random.default_rng([seed, layer_slot, _SLOT_IDS[base]])
    z = rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    z *= np.float32(0.02)
    if kind == "gain":
        z += np.float32(1.0)
    return z.astype(np.float16)


def synth_weights(cfg: ModelConfig, seed: int | None = None, layers=None) -> dict:
    """Return {name: float16 ndarray} for every slot of `cfg`.

    `layers`, if given, restricts the per-layer tensors to those layer indices (global
    tensors are always included); used to build truncated models cheaply.
    """
    seed = cfg.seed if seed is None else seed
    todo = []
    for name, shape, kind in weight_slots(cfg):
        if layers is not None and name.startswith("layers."):
            if int(name.split(".")[1]) not in layers:
                continue
        todo.append((name, shape, kind))
    # Each slot has its own stream, so drawing slots on several threads gives the same
    # values as drawing them one after another.
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        arrays = list(ex.map(lambda t: _draw(seed, *t), todo))
    return {t[0]: a for t, a in zip(todo, arrays)}


def synth_ids(cfg: ModelConfig, seed: int | None = None, batch=None, seq=None) -> np.ndarray:
    """Uniform token ids in [0, vocab), int32 [batch, seq]."""
    seed = cfg.seed if seed is None else seed
    b = cfg.batch if batch is None else batch
    s = cfg.seq if seq is None else seq
    rng = np.random.default_rng([seed, 10 ** 6])
    return rng.integers(0, cfg.vocab, size=(b, s), dtype=np.int32)
