"""Model/workload configurations.

A `ModelConfig` fixes the architecture flags of one dense decoder-only model and the
(batch, seq) of one prefill call. The five named workloads are

  c0_tiny          tiny StableLM-2-style model, batch 1, seq 12
  c1_stablelm2_s512    StableLM-2-1.6B shape, batch 1, seq 512
  c2_stablelm2_b8s2048 StableLM-2-1.6B shape, batch 8, seq 2048 (throughput size)
  c3_bloom560m     Bloom-560m shape with ALiBi, batch 4, seq 1024
  c4_olmo2_1b      OLMo-2-1B shape with post-norm and full-width QK RMSNorm, batch 4, seq 4096
  c5_slm12b_block_b8s2048  StableLM-2-1.6B sizes with StableLM-2-12B's block: parallel
                   residual, 8 key/value heads, per-head Q/K LayerNorm, no QKV bias
  c6_learned_pos_b4s1024   learned absolute positions on GPT-2-small sizes
  c7_stablelm2_q8_b8s2048  the throughput size with Q8_0 weights
  c2_share_b1s2048 one batch row of the throughput size (one GPU's data-parallel share)

StableLM-2-1.6B sizes follow the model card's config listing (nnterp encyclopedia,
"StableLM" page, "Config" and "Printout" sections): 24 layers, hidden 2048, 32 heads of
64, intermediate 5632, vocab 100352, LayerNorm eps 1e-5, partial rotary factor 0.25,
rope theta 10000, biased q/k/v projections, untied lm_head.
"""
from __future__ import annotations

from dataclasses import dataclass, replace, asdict


@dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    hidden: int
    n_heads: int
    head_dim: int
    inter: int
    vocab: int
    batch: int
    seq: int
    max_seq: int = 4096
    norm_kind: str = "layernorm"      # "layernorm" (gain + bias) or "rms" (gain only)
    norm_place: str = "pre"           # "pre": x + f(norm(x)); "post": x + norm(f(x))
    embed_norm: bool = False          # LayerNorm on the embeddings before block 0
    rot_dim: int = 16                 # leading head dims that are rotated (0 = no RoPE)
    rope_theta: float = 10000.0
    alibi: bool = False               # per-head linear pre-softmax bias
    qk_norm: str = "none"             # "none", "full_rms" (RMSNorm over the whole Q/K row) or
                                      # "head_ln" (LayerNorm without bias per Q / KV head)
    n_kv_heads: int = 0               # key/value heads (0 = n_heads); divides n_heads
    parallel_residual: bool = False   # out = x + attn(LN1(x)) + mlp(LN1(x)); no second norm
    learned_pos: bool = False         # learned absolute position rows [max_seq, h] added to
                                      # the token embeddings (positions 0..s-1)
    weight_format: str = "f16"        # "f16", or "q8_0": every projection matrix and the
                                      # lm_head stored as int8 blocks of 32 with an fp16 scale
    qkv_bias: bool = True
    o_bias: bool = False
    mlp_bias: bool = False
    qkv_layout: str = "separate"      # "separate" q/k/v tensors, or "fused" per-head interleaved
    mlp_kind: str = "swiglu"          # "swiglu" or "gelu_tanh"
    norm_eps: float = 1e-5
    qk_norm_eps: float = 1e-6
    seed: int = 0                     # seed of the synthetic weights and ids

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def kv_heads(self) -> int:
        return self.n_kv_heads or self.n_heads

    def with_(self, **kw) -> "ModelConfig":
        return replace(self, **kw)

    def to_dict(self) -> dict:
        return asdict(self)

    def flops(self) -> float:
        """Algorithmic FLOPs of one prefill (2 per multiply-add; causal pairs j <= i only)."""
        T, h, I, V, L = self.tokens, self.hidden, self.inter, self.vocab, self.n_layers
        hd = self.n_heads * self.head_dim
        g = 2 if self.mlp_kind == "swiglu" else 1
        s = self.seq
        kvd = self.kv_heads * self.head_dim
        per_layer = (2 * T * h * (hd + 2 * kvd) + 2 * T * hd * h + 2 * T * h * g * I + 2 * T * I * h
                     + 4 * self.batch * self.n_heads * self.head_dim * s * (s + 1) // 2)
        return float(L * per_layer + 2 * T * h * V)


_STABLELM2_1_6B = dict(n_layers=24, hidden=2048, n_heads=32, head_dim=64, inter=5632,
                       vocab=100352, rot_dim=16, rope_theta=10000.0, norm_kind="layernorm",
                       qkv_bias=True, mlp_kind="swiglu", norm_eps=1e-5)

CONFIGS = {
    "c0_tiny": ModelConfig(name="c0_tiny", n_layers=2, hidden=256, n_heads=4, head_dim=64,
                           inter=704, vocab=1024, batch=1, seq=12, rot_dim=16,
                           rope_theta=10000.0, seed=0),
    "c1_stablelm2_s512": ModelConfig(name="c1_stablelm2_s512", batch=1, seq=512, seed=1,
                                     **_STABLELM2_1_6B),
    "c2_stablelm2_b8s2048": ModelConfig(name="c2_stablelm2_b8s2048", batch=8, seq=2048,
                                        seed=2, **_STABLELM2_1_6B),
    "c3_bloom560m": ModelConfig(name="c3_bloom560m", n_layers=24, hidden=1024, n_heads=16,
                                head_dim=64, inter=4096, vocab=250880, batch=4, seq=1024,
                                rot_dim=0, alibi=True, embed_norm=True, qkv_layout="fused",
                                qkv_bias=True, o_bias=True, mlp_bias=True,
                                mlp_kind="gelu_tanh", norm_kind="layernorm", norm_eps=1e-5,
                                seed=3),
    "c4_olmo2_1b": ModelConfig(name="c4_olmo2_1b", n_layers=16, hidden=2048, n_heads=16,
                               head_dim=128, inter=8192, vocab=100352, batch=4, seq=4096,
                               norm_kind="rms", norm_place="post", rot_dim=128,
                               rope_theta=500000.0, qk_norm="full_rms", qkv_bias=False,
                               mlp_kind="swiglu", norm_eps=1e-6, qk_norm_eps=1e-6, seed=4),
    # StableLM-2-12B's block ([NNT] Notes: parallel residual, qk_layernorm, 32 query heads
    # over 8 key/value heads, no qkv bias) on the 1.6B sizes: 12B's own head_dim of 160 is
    # outside what the attention kernel runs (64, 128).
    "c5_slm12b_block_b8s2048": ModelConfig(name="c5_slm12b_block_b8s2048", batch=8, seq=2048,
                                           seed=5, **{**_STABLELM2_1_6B, "qkv_bias": False},
                                           n_kv_heads=8, parallel_residual=True,
                                           qk_norm="head_ln", qk_norm_eps=1e-5),
    # Learned-absolute positions ([BLM] Contribution: the third positional paradigm the
    # engine spans, beside RoPE and ALiBi) on a GPT-2-small-sized pre-norm LayerNorm block
    # with biases and a tanh-GELU MLP; no rotary, no ALiBi.
    "c6_learned_pos_b4s1024": ModelConfig(name="c6_learned_pos_b4s1024", n_layers=12,
                                          hidden=768, n_heads=12, head_dim=64, inter=3072,
                                          vocab=50257, batch=4, seq=1024, max_seq=1024,
                                          rot_dim=0, learned_pos=True, qkv_bias=True,
                                          o_bias=True, mlp_bias=True, mlp_kind="gelu_tanh",
                                          norm_kind="layernorm", norm_eps=1e-5, seed=6),
    # One GPU's share of the benchmark workload split data-parallel over 8 GPUs: one batch
    # row of 2048 tokens, the same weights (same seed) and the ids of the benchmark's row 0.
    "c2_share_b1s2048": ModelConfig(name="c2_share_b1s2048", batch=1, seq=2048, seed=2,
                                    **_STABLELM2_1_6B),
    # The benchmark shape with Q8_0 weights (the pages' q8 results; GGUF's Q8_0 encoding).
    "c7_stablelm2_q8_b8s2048": ModelConfig(name="c7_stablelm2_q8_b8s2048", batch=8, seq=2048,
                                           seed=7, weight_format="q8_0", **_STABLELM2_1_6B),
}

# Order of the named workloads (their index is also their default seed).
CONFIG_ORDER = ["c0_tiny", "c1_stablelm2_s512", "c2_stablelm2_b8s2048", "c3_bloom560m",
                "c4_olmo2_1b", "c5_slm12b_block_b8s2048", "c6_learned_pos_b4s1024",
                "c7_stablelm2_q8_b8s2048", "c2_share_b1s2048"]


def config_by_name(name: str) -> ModelConfig:
    return CONFIGS[name]
