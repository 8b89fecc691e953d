"""Whole-model pins of the oracle: agreement with Hugging Face transformers' own StableLM,
Bloom and OLMo-2 classes (float64, CPU) on the synthetic weights, model invariants that
hold at any size, and the pages' negative controls reproduced on the oracle."""
import json
import os

import numpy as np
import pytest

import oracle
from workloads import CONFIGS, ModelConfig, synth_ids, synth_weights

from . import hf_reference as hf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

TINY_SLM = ModelConfig(name="tiny_slm", n_layers=2, hidden=256, n_heads=4, head_dim=64,
                       inter=704, vocab=512, batch=2, seq=20, seed=7)
TINY_BLOOM = ModelConfig(name="tiny_bloom", n_layers=2, hidden=256, n_heads=4, head_dim=64,
                         inter=1024, vocab=512, batch=2, seq=20, rot_dim=0, alibi=True,
                         embed_norm=True, qkv_layout="fused", qkv_bias=True, o_bias=True,
                         mlp_bias=True, mlp_kind="gelu_tanh", seed=8)
TINY_OLMO = ModelConfig(name="tiny_olmo", n_layers=2, hidden=256, n_heads=2, head_dim=128,
                        inter=512, vocab=512, batch=2, seq=20, norm_kind="rms",
                        norm_place="post", rot_dim=128, rope_theta=500000.0,
                        qk_norm="full_rms", qkv_bias=False, norm_eps=1e-6, qk_norm_eps=1e-6,
                        seed=9)
TINY_POS = ModelConfig(name="tiny_learned_pos", n_layers=2, hidden=256, n_heads=4, head_dim=64,
                       inter=1024, vocab=512, batch=2, seq=20, max_seq=32, rot_dim=0,
                       learned_pos=True, qkv_bias=True, o_bias=True, mlp_bias=True,
                       mlp_kind="gelu_tanh", seed=10)


def _cos(a, b):
    a = a.reshape(-1, a.shape[-1]).astype(np.float64)
    b = b.reshape(-1, b.shape[-1]).astype(np.float64)
    return (a * b).sum(-1) / np.linalg.norm(a, axis=-1) / np.linalg.norm(b, axis=-1)


# --------------------------------------------------------------- transformers cross-checks
# HF evaluates rotary angles in float32 (StableLM, OLMo-2), RMSNorm in float32 (OLMo-2) and
# GELU with a rounded constant (Bloom); the tolerances allow those and nothing more. The
# "teeth" asserts show that a plausible misreading moves the logits far beyond them.

def test_oracle_matches_hf_stablelm():
    W, ids = synth_weights(TINY_SLM), synth_ids(TINY_SLM)
    ref = hf.stablelm_logits(TINY_SLM, W, ids)
    got = oracle.forward(TINY_SLM, W, ids)
    assert np.abs(got - ref).max() < 1e-7
    # teeth: rotating the full head, or rotating with a 64-dim frequency denominator
    full = oracle.forward(TINY_SLM.with_(rot_dim=64), W, ids)
    assert np.abs(full - ref).max() > 1e-3


@pytest.mark.parametrize("feat", ["parallel", "gqa", "head_ln", "all"])
def test_oracle_matches_hf_stablelm_12b_block(feat):
    """StableLM-2-12B's block options one at a time and together, against HF's class."""
    kw = dict(parallel=dict(parallel_residual=True), gqa=dict(n_kv_heads=2),
              head_ln=dict(qk_norm="head_ln", qk_norm_eps=TINY_SLM.norm_eps),
              all=dict(parallel_residual=True, n_kv_heads=2, qk_norm="head_ln",
                       qk_norm_eps=TINY_SLM.norm_eps, qkv_bias=False))[feat]
    cfg = TINY_SLM.with_(**kw)
    W, ids = synth_weights(cfg), synth_ids(cfg)
    ref = hf.stablelm_logits(cfg, W, ids)
    got = oracle.forward(cfg, W, ids)
    assert np.abs(got - ref).max() < 1e-7
    # teeth: a misreading of the feature moves the logits far beyond the tolerance
    if cfg.parallel_residual:  # the sequential block on the same weights (LN2 := LN1)
        Ws = dict(W)
        for l in range(cfg.n_layers):
            Ws[f"layers.{l}.mlp_norm_w"] = W[f"layers.{l}.attn_norm_w"]
            Ws[f"layers.{l}.mlp_norm_b"] = W[f"layers.{l}.attn_norm_b"]
        seq = oracle.forward(cfg.with_(parallel_residual=False), Ws, ids)
        assert np.abs(seq - ref).max() > 1e-3
    if cfg.kv_heads != cfg.n_heads:  # query head a reading key/value head a % H_kv instead
        Wp = dict(W)
        d, g = cfg.head_dim, cfg.n_heads // cfg.kv_heads
        perm = np.concatenate([np.arange(a * d, (a + 1) * d)
                               for a in [(a % cfg.kv_heads) * g + a // cfg.kv_heads
                                         for a in range(cfg.n_heads)]])
        for l in range(cfg.n_layers):
            Wp[f"layers.{l}.q_w"] = W[f"layers.{l}.q_w"][perm]
            if cfg.qkv_bias:
                Wp[f"layers.{l}.q_b"] = W[f"layers.{l}.q_b"][perm]
            if cfg.qk_norm == "head_ln":
                Wp[f"layers.{l}.q_norm_w"] = W[f"layers.{l}.q_norm_w"][perm]
            Wp[f"layers.{l}.o_w"] = W[f"layers.{l}.o_w"][:, perm]
        wrong = oracle.forward(cfg, Wp, ids)
        assert np.abs(wrong - ref).max() > 1e-3
    if cfg.qk_norm == "head_ln":  # the projections without the per-head norms
        full = oracle.forward(cfg.with_(qk_norm="none"), W, ids)
        assert np.abs(full - ref).max() > 1e-3


def test_oracle_matches_hf_bloom():
    W, ids = synth_weights(TINY_BLOOM), synth_ids(TINY_BLOOM)
    W["lm_head"] = W["embed"]
    ref = hf.bloom_logits(TINY_BLOOM, W, ids)
    got = oracle.forward(TINY_BLOOM, W, ids)
    assert np.abs(got - ref).max() < 1e-7
    # teeth: the [Q; K; V] block reading of the fused tensor
    Wb = dict(W)
    for l in range(TINY_BLOOM.n_layers):
        p = f"layers.{l}."
        q, k, v = np.split(W[p + "qkv_fused_w"], 3)
        Wb[p + "q_w"], Wb[p + "k_w"], Wb[p + "v_w"] = q, k, v
        qb, kb, vb = np.split(W[p + "qkv_fused_b"], 3)
        Wb[p + "q_b"], Wb[p + "k_b"], Wb[p + "v_b"] = qb, kb, vb
    blocks = oracle.forward(TINY_BLOOM.with_(qkv_layout="separate"), Wb, ids)
    assert np.abs(blocks - ref).max() > 1e-3


def test_oracle_matches_hf_gpt2_learned_positions():
    """Learned absolute positions pinned by HF's GPT-2 class (learned position rows added to
    the token embeddings; positions 0..s-1)."""
    W, ids = synth_weights(TINY_POS), synth_ids(TINY_POS)
    ref = hf.gpt2_logits(TINY_POS, W, ids)
    got = oracle.forward(TINY_POS, W, ids)
    assert np.abs(got - ref).max() < 1e-7
    # teeth: dropping the positions, or taking them from the end of the table
    nopos = oracle.forward(TINY_POS.with_(learned_pos=False), W, ids)
    assert np.abs(nopos - ref).max() > 1e-3
    Ws = dict(W)
    Ws["pos_embed"] = W["pos_embed"][::-1].copy()
    assert np.abs(oracle.forward(TINY_POS, Ws, ids) - ref).max() > 1e-3


def test_learned_positions_are_per_position_not_per_token():
    """The same token at two positions gets two different residual rows; at one position
    in two batch rows, the same row."""
    cfg = TINY_POS.with_(n_layers=1)
    W = synth_weights(cfg)
    ids = np.full((2, 5), 7, dtype=np.int32)
    _, res = oracle.forward(cfg, W, ids, residuals=True)
    x0 = res[0]
    assert np.array_equal(x0[0], x0[1])
    assert not np.allclose(x0[0, 0], x0[0, 1])
    np.testing.assert_allclose(x0[0, 3] - x0[0, 2],
                               W["pos_embed"][3].astype(np.float64) - W["pos_embed"][2])


PAD_MASK = np.array([[0, 0, 0, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1],
                     [1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 0, 0, 0, 0]], dtype=np.int32)


@pytest.mark.parametrize("model", ["stablelm", "gpt2"])
def test_oracle_attention_mask_matches_hf(model):
    """Padding through the model's attention_mask ([NNT] The API, zeros are padding): left
    padding in row 0, right padding in row 1. HF's logits at every real position match,
    and at row 1's padding positions too (they see only the real tokens before them).
    HF keeps positions 0..s-1 when called with a mask and no position ids; with learned
    positions that convention is visible, with rotary it is not."""
    cfg = TINY_SLM if model == "stablelm" else TINY_POS
    W, ids = synth_weights(cfg), synth_ids(cfg)
    fn = hf.stablelm_logits if model == "stablelm" else hf.gpt2_logits
    ref = fn(cfg, W, ids, attention_mask=PAD_MASK)
    got = oracle.forward(cfg, W, ids, attention_mask=PAD_MASK)
    real = PAD_MASK.astype(bool)
    scale = max(1.0, np.abs(ref).max())
    assert np.abs(got[real] - ref[real]).max() < 1e-7 * scale
    assert np.abs(got[1] - ref[1]).max() < 1e-7 * scale
    # teeth: ignoring the mask changes the left-padded row's real positions
    nomask = oracle.forward(cfg, W, ids)
    assert np.abs(nomask[0][real[0]] - ref[0][real[0]]).max() > 1e-3


def test_oracle_matches_hf_olmo2():
    W, ids = synth_weights(TINY_OLMO), synth_ids(TINY_OLMO)
    ref = hf.olmo2_logits(TINY_OLMO, W, ids)
    got = oracle.forward(TINY_OLMO, W, ids)
    assert np.abs(got - ref).max() < 2e-6 * max(1.0, np.abs(ref).max())
    # teeth: the post-attention norm loaded into the post-feedforward slot (loader clobber)
    Wc = dict(W)
    for l in range(TINY_OLMO.n_layers):
        Wc[f"layers.{l}.post_ff_norm_w"] = W[f"layers.{l}.post_attn_norm_w"]
    clob = oracle.forward(TINY_OLMO, Wc, ids)
    assert np.abs(clob - ref).max() > 1e-3


# -------------------------------------------------------------------------- config fixture

def test_stablelm2_shape_matches_model_card():
    g = json.load(open(os.path.join(GOLDEN, "stablelm2_1_6b_config.json")))
    for name in ("c1_stablelm2_s512", "c2_stablelm2_b8s2048"):
        c = CONFIGS[name]
        assert c.n_layers == g["num_hidden_layers"] and c.hidden == g["hidden_size"]
        assert c.inter == g["intermediate_size"] and c.n_heads == g["num_attention_heads"]
        assert c.head_dim == g["head_dim"] and c.vocab == g["vocab_size"]
        assert c.rot_dim == g["rotary_dims"] == int(g["head_dim"] * g["partial_rotary_factor"])
        assert c.rope_theta == g["rope_theta"] and c.norm_eps == g["layer_norm_eps"]
        assert c.qkv_bias and not c.o_bias and not c.mlp_bias and c.norm_kind == "layernorm"
        assert c.max_seq >= g["max_position_embeddings"]


# ------------------------------------------------------------------------------ invariants

def test_fp32_oracle_close_to_fp64():
    cfg = CONFIGS["c0_tiny"]
    W, ids = synth_weights(cfg), synth_ids(cfg)
    a = oracle.forward(cfg, W, ids)
    b = oracle.forward(cfg, W, ids, dtype=np.float32)
    assert _cos(a, b).min() > 1 - 1e-9


def test_batch_rows_independent_and_permutable():
    W = synth_weights(TINY_SLM)
    ids = synth_ids(TINY_SLM, batch=3)
    ids[2] = ids[0]
    out = oracle.forward(TINY_SLM, W, ids)
    assert np.array_equal(out[2], out[0])
    perm = oracle.forward(TINY_SLM, W, ids[[1, 0, 2]])
    np.testing.assert_allclose(perm[0], out[1], atol=1e-12)


def test_prefix_consistency_and_causality():
    W = synth_weights(TINY_SLM)
    ids = synth_ids(TINY_SLM)
    full = oracle.forward(TINY_SLM, W, ids)
    pre = oracle.forward(TINY_SLM, W, ids[:, :7])
    np.testing.assert_allclose(pre, full[:, :7], atol=1e-12)
    ids2 = ids.copy()
    ids2[:, 10:] = (ids2[:, 10:] + 1) % TINY_SLM.vocab
    out2 = oracle.forward(TINY_SLM, W, ids2)
    np.testing.assert_allclose(out2[:, :10], full[:, :10], atol=1e-12)
    assert np.abs(out2[:, 10:] - full[:, 10:]).max() > 1e-3


def test_single_token_closed_form():
    """At s = 1 attention returns V_0, so each block is an attention-free map:
    x + (LN1(x) Wv^T + bv) Wo^T, then the MLP. Computed here without any softmax."""
    cfg = TINY_SLM.with_(batch=2, seq=1)
    W, ids = synth_weights(cfg), synth_ids(cfg)
    x = W["embed"][ids].astype(np.float64)
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        g = lambda n: W[p + n].astype(np.float64)
        n1 = oracle.layer_norm(x, g("attn_norm_w"), g("attn_norm_b"), 1e-5)
        x = x + (n1 @ g("v_w").T + g("v_b")) @ g("o_w").T
        n2 = oracle.layer_norm(x, g("mlp_norm_w"), g("mlp_norm_b"), 1e-5)
        x = x + (oracle.silu(n2 @ g("gate_w").T) * (n2 @ g("up_w").T)) @ g("down_w").T
    y = oracle.layer_norm(x, W["final_norm_w"].astype(np.float64),
                          W["final_norm_b"].astype(np.float64), 1e-5)
    ref = y @ W["lm_head"].astype(np.float64).T
    np.testing.assert_allclose(oracle.forward(cfg, W, ids), ref, atol=1e-12)


def test_residual_identity_exact():
    """layer_output == layer_input + attention contribution + mlp contribution, exactly in
    float32 (nnterp StableLM page, "The contributions are the modules' outputs")."""
    cfg = CONFIGS["c0_tiny"]
    W, ids = synth_weights(cfg), synth_ids(cfg)
    x = oracle.embed(cfg, W, ids, np.float32)
    tr = {}
    out = oracle.block(cfg, W, 0, x, np.float32, trace=tr)
    assert out.dtype == np.float32
    assert np.array_equal(tr["layer_input"] + tr["attention_output"] + tr["mlp_output"], out)
    # past the rotary span, the queries equal the projection output split into heads
    n = oracle.layer_norm(x, W["layers.0.attn_norm_w"].astype(np.float32),
                          W["layers.0.attn_norm_b"].astype(np.float32), np.float32(1e-5))
    q_raw = n @ W["layers.0.q_w"].astype(np.float32).T + W["layers.0.q_b"].astype(np.float32)
    q_pre = q_raw.reshape(1, cfg.seq, cfg.n_heads, cfg.head_dim).transpose(0, 2, 1, 3)
    assert np.array_equal(q_pre[..., 16:], tr["attention_queries"][..., 16:])


def test_full_rope_negative_control_on_oracle():
    """Rotating all 64 dims changes every position p >= 1 and leaves p = 0 unchanged (the
    StableLM report's full-RoPE control)."""
    cfg = CONFIGS["c0_tiny"]
    W, ids = synth_weights(cfg), synth_ids(cfg)
    a = oracle.forward(cfg, W, ids)
    b = oracle.forward(cfg.with_(rot_dim=64), W, ids)
    c = _cos(a, b)
    assert c[0] > 1 - 1e-12
    assert c[1:].max() < 1 - 1e-7


def test_alibi_model_finite_without_rotary():
    cfg = TINY_BLOOM.with_(seq=64)
    W, ids = synth_weights(cfg), synth_ids(cfg)
    assert np.isfinite(oracle.forward(cfg, W, ids)).all()


def test_out_of_range_ids_rejected():
    cfg = CONFIGS["c0_tiny"]
    W = synth_weights(cfg)
    with pytest.raises(ValueError):
        oracle.forward(cfg, W, np.array([[0, cfg.vocab]], dtype=np.int32))
