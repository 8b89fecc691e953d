"""Run Hugging Face transformers' own model classes (StableLM, Bloom, OLMo-2), in float64
on the CPU, on the repository's synthetic weights. Used only to pin the oracle: the
transformers implementations are independent of this repository's code."""
import numpy as np
import torch


def _t(a):
    return torch.from_numpy(np.asarray(a).astype(np.float64))


def _run(model, sd, ids, attention_mask=None):
    missing, unexpected = model.load_state_dict({k: _t(v) for k, v in sd.items()}, strict=False)
    assert not unexpected, unexpected
    # only non-persistent buffers may be absent from the state dict
    assert all("rotary" in k or "inv_freq" in k for k in missing), missing
    kw = {}
    if attention_mask is not None:
        kw["attention_mask"] = torch.from_numpy(np.asarray(attention_mask, dtype=np.int64))
    with torch.no_grad():
        return model(torch.from_numpy(np.asarray(ids, dtype=np.int64)), **kw).logits.numpy()


def stablelm_logits(cfg, W, ids, attention_mask=None):
    """StableLM(-2) in HF's own class; the 12B block's options (parallel residual, per-head
    q/k LayerNorm, grouped key/value heads) map to use_parallel_residual, qk_layernorm and
    num_key_value_heads. HF's per-head norms use layer_norm_eps, so callers set
    qk_norm_eps == norm_eps for qk_norm "head_ln"."""
    from transformers import StableLmConfig, StableLmForCausalLM
    head_ln = cfg.qk_norm == "head_ln"
    assert cfg.qk_norm in ("none", "head_ln") and (not head_ln or cfg.qk_norm_eps == cfg.norm_eps)
    hc = StableLmConfig(vocab_size=cfg.vocab, intermediate_size=cfg.inter,
                        hidden_size=cfg.hidden, num_hidden_layers=cfg.n_layers,
                        num_attention_heads=cfg.n_heads, num_key_value_heads=cfg.kv_heads,
                        max_position_embeddings=cfg.max_seq, layer_norm_eps=cfg.norm_eps,
                        use_qkv_bias=cfg.qkv_bias, qk_layernorm=head_ln,
                        use_parallel_residual=cfg.parallel_residual, tie_word_embeddings=False,
                        rope_parameters={"rope_type": "default", "rope_theta": cfg.rope_theta,
                                         "partial_rotary_factor": cfg.rot_dim / cfg.head_dim})
    m = StableLmForCausalLM(hc).double().eval()
    sd = {"model.embed_tokens.weight": W["embed"], "model.norm.weight": W["final_norm_w"],
          "model.norm.bias": W["final_norm_b"], "lm_head.weight": W["lm_head"]}
    d = cfg.head_dim
    for l in range(cfg.n_layers):
        p, q = f"layers.{l}.", f"model.layers.{l}."
        for c in "qkvo":
            sd[q + f"self_attn.{c}_proj.weight"] = W[p + f"{c}_w"]
        if cfg.qkv_bias:
            for c in "qkv":
                sd[q + f"self_attn.{c}_proj.bias"] = W[p + f"{c}_b"]
        if head_ln:
            for c, n in (("q", cfg.n_heads), ("k", cfg.kv_heads)):
                g = np.asarray(W[p + f"{c}_norm_w"])
                for a in range(n):
                    sd[q + f"self_attn.{c}_layernorm.norms.{a}.weight"] = g[a * d:(a + 1) * d]
        for c in ("gate", "up", "down"):
            sd[q + f"mlp.{c}_proj.weight"] = W[p + f"{c}_w"]
        sd[q + "input_layernorm.weight"] = W[p + "attn_norm_w"]
        sd[q + "input_layernorm.bias"] = W[p + "attn_norm_b"]
        if not cfg.parallel_residual:
            sd[q + "post_attention_layernorm.weight"] = W[p + "mlp_norm_w"]
            sd[q + "post_attention_layernorm.bias"] = W[p + "mlp_norm_b"]
    return _run(m, sd, ids, attention_mask)


def bloom_logits(cfg, W, ids):
    """Bloom ties lm_head to the embeddings; callers pass W with W['lm_head'] is W['embed']."""
    from transformers import BloomConfig, BloomForCausalLM
    assert cfg.inter == 4 * cfg.hidden
    hc = BloomConfig(vocab_size=cfg.vocab, hidden_size=cfg.hidden, n_layer=cfg.n_layers,
                     n_head=cfg.n_heads, layer_norm_epsilon=cfg.norm_eps,
                     tie_word_embeddings=True)
    m = BloomForCausalLM(hc).double().eval()
    sd = {"transformer.word_embeddings.weight": W["embed"],
          "transformer.word_embeddings_layernorm.weight": W["embed_norm_w"],
          "transformer.word_embeddings_layernorm.bias": W["embed_norm_b"],
          "transformer.ln_f.weight": W["final_norm_w"], "transformer.ln_f.bias": W["final_norm_b"],
          "lm_head.weight": W["lm_head"]}
    for l in range(cfg.n_layers):
        p, q = f"layers.{l}.", f"transformer.h.{l}."
        sd[q + "input_layernorm.weight"] = W[p + "attn_norm_w"]
        sd[q + "input_layernorm.bias"] = W[p + "attn_norm_b"]
        sd[q + "post_attention_layernorm.weight"] = W[p + "mlp_norm_w"]
        sd[q + "post_attention_layernorm.bias"] = W[p + "mlp_norm_b"]
        sd[q + "self_attention.query_key_value.weight"] = W[p + "qkv_fused_w"]
        sd[q + "self_attention.query_key_value.bias"] = W[p + "qkv_fused_b"]
        sd[q + "self_attention.dense.weight"] = W[p + "o_w"]
        sd[q + "self_attention.dense.bias"] = W[p + "o_b"]
        sd[q + "mlp.dense_h_to_4h.weight"] = W[p + "fc1_w"]
        sd[q + "mlp.dense_h_to_4h.bias"] = W[p + "fc1_b"]
        sd[q + "mlp.dense_4h_to_h.weight"] = W[p + "down_w"]
        sd[q + "mlp.dense_4h_to_h.bias"] = W[p + "down_b"]
    return _run(m, sd, ids)


def olmo2_logits(cfg, W, ids):
    from transformers import Olmo2Config, Olmo2ForCausalLM
    hc = Olmo2Config(vocab_size=cfg.vocab, hidden_size=cfg.hidden, intermediate_size=cfg.inter,
                     num_hidden_layers=cfg.n_layers, num_attention_heads=cfg.n_heads,
                     num_key_value_heads=cfg.n_heads, rms_norm_eps=cfg.norm_eps,
                     rope_parameters={"rope_type": "default", "rope_theta": cfg.rope_theta},
                     tie_word_embeddings=False, attention_bias=False,
                     max_position_embeddings=cfg.max_seq, eos_token_id=None, pad_token_id=None)
    m = Olmo2ForCausalLM(hc).double().eval()
    sd = {"model.embed_tokens.weight": W["embed"], "model.norm.weight": W["final_norm_w"],
          "lm_head.weight": W["lm_head"]}
    for l in range(cfg.n_layers):
        p, q = f"layers.{l}.", f"model.layers.{l}."
        for c in "qkvo":
            sd[q + f"self_attn.{c}_proj.weight"] = W[p + f"{c}_w"]
        sd[q + "self_attn.q_norm.weight"] = W[p + "q_norm_w"]
        sd[q + "self_attn.k_norm.weight"] = W[p + "k_norm_w"]
        for c in ("gate", "up", "down"):
            sd[q + f"mlp.{c}_proj.weight"] = W[p + f"{c}_w"]
        sd[q + "post_attention_layernorm.weight"] = W[p + "post_attn_norm_w"]
        sd[q + "post_feedforward_layernorm.weight"] = W[p + "post_ff_norm_w"]
    return _run(m, sd, ids)


def gpt2_logits(cfg, W, ids, attention_mask=None):
    """A learned-absolute-position model in HF's GPT-2 class: pre-norm LayerNorm blocks with
    biases, tanh-GELU ("gelu_new") MLP, Q | K | V from one Conv1D ([in, out] layout, so the
    nn.Linear tensors enter transposed), untied lm_head."""
    from transformers import GPT2Config, GPT2LMHeadModel
    assert cfg.learned_pos and cfg.rot_dim == 0 and not cfg.alibi
    hc = GPT2Config(vocab_size=cfg.vocab, n_positions=cfg.max_seq, n_embd=cfg.hidden,
                    n_layer=cfg.n_layers, n_head=cfg.n_heads, n_inner=cfg.inter,
                    activation_function="gelu_new", layer_norm_epsilon=cfg.norm_eps,
                    resid_pdrop=0.0, embd_pdrop=0.0, attn_pdrop=0.0, tie_word_embeddings=False)
    m = GPT2LMHeadModel(hc).double().eval()
    T = lambda a: np.ascontiguousarray(np.asarray(a).T)
    sd = {"transformer.wte.weight": W["embed"], "transformer.wpe.weight": W["pos_embed"],
          "transformer.ln_f.weight": W["final_norm_w"], "transformer.ln_f.bias": W["final_norm_b"],
          "lm_head.weight": W["lm_head"]}
    for l in range(cfg.n_layers):
        p, q = f"layers.{l}.", f"transformer.h.{l}."
        sd[q + "ln_1.weight"] = W[p + "attn_norm_w"]
        sd[q + "ln_1.bias"] = W[p + "attn_norm_b"]
        sd[q + "ln_2.weight"] = W[p + "mlp_norm_w"]
        sd[q + "ln_2.bias"] = W[p + "mlp_norm_b"]
        sd[q + "attn.c_attn.weight"] = T(np.concatenate([W[p + "q_w"], W[p + "k_w"], W[p + "v_w"]]))
        sd[q + "attn.c_attn.bias"] = np.concatenate([W[p + "q_b"], W[p + "k_b"], W[p + "v_b"]])
        sd[q + "attn.c_proj.weight"] = T(W[p + "o_w"])
        sd[q + "attn.c_proj.bias"] = W[p + "o_b"]
        sd[q + "mlp.c_fc.weight"] = T(W[p + "fc1_w"])
        sd[q + "mlp.c_fc.bias"] = W[p + "fc1_b"]
        sd[q + "mlp.c_proj.weight"] = T(W[p + "down_w"])
        sd[q + "mlp.c_proj.bias"] = W[p + "down_b"]
    return _run(m, sd, ids, attention_mask)
