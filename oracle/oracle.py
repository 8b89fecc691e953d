"""Plain CPU oracle of the dense decoder-only prefill forward (token ids -> logits).

TEST INFRASTRUCTURE ONLY. This module is imported by `tests/`, by `__graft_entry__.smoke()`
and by the `cpu_baseline` leg of `bench.py`, and by nothing else. It shares no code with the
HIP library: no kernels, tables, constants or helpers.

It is the plain definition of the forward, written out in numpy with one library primitive
(matrix multiply, `@`). Everything is computed in `dtype` (float64 by default; float32 on
request for the large sampled checks), from the float16 weights upcast exactly. Nothing is
blocked, fused or reordered beyond what the definitions below state.

Sources (page title, then section):
  [SLM]   "StableLM-2: partial RoPE and a first LayerNorm-with-bias path in a dense ROCm
          engine" -- Abstract, 1. Contribution, 4. Ablations / Negative controls.
  [NNT]   nnterp encyclopedia, "stablelm" page -- "The block", "Printout", "Config",
          "The Notes" (sequential block; rotary on a quarter of each head; biased q/k/v;
          query scale; readout and tokenizer).
  [BLM]   "Bloom in a sovereign engine: ALiBi as the third positional paradigm" --
          Contribution, Ablations / Negative controls.
  [OLMO]  "OLMo-2: reordered (post) normalization and a loader-clobber root-cause" --
          1. Contribution, 4. Ablations / Negative controls.

Readings taken where the pages are silent (each is also listed with its reason in the
design notes of the repository):
  rope frequency   f_i = theta^(-2i/r) over the rotated span r (i < r/2), pairs (i, i+r/2)
  rope angles      f_i and p * f_i evaluated in float64 from the exact positions 0..s-1,
                   cos and sin rounded once to the working dtype
  layer norm       population variance, eps inside the square root
  rms norm         z / sqrt(mean(z^2) + eps) * w
  alibi slopes     m_a = 2^(-8(a+1)/H) for head a = 0..H-1; bias m_a * (j - i), unscaled
  fused qkv        row a*3d + c*d + e of the fused tensor is (head a, c in q/k/v, dim e)
  gelu             tanh approximation
  post-norm qk     RMSNorm over the whole Q (and K) projection row, before the head split
  per-head qk norm LayerNorm without bias over each head's d dims, epsilon qk_norm_eps
  grouped kv heads query head a reads key/value head a // (H / H_kv)
  learned positions the row of position p (0..s-1) is added to the token embedding, before
                   any embedding LayerNorm
  attention mask   zeros mark padding keys, excluded for every query; positions stay
                   0..s-1; a query with no key left outputs zero attention
  next-token probs softmax over the vocabulary of the logits at position s-1
  q8 weights       GGUF Q8_0 on every projection matrix and the lm_head: blocks of 32 along
                   the input dimension, scale max|x|/127 in float16, codes rounded half away
                   from zero in float32
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------- primitives


def layer_norm(z, w, b, eps):
    """LayerNorm with gain and bias over the last axis ([NNT] Printout: LayerNorm((2048,),
    eps=1e-05, elementwise_affine=True, bias=True); [SLM] Contribution: LayerNorm-with-bias).
    Population variance, eps inside the square root."""
    mu = z.mean(axis=-1, keepdims=True)
    c = z - mu
    var = (c * c).mean(axis=-1, keepdims=True)
    y = c / np.sqrt(var + eps)
    y = y * w
    if b is not None:
        y = y + b
    return y


def rms_norm(z, w, eps):
    """RMSNorm with gain over the last axis ([OLMO] Contribution: post-attention and
    post-feedforward norms, and the full-width Q/K norm)."""
    ms = (z * z).mean(axis=-1, keepdims=True)
    return z / np.sqrt(ms + eps) * w


def rope_frequencies(rot_dim, theta, dtype):
    """f_i = theta^(-2i/r), i = 0 .. r/2-1 ([NNT] Notes, "Rotary turns a quarter of each
    head": the first r dims are rotated as two halves; rope_theta from the Config)."""
    half = rot_dim // 2
    i = np.arange(half, dtype=dtype)
    return np.power(dtype(theta), -2.0 * i / dtype(rot_dim)).astype(dtype)


def apply_rope(u, positions, rot_dim, theta):
    """Split-half (NeoX) rotary on the first `rot_dim` dims of the last axis; the rest
    pass through unchanged ([SLM] Abstract: span 16 of 64, NeoX split-half; [NNT] Notes:
    dims past the span equal the projection's output).

    u: [..., s, d]; positions: [s] integers. For i < r/2 and angle phi = p * f_i:
        u'_i        = u_i cos phi - u_{i+r/2} sin phi
        u'_{i+r/2}  = u_{i+r/2} cos phi + u_i sin phi
    """
    if rot_dim == 0:
        return u
    dt = u.dtype.type
    half = rot_dim // 2
    # The angle is formed in float64 whatever the working dtype (in float32, p * f_i alone
    # would carry about 2e-4 rad of rounding at p = 4095); cos and sin are then rounded
    # once to the working dtype.
    f = rope_frequencies(rot_dim, theta, np.float64)
    phi = np.asarray(positions, dtype=np.float64)[:, None] * f[None, :]   # [s, half]
    cos, sin = np.cos(phi).astype(dt), np.sin(phi).astype(dt)
    lo = u[..., :half]
    hi = u[..., half:rot_dim]
    out = u.copy()
    out[..., :half] = lo * cos - hi * sin
    out[..., half:rot_dim] = hi * cos + lo * sin
    return out


def alibi_slopes(n_heads, dtype=np.float64):
    """Per-head geometric slopes m_a = 2^(-8(a+1)/H) ([BLM] Contribution: per-head
    geometric-series slope applied as a linear pre-softmax bias)."""
    a = np.arange(1, n_heads + 1, dtype=np.float64)
    return np.power(2.0, -8.0 * a / n_heads).astype(dtype)


def silu(z):
    """SiLU(z) = z / (1 + e^-z) ([NNT] Config: hidden_act silu)."""
    return z / (1.0 + np.exp(-z))


def gelu_tanh(z):
    """GELU, tanh approximation: z/2 (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))."""
    dt = z.dtype.type
    c = dt(np.sqrt(2.0 / np.pi))
    return dt(0.5) * z * (dt(1.0) + np.tanh(c * (z + dt(0.044715) * z * z * z)))


def causal_attention(q, k, v, slopes=None, key_mask=None):
    """Causal softmax attention, one batch row at a time.

    q: [b, H, s, d]; k, v: [b, H_kv, s, d] with H_kv dividing H -- key/value head j serves
    query heads j*H/H_kv .. (j+1)*H/H_kv - 1 ([NNT] Notes, "Grouped-query attention on
    12B"), so each is repeated for its group. Scores S_ij = (q_i . k_j) * d^-1/2 (+ m_a (j - i) with ALiBi),
    keys j > i excluded, softmax over j with the row max subtracted, output sum_j P_ij v_j
    ([NNT] Notes: query scale head_dim ** -0.5, no window, softcap or sink; the attention
    scores are masked before the softmax; [BLM] Contribution: linear pre-softmax bias).
    key_mask: optional bool [b, s]; False marks a padding position ([NNT] The API:
    attention_mask, zeros are padding), which no query attends to. A query with no key left
    (a padding position before the row's first token) gets a zero output.
    Returns [b, H, s, d].
    """
    b, H, s, d = q.shape
    Hkv = k.shape[1]
    assert H % Hkv == 0
    if Hkv != H:
        k = np.repeat(k, H // Hkv, axis=1)
        v = np.repeat(v, H // Hkv, axis=1)
    dt = q.dtype.type
    scale = dt(1.0) / np.sqrt(dt(d))
    i = np.arange(s)
    allowed = i[None, :] <= i[:, None]                                 # [s(query), s(key)]
    out = np.empty_like(q)
    for bi in range(b):
        S = (q[bi] @ np.swapaxes(k[bi], -1, -2)) * scale              # [H, s, s]
        if slopes is not None:
            rel = (i[None, :] - i[:, None]).astype(dt)                 # j - i
            S = S + slopes.astype(dt)[:, None, None] * rel[None]
        ok = allowed if key_mask is None else allowed & np.asarray(key_mask[bi], bool)[None, :]
        S = np.where(ok[None], S, -np.inf)
        empty = ~ok.any(axis=-1)                                       # [s]: no key left
        S = S - np.where(empty[:, None], 0, S.max(axis=-1, keepdims=True))
        P = np.exp(S)                                                  # 0 on masked keys
        den = P.sum(axis=-1, keepdims=True)
        P = P / np.where(den > 0, den, 1)
        out[bi] = P @ v[bi]
    return out


# ------------------------------------------------------------------------------ the model


def _w(W, name, dt):
    a = W.get(name)
    return None if a is None else a.astype(dt)


def split_fused_qkv(w_fused, n_heads, head_dim):
    """De-interleave a per-head fused QKV tensor ([BLM] Contribution, item 3).

    Reading: the fused tensor has rows ordered (head a, c in {q, k, v}, dim e), i.e. it is
    a [H, 3, d, ...] view. Returns the q, k and v parts, each with rows ordered (a, e).
    Works for weights [3hd, h] and biases [3hd].
    """
    rest = w_fused.shape[1:]
    v = w_fused.reshape((n_heads, 3, head_dim) + rest)
    return tuple(v[:, c].reshape((n_heads * head_dim,) + rest) for c in range(3))


def qkv_weights(cfg, W, l, dt):
    p = f"layers.{l}."
    if cfg.qkv_layout == "fused":
        wq, wk, wv = split_fused_qkv(W[p + "qkv_fused_w"], cfg.n_heads, cfg.head_dim)
        if cfg.qkv_bias:
            bq, bk, bv = split_fused_qkv(W[p + "qkv_fused_b"], cfg.n_heads, cfg.head_dim)
        else:
            bq = bk = bv = None
    else:
        wq, wk, wv = W[p + "q_w"], W[p + "k_w"], W[p + "v_w"]
        bq, bk, bv = (W.get(p + "q_b"), W.get(p + "k_b"), W.get(p + "v_b"))
    conv = (lambda a: None if a is None else a.astype(dt))
    return tuple(conv(a) for a in (wq, wk, wv, bq, bk, bv))


def attention(cfg, W, l, z, dt, trace=None, key_mask=None):
    """Attention sublayer on the normed (pre-norm) or raw (post-norm) stream z [b, s, h]."""
    b, s, _ = z.shape
    H, d, Hkv = cfg.n_heads, cfg.head_dim, cfg.kv_heads
    wq, wk, wv, bq, bk, bv = qkv_weights(cfg, W, l, dt)
    # Biased projections; the bias is added before the rotary ([NNT] Notes, "Biased
    # queries, keys and values").
    q = z @ wq.T
    k = z @ wk.T
    v = z @ wv.T
    if bq is not None:
        q, k, v = q + bq, k + bk, v + bv
    if cfg.qk_norm == "full_rms":
        # RMSNorm over the whole Q / K projection row, not per head ([OLMO] Contribution).
        p = f"layers.{l}."
        q = rms_norm(q, _w(W, p + "q_norm_w", dt), dt(cfg.qk_norm_eps))
        k = rms_norm(k, _w(W, p + "k_norm_w", dt), dt(cfg.qk_norm_eps))
    # Head split: head a is projection columns [a*d, (a+1)*d) ([NNT] Notes, q_raw.view(b, s,
    # -1, head_dim).transpose(1, 2)); keys and values have H_kv heads.
    split = lambda t, n: t.reshape(b, s, n, d).transpose(0, 2, 1, 3)
    q, k, v = split(q, H), split(k, Hkv), split(v, Hkv)
    if cfg.qk_norm == "head_ln":
        # One LayerNorm without bias per query head and per key/value head, on the split
        # heads, before the rotary ([NNT] Notes, "Per-head LayerNorms on queries and keys
        # on 12B"); gains stored [heads * d], head a's at [a*d, (a+1)*d).
        p = f"layers.{l}."
        gq = _w(W, p + "q_norm_w", dt).reshape(1, H, 1, d)
        gk = _w(W, p + "k_norm_w", dt).reshape(1, Hkv, 1, d)
        q = layer_norm(q, gq, np.zeros(d, dt), dt(cfg.qk_norm_eps))
        k = layer_norm(k, gk, np.zeros(d, dt), dt(cfg.qk_norm_eps))
    pos = np.arange(s)           # positions from 0, no BOS ([NNT] The Notes, readout)
    q = apply_rope(q, pos, cfg.rot_dim, cfg.rope_theta)
    k = apply_rope(k, pos, cfg.rot_dim, cfg.rope_theta)
    slopes = alibi_slopes(H, dt) if cfg.alibi else None
    o = causal_attention(q, k, v, slopes, key_mask)                     # [b, H, s, d]
    premix = o.transpose(0, 2, 1, 3).reshape(b, s, H * d)              # attention_premix
    out = premix @ _w(W, f"layers.{l}.o_w", dt).T
    if cfg.o_bias:
        out = out + _w(W, f"layers.{l}.o_b", dt)
    if trace is not None:
        trace.update(attention_queries=q, attention_keys=k, attention_values=v,
                     attention_premix=premix, attention_output=out)
    return out


def mlp(cfg, W, l, z, dt, trace=None):
    """MLP sublayer: SwiGLU down(SiLU(gate z) * up z) ([NNT] Printout: gate/up/down without
    bias, act_fn SiLU), or GELU(fc1 z + b1) -> down (+ b2) for the Bloom-style variant."""
    p = f"layers.{l}."
    if cfg.mlp_kind == "swiglu":
        neurons = silu(z @ _w(W, p + "gate_w", dt).T) * (z @ _w(W, p + "up_w", dt).T)
    else:
        a = z @ _w(W, p + "fc1_w", dt).T
        if cfg.mlp_bias:
            a = a + _w(W, p + "fc1_b", dt)
        neurons = gelu_tanh(a)
    out = neurons @ _w(W, p + "down_w", dt).T
    if cfg.mlp_bias:
        out = out + _w(W, p + "down_b", dt)
    if trace is not None:
        trace.update(mlp_neurons=neurons, mlp_output=out)
    return out


def _norm(cfg, W, wname, bname, z, dt):
    if cfg.norm_kind == "layernorm":
        return layer_norm(z, _w(W, wname, dt), _w(W, bname, dt), dt(cfg.norm_eps))
    return rms_norm(z, _w(W, wname, dt), dt(cfg.norm_eps))


def block(cfg, W, l, x, dt, trace=None, key_mask=None):
    """One transformer block.

    pre-norm  ([NNT] Notes, sequential block):  h = x + attn(LN1(x)); out = h + mlp(LN2(h))
    parallel  ([NNT] Notes, 12B block):         n = LN1(x); out = x + attn(n) + mlp(n)
    post-norm ([OLMO] Contribution):            h = x + RMS(attn(x)); out = h + RMS(mlp(h))
    """
    p = f"layers.{l}."
    if cfg.parallel_residual:
        n = _norm(cfg, W, p + "attn_norm_w", p + "attn_norm_b", x, dt)
        a = attention(cfg, W, l, n, dt, trace, key_mask)
        f = mlp(cfg, W, l, n, dt, trace)
        h = x + a
        out = x + a + f
    elif cfg.norm_place == "pre":
        n = _norm(cfg, W, p + "attn_norm_w", p + "attn_norm_b", x, dt)
        a = attention(cfg, W, l, n, dt, trace, key_mask)
        h = x + a
        m = _norm(cfg, W, p + "mlp_norm_w", p + "mlp_norm_b", h, dt)
        f = mlp(cfg, W, l, m, dt, trace)
        out = h + f
    else:
        a = rms_norm(attention(cfg, W, l, x, dt, trace, key_mask), _w(W, p + "post_attn_norm_w", dt),
                     dt(cfg.norm_eps))
        h = x + a
        f = rms_norm(mlp(cfg, W, l, h, dt, trace), _w(W, p + "post_ff_norm_w", dt),
                     dt(cfg.norm_eps))
        out = h + f
    if trace is not None:
        trace.update(layer_input=x, layer_mid=h, block_attn=a, block_mlp=f, layer_output=out)
    return out


def embed(cfg, W, ids, dt):
    """Token embedding lookup ([NNT] The block: embed_tokens -> token_embeddings). With
    learned absolute positions ([BLM] Contribution: learned-absolute is one of the three
    positional paradigms), position p's learned row is added to the token row at p, for
    p = 0..s-1 in every batch row. Then the embedding LayerNorm when the config has one
    ([BLM] Contribution, item 2)."""
    x = W["embed"][ids].astype(dt)
    if cfg.learned_pos:
        s = ids.shape[1]
        x = x + W["pos_embed"][:s].astype(dt)[None, :, :]
    if cfg.embed_norm:
        x = layer_norm(x, _w(W, "embed_norm_w", dt), _w(W, "embed_norm_b", dt),
                       dt(cfg.norm_eps))
    return x


# ---------------------------------------------------------------------- Q8_0 weights
# The pages report q8 / int8 parity results without naming the scheme ([SLM] Results;
# [OLMO] 1. Contribution); the one quantised format they name is GGUF's Q8_0 ([RF], the
# model file it runs). Q8_0 splits a row into blocks of 32 consecutive values; a block
# stores d = max|x| / 127 as float16 and the codes q = round(x / d) as int8 (x times the
# float32 reciprocal of d, rounded half away from zero); a value decodes as q * d.

Q8_BLOCK = 32
Q8_MATRICES = ("q_w", "k_w", "v_w", "qkv_fused_w", "o_w", "gate_w", "up_w", "fc1_w", "down_w")


def quantize_q8_0(w):
    """w: float16 [rows, cols], cols a multiple of 32 -> (codes int8 [rows, cols],
    scales float16 [rows, cols / 32]). The block scale and the codes are decided in
    float32 (the decision that makes an integer is taken in one stated precision)."""
    w = np.asarray(w)
    rows, cols = w.shape
    assert cols % Q8_BLOCK == 0
    x = w.astype(np.float32).reshape(rows, cols // Q8_BLOCK, Q8_BLOCK)
    amax = np.abs(x).max(axis=-1)
    d = (amax / np.float32(127)).astype(np.float32)
    inv = np.zeros_like(d)
    nz = d != 0
    inv[nz] = np.float32(1) / d[nz]
    x0 = (x * inv[..., None]).astype(np.float32).astype(np.float64)   # exact from here
    q = np.where(x0 >= 0, np.floor(x0 + 0.5), np.ceil(x0 - 0.5))       # ties away from 0
    return q.astype(np.int8).reshape(rows, cols), d.astype(np.float16)


def dequantize_q8_0(q, d):
    """codes int8 [rows, cols], scales float16 [rows, cols / 32] -> float64 [rows, cols]."""
    rows, cols = q.shape
    v = q.astype(np.float64).reshape(rows, cols // Q8_BLOCK, Q8_BLOCK) * \
        d.astype(np.float64)[..., None]
    return v.reshape(rows, cols)


def q8_0_weights(cfg, W):
    """The weights the Q8_0 model computes with: every projection matrix (q/k/v or the
    fused QKV, o, gate/up or fc1, down) and the lm_head replaced by its decoded Q8_0
    values; embeddings, position rows, norms and biases unchanged."""
    out = dict(W)
    for name, a in W.items():
        base = name.split(".")[-1]
        if base in Q8_MATRICES or name == "lm_head":
            out[name] = dequantize_q8_0(*quantize_q8_0(a))
    return out


def forward(cfg, W, ids, dtype=np.float64, residuals=False, logit_positions=None,
            n_layers=None, attention_mask=None):
    """Full prefill forward. ids: int [b, s]. Returns logits [b, s, V] in `dtype`.

    After the last block: final norm (LayerNorm with bias, or RMSNorm for the post-norm
    variant), then the untied lm_head with no bias and nothing applied past it ([NNT]
    Printout and Notes, "The readout and the tokenizer").

    residuals=True also returns the residual stream after the embedding and after each
    block, a list of L+1 arrays [b, s, h]. logit_positions, if given, restricts the
    lm_head to those sequence positions (logits [b, len(positions), V]).

    attention_mask: optional int [b, s], zeros marking padding ([NNT] The API: the mask the
    model is called with, zeros are padding). Padding keys are excluded from every query's
    softmax; positions stay 0..s-1 in every row, as for an unpadded call (rotary and ALiBi
    scores depend only on position differences, so a row's left padding shifts nothing).
    Ids at padding positions must still be valid; their outputs are computed like any
    other position's (a padding query with no key left attends to nothing).
    """
    dt = np.dtype(dtype).type
    ids = np.asarray(ids)
    assert ids.ndim == 2
    if ids.size and (ids.min() < 0 or ids.max() >= cfg.vocab):
        raise ValueError("token id out of range")
    L = cfg.n_layers if n_layers is None else n_layers
    if getattr(cfg, "weight_format", "f16") == "q8_0":
        W = q8_0_weights(cfg, W)
    key_mask = None if attention_mask is None else np.asarray(attention_mask) != 0
    x = embed(cfg, W, ids, dt)
    res = [x.copy()] if residuals else None
    for l in range(L):
        x = block(cfg, W, l, x, dt, key_mask=key_mask)
        if residuals:
            res.append(x.copy())
    y = _norm(cfg, W, "final_norm_w", "final_norm_b", x, dt)
    if logit_positions is not None:
        y = y[:, np.asarray(logit_positions)]
    logits = y @ _w(W, "lm_head", dt).T
    return (logits, res) if residuals else logits


def next_token_probs(logits):
    """Next-token distribution at the last position: softmax over the vocabulary of
    logits[:, -1, :] ([NNT] The API: next_token_probs [batch vocab_size], derived from the
    logits at the last position). Max subtracted first. Returns [b, V]."""
    z = np.asarray(logits)[:, -1, :]
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)
