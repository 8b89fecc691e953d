"""Test-side emulation of the HIP path's fp16 storage, for error floors.

The library keeps the residual stream and every accumulation in fp32 but stores some
intermediates in fp16: the normed block inputs, the projected q, k and v (q already
multiplied by the exp2-domain score scale log2(e) / sqrt(d)), the softmax probabilities P
it multiplies with v, the attention output and the MLP activation. This module runs the
forward in float64 with exactly those roundings inserted (round to nearest even, as
`numpy.astype(float16)`), so its distance from the float64 oracle is the error that fp16
storage alone costs on a given input: the floor no kernel with that storage can beat.

The probabilities are rounded the way the attention kernel forms them: keys in tiles of
64, queries in groups of 32 (one wave), a running max per query that the whole group moves
only when some query's tile max exceeds it by more than 8 (log2 domain), and
P = fp16(2^(score - running max)); numerator and denominator take the same fp16 values.

Built from the oracle's primitives (norms, rotary, SiLU); nothing here is imported by the
library or by the oracle.
"""
from __future__ import annotations

import numpy as np

import oracle

KEY_TILE = 64
WAVE_QUERIES = 32
RESCALE_MARGIN = 8.0


def _h(a):
    """Round to fp16 (nearest even) and back to float64."""
    return np.asarray(a, np.float64).astype(np.float16).astype(np.float64)


def _w(W, name):
    a = W.get(name)
    return None if a is None else a.astype(np.float64)


def attention_fp16_p(q16, k16, v16, key_mask=None):
    """q16 [b, H, s, d] (log2-domain scale applied), k16 / v16 [b, Hkv, s, d], all
    fp16-valued float64. Returns the unrounded attention output [b, H, s, d]."""
    b, H, s, d = q16.shape
    Hkv = k16.shape[1]
    rep = H // Hkv
    out = np.zeros((b, H, s, d))
    for bi in range(b):
        for a in range(H):
            q, k, v = q16[bi, a], k16[bi, a // rep], v16[bi, a // rep]
            t_all = q @ k.T                                       # [s, s], log2 domain
            for q0 in range(0, s, WAVE_QUERIES):
                qs = np.arange(q0, min(q0 + WAVE_QUERIES, s))
                m = np.full(len(qs), -np.inf)
                lsum = np.zeros(len(qs))
                acc = np.zeros((len(qs), d))
                last_key = qs[-1]
                for k0 in range(0, last_key + 1, KEY_TILE):
                    keys = np.arange(k0, min(k0 + KEY_TILE, s))
                    t = t_all[np.ix_(qs, keys)]
                    ok = keys[None, :] <= qs[:, None]
                    if key_mask is not None:
                        ok = ok & np.asarray(key_mask[bi], bool)[keys][None, :]
                    t = np.where(ok, t, -np.inf)
                    mx = t.max(axis=1)
                    if np.any(mx > m + RESCALE_MARGIN):
                        mnew = np.maximum(m, mx)
                        with np.errstate(invalid="ignore"):
                            alpha = np.where(mnew == -np.inf, 1.0, np.exp2(m - mnew))
                        lsum *= alpha
                        acc *= alpha[:, None]
                        m = mnew
                    muse = np.where(m == -np.inf, 0.0, m)
                    p = _h(np.exp2(t - muse[:, None]))            # 0 on masked keys
                    lsum += p.sum(axis=1)
                    acc += p @ v[keys]
                inv = np.where(lsum > 0, 1.0 / np.where(lsum > 0, lsum, 1.0), 0.0)
                out[bi, a, qs] = acc * inv[:, None]
    return out


def forward(cfg, W, ids, attention_mask=None):
    """The forward with the library's fp16 storage points; returns (logits [b, s, V],
    residuals: list of L+1 arrays [b, s, h]), like oracle.forward(..., residuals=True)."""
    assert cfg.mlp_kind == "swiglu" and not cfg.alibi and not cfg.parallel_residual
    assert not cfg.learned_pos and not cfg.embed_norm and cfg.qkv_layout == "separate"
    assert cfg.qk_norm in ("none", "full_rms")
    assert getattr(cfg, "weight_format", "f16") == "f16"
    H, d, Hkv = cfg.n_heads, cfg.head_dim, cfg.kv_heads
    ids = np.asarray(ids)
    b, s = ids.shape
    pre = cfg.norm_place == "pre"
    eps = cfg.norm_eps
    scale = np.log2(np.e) / np.sqrt(d)
    key_mask = None if attention_mask is None else np.asarray(attention_mask) != 0

    def norm(z, wn, bn):
        if cfg.norm_kind == "layernorm":
            return oracle.layer_norm(z, _w(W, wn), _w(W, bn), eps)
        return oracle.rms_norm(z, _w(W, wn), eps)

    def attn(z16, p):
        q = z16 @ _w(W, p + "q_w").T
        k = z16 @ _w(W, p + "k_w").T
        v = z16 @ _w(W, p + "v_w").T
        if cfg.qkv_bias:
            q, k, v = q + _w(W, p + "q_b"), k + _w(W, p + "k_b"), v + _w(W, p + "v_b")
        if cfg.qk_norm == "full_rms":
            q = oracle.rms_norm(q, _w(W, p + "q_norm_w"), cfg.qk_norm_eps)
            k = oracle.rms_norm(k, _w(W, p + "k_norm_w"), cfg.qk_norm_eps)
        split = lambda t, n: t.reshape(b, s, n, d).transpose(0, 2, 1, 3)
        q, k, v = split(q, H), split(k, Hkv), split(v, Hkv)
        pos = np.arange(s)
        q = oracle.apply_rope(q, pos, cfg.rot_dim, cfg.rope_theta)
        k = oracle.apply_rope(k, pos, cfg.rot_dim, cfg.rope_theta)
        o = attention_fp16_p(_h(q * scale), _h(k), _h(v), key_mask)
        o16 = _h(o.transpose(0, 2, 1, 3).reshape(b, s, H * d))
        return o16 @ _w(W, p + "o_w").T

    def mlp(z16, p):
        g = z16 @ _w(W, p + "gate_w").T
        u = z16 @ _w(W, p + "up_w").T
        return _h(oracle.silu(g) * u) @ _w(W, p + "down_w").T

    x = W["embed"][ids].astype(np.float64)
    res = [x.copy()]
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        if pre:
            h = x + attn(_h(norm(x, p + "attn_norm_w", p + "attn_norm_b")), p)
            x = h + mlp(_h(norm(h, p + "mlp_norm_w", p + "mlp_norm_b")), p)
        else:
            h = x + oracle.rms_norm(attn(_h(x), p), _w(W, p + "post_attn_norm_w"), eps)
            x = h + oracle.rms_norm(mlp(_h(h), p), _w(W, p + "post_ff_norm_w"), eps)
        res.append(x.copy())
    y16 = _h(norm(x, "final_norm_w", "final_norm_b"))
    return y16 @ _w(W, "lm_head").T, res
