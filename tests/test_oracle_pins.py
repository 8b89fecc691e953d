"""Pins of the oracle's primitives against facts that do not come from the oracle itself:
closed forms, invariants, brute force on tiny inputs, library routines and fixtures
holding values the pages fix. Each test names the mistake it is meant to catch.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------------------ LayerNorm

def test_layer_norm_moments_before_affine():
    """With w = 1, b = 0 the output rows have mean 0 and variance var/(var+eps) (eps
    inside the root; population variance). Catches eps outside the root, n-1 variance."""
    z = _rng().normal(0.3, 0.05, size=(7, 2048))
    eps = 1e-5
    y = oracle.layer_norm(z, np.ones(2048), np.zeros(2048), eps)
    var = z.var(axis=-1)
    assert np.abs(y.mean(axis=-1)).max() < 1e-12
    np.testing.assert_allclose(y.var(axis=-1), var / (var + eps), rtol=1e-12)
    # eps = 0: exactly unit variance
    y0 = oracle.layer_norm(z, np.ones(2048), np.zeros(2048), 0.0)
    np.testing.assert_allclose(y0.var(axis=-1), 1.0, rtol=1e-12)


def test_layer_norm_matches_torch_float64():
    r = _rng(1)
    z, w, b = r.normal(size=(5, 256)), r.normal(1, 0.1, 256), r.normal(0, 0.1, 256)
    ref = F.layer_norm(torch.from_numpy(z), (256,), torch.from_numpy(w), torch.from_numpy(b),
                       1e-5).numpy()
    np.testing.assert_allclose(oracle.layer_norm(z, w, b, 1e-5), ref, rtol=0, atol=1e-12)


def test_layer_norm_gain_and_bias_roles():
    """Gain scales and bias shifts the normalised row (catches swapped gain/bias)."""
    z = _rng(2).normal(size=(3, 64))
    base = oracle.layer_norm(z, np.ones(64), np.zeros(64), 1e-5)
    w = np.full(64, 2.0)
    b = np.full(64, 0.5)
    np.testing.assert_allclose(oracle.layer_norm(z, w, b, 1e-5), 2.0 * base + 0.5, atol=1e-12)


# -------------------------------------------------------------------------------- RMSNorm

def test_rms_norm_mean_square_and_torch():
    r = _rng(3)
    z = r.normal(0.2, 1.5, size=(6, 512))
    eps = 1e-6
    y = oracle.rms_norm(z, np.ones(512), eps)
    ms = (z * z).mean(-1)
    np.testing.assert_allclose((y * y).mean(-1), ms / (ms + eps), rtol=1e-12)
    w = r.normal(1, 0.1, 512)
    ref = F.rms_norm(torch.from_numpy(z), (512,), torch.from_numpy(w), eps).numpy()
    np.testing.assert_allclose(oracle.rms_norm(z, w, eps), ref, atol=1e-12)
    # RMSNorm does not subtract the mean: a constant row maps to sign * w
    c = np.full((1, 8), 3.0)
    np.testing.assert_allclose(oracle.rms_norm(c, np.ones(8), 0.0), np.ones((1, 8)), atol=1e-15)


# ----------------------------------------------------------------------------------- RoPE

def test_rope_pass_through_dims_bitwise():
    """Dims past the rotary span are the projection output unchanged (the StableLM page
    checks torch.equal(q_pre[..., 16:], q[..., 16:]))."""
    u = _rng(4).normal(size=(2, 3, 40, 64))
    out = oracle.apply_rope(u, np.arange(40), 16, 10000.0)
    assert np.array_equal(out[..., 16:], u[..., 16:])
    assert not np.array_equal(out[..., :16], u[..., :16])


def test_rope_position_zero_is_identity_and_pair_norms_preserved():
    u = _rng(5).normal(size=(1, 2, 50, 64))
    out = oracle.apply_rope(u, np.arange(50), 16, 10000.0)
    assert np.array_equal(out[..., 0, :], u[..., 0, :])
    for i in range(8):
        n0 = u[..., i] ** 2 + u[..., i + 8] ** 2
        n1 = out[..., i] ** 2 + out[..., i + 8] ** 2
        np.testing.assert_allclose(n1, n0, rtol=1e-12)


def test_rope_closed_form_angles_and_sign():
    """Pair (0, 8) has frequency theta^0 = 1: at position p the unit vector e_0 turns by p
    radians towards e_8, i.e. (cos p, sin p); e_8 turns to (-sin p, cos p). The last pair
    (7, 15) has frequency theta^(-14/16) for a 16-dim span. Catches the rotation sign, the
    pairing (i, i+8) vs (2i, 2i+1) and the frequency denominator (16, not 64)."""
    s, d, r, theta = 9, 64, 16, 10000.0
    pos = np.arange(s)
    e0 = np.zeros((s, d)); e0[:, 0] = 1.0
    out = oracle.apply_rope(e0, pos, r, theta)
    np.testing.assert_allclose(out[:, 0], np.cos(pos), atol=1e-15)
    np.testing.assert_allclose(out[:, 8], np.sin(pos), atol=1e-15)
    assert np.abs(np.delete(out, [0, 8], axis=1)).max() == 0.0
    e8 = np.zeros((s, d)); e8[:, 8] = 1.0
    out = oracle.apply_rope(e8, pos, r, theta)
    np.testing.assert_allclose(out[:, 0], -np.sin(pos), atol=1e-15)
    np.testing.assert_allclose(out[:, 8], np.cos(pos), atol=1e-15)
    e7 = np.zeros((s, d)); e7[:, 7] = 1.0
    out = oracle.apply_rope(e7, pos, r, theta)
    f7 = 10000.0 ** (-14.0 / 16.0)
    np.testing.assert_allclose(out[:, 7], np.cos(pos * f7), atol=1e-15)
    np.testing.assert_allclose(out[:, 15], np.sin(pos * f7), atol=1e-15)


def test_rope_equals_complex_rotation():
    """Textbook form: with z_i = u_i + i*u_{i+r/2}, the rotation is z_i * exp(i p f_i)."""
    r, theta = 16, 10000.0
    u = _rng(6).normal(size=(30, 64))
    pos = np.arange(30)
    out = oracle.apply_rope(u, pos, r, theta)
    z = u[:, :8] + 1j * u[:, 8:16]
    f = np.array([theta ** (-2.0 * i / r) for i in range(8)])
    zr = z * np.exp(1j * pos[:, None] * f[None, :])
    np.testing.assert_allclose(out[:, :8], zr.real, atol=1e-13)
    np.testing.assert_allclose(out[:, 8:16], zr.imag, atol=1e-13)


def test_rope_angles_exact_in_float32():
    """The rotary angle is formed in float64 whatever the working dtype, and cos / sin are
    rounded once: at the longest OLMo-2-shaped position (p = 4095, theta = 5e5, the whole
    128-dim head rotated) the float32 oracle's factors equal the float64 values rounded to
    float32 bit for bit. A float32 angle p * f_i would be off by up to ~2e-4 rad there and
    move many of them. Unit vectors read the factors out exactly (1 * c - 0 * s = c)."""
    import math
    r, theta, half = 128, 500000.0, 64
    pos = np.array([1, 977, 2048, 4094, 4095])
    for i in (0, 1, 17, 40, 63):
        e = np.zeros((len(pos), r), np.float32)
        e[:, i] = 1.0
        out = oracle.apply_rope(e, pos, r, theta)
        assert out.dtype == np.float32
        f = theta ** (-2.0 * i / r)
        want_c = np.array([math.cos(p * f) for p in pos]).astype(np.float32)
        want_s = np.array([math.sin(p * f) for p in pos]).astype(np.float32)
        assert np.array_equal(out[:, i].view(np.uint32), want_c.view(np.uint32)), i
        assert np.array_equal(out[:, i + half].view(np.uint32), want_s.view(np.uint32)), i


def test_rope_relative_position_property():
    """<R_p a, R_t b> depends only on p - t."""
    r = _rng(7)
    a, b = r.normal(size=64), r.normal(size=64)
    def rot(v, p):
        return oracle.apply_rope(v[None, :], np.array([p]), 64, 500000.0)[0]
    for p, t, delta in [(3, 1, 5), (100, 40, 900), (7, 7, 4000)]:
        lhs = rot(a, p) @ rot(b, t)
        rhs = rot(a, p + delta) @ rot(b, t + delta)
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(lhs))


# --------------------------------------------------------------------------------- ALiBi

def test_alibi_slopes_match_fixture():
    vals = [float(x) for x in open(os.path.join(GOLDEN, "alibi_slopes_h16.txt"))
            if x.strip() and not x.startswith("#")]
    np.testing.assert_allclose(oracle.alibi_slopes(16), vals, rtol=1e-15)


def test_alibi_slopes_geometric():
    for H in (4, 8, 16, 32):
        m = oracle.alibi_slopes(H)
        np.testing.assert_allclose(m[1:] / m[:-1], 2.0 ** (-8.0 / H), rtol=1e-14)
        assert m[-1] == 2.0 ** -8          # last head always 1/256
        assert m[0] == 2.0 ** (-8.0 / H)   # first slope is the ratio itself, not 1


# ------------------------------------------------------------------------------ attention

def _attention_brute(q, k, v, slopes=None, key_mask=None):
    """Triple loop in plain Python floats; keys with key_mask False are skipped and a query
    with no key left keeps a zero output."""
    b, H, s, d = q.shape
    out = np.zeros_like(q)
    for bi, a, i in itertools.product(range(b), range(H), range(s)):
        keys = [j for j in range(i + 1) if key_mask is None or key_mask[bi][j]]
        if not keys:
            continue
        sc = []
        for j in keys:
            t = sum(q[bi, a, i, e] * k[bi, a, j, e] for e in range(d)) / math.sqrt(d)
            if slopes is not None:
                t += slopes[a] * (j - i)
            sc.append(t)
        mx = max(sc)
        w = [math.exp(t - mx) for t in sc]
        tot = sum(w)
        for e in range(d):
            out[bi, a, i, e] = sum(wj * v[bi, a, j, e] for wj, j in zip(w, keys)) / tot
    return out


@pytest.mark.parametrize("d", [4, 8])
@pytest.mark.parametrize("alibi", [False, True])
def test_attention_brute_force(d, alibi):
    r = _rng(8 + d)
    q, k, v = (r.normal(size=(2, 2, 7, d)) for _ in range(3))
    slopes = oracle.alibi_slopes(2) if alibi else None
    np.testing.assert_allclose(oracle.causal_attention(q, k, v, slopes),
                               _attention_brute(q, k, v, slopes), atol=1e-13)


@pytest.mark.parametrize("alibi", [False, True])
def test_attention_key_mask_brute_force(alibi):
    """Padding keys: left padding (a row's first positions), right padding, a hole in the
    middle and no padding, against the triple loop."""
    r = _rng(30)
    q, k, v = (r.normal(size=(4, 2, 7, 4)) for _ in range(3))
    mask = np.array([[0, 0, 1, 1, 1, 1, 1], [1, 1, 1, 1, 0, 0, 0], [1, 1, 0, 1, 1, 0, 1],
                     [1, 1, 1, 1, 1, 1, 1]], dtype=bool)
    slopes = oracle.alibi_slopes(2) if alibi else None
    got = oracle.causal_attention(q, k, v, slopes, mask)
    np.testing.assert_allclose(got, _attention_brute(q, k, v, slopes, mask), atol=1e-13)
    assert np.all(got[0, :, :2] == 0)           # padding queries with no key left
    np.testing.assert_allclose(got[3], oracle.causal_attention(q, k, v, slopes)[3], atol=0)


def test_attention_key_mask_matches_torch_sdpa():
    """Boolean SDPA mask = causal AND key kept, on every query row with a key left."""
    r = _rng(31)
    b, s = 3, 29
    q, k, v = (r.normal(size=(b, 2, s, 8)) for _ in range(3))
    mask = r.random((b, s)) > 0.3
    mask[:, 0] = True                           # every query keeps at least key 0
    i = np.arange(s)
    allowed = (i[None, :] <= i[:, None])[None, None] & mask[:, None, None, :]
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(t) for t in (q, k, v)),
                                         attn_mask=torch.from_numpy(allowed)).numpy()
    np.testing.assert_allclose(oracle.causal_attention(q, k, v, None, mask), ref, atol=1e-12)


def test_attention_right_padding_is_a_prefix():
    """A row padded on the right gives, at its real positions, exactly the unpadded
    shorter row's outputs (causality: real queries never see the padding after them)."""
    r = _rng(32)
    q, k, v = (r.normal(size=(1, 2, 9, 8)) for _ in range(3))
    mask = np.array([[1] * 6 + [0] * 3], dtype=bool)
    full = oracle.causal_attention(q, k, v, None, mask)
    short = oracle.causal_attention(q[:, :, :6], k[:, :, :6], v[:, :, :6])
    np.testing.assert_allclose(full[:, :, :6], short, atol=1e-15)


def test_next_token_probs():
    r = _rng(33)
    logits = r.normal(size=(3, 5, 40)) * 10
    p = oracle.next_token_probs(logits)
    assert p.shape == (3, 40)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-14)
    np.testing.assert_allclose(p, torch.softmax(torch.from_numpy(logits[:, -1]), -1).numpy(),
                               atol=1e-15)
    assert np.array_equal(p.argmax(-1), logits[:, -1].argmax(-1))
    # shift invariance and a closed form: two logits apart by log 3 give odds 3:1
    np.testing.assert_allclose(oracle.next_token_probs(logits + 1000.0), p, atol=1e-12)
    two = np.array([[[0.0, math.log(3.0)]]])
    np.testing.assert_allclose(oracle.next_token_probs(two), [[0.25, 0.75]], atol=1e-15)


def test_attention_matches_torch_sdpa():
    r = _rng(11)
    q, k, v = (r.normal(size=(2, 3, 33, 16)) for _ in range(3))
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(t) for t in (q, k, v)),
                                         is_causal=True).numpy()
    np.testing.assert_allclose(oracle.causal_attention(q, k, v), ref, atol=1e-12)
    # ALiBi as an additive mask
    s = 33
    m = oracle.alibi_slopes(3)
    i = np.arange(s)
    bias = m[:, None, None] * (i[None, :] - i[:, None])[None]
    bias = np.where(i[None, :] <= i[:, None], bias, -np.inf)
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(t) for t in (q, k, v)),
                                         attn_mask=torch.from_numpy(bias)).numpy()
    np.testing.assert_allclose(oracle.causal_attention(q, k, v, m), ref, atol=1e-12)


def test_attention_closed_forms():
    """Row 0 attends only to key 0; with K = 0 all visible scores tie, so row i is the
    mean of V_0..V_i; with ALiBi and K = 0 the weights are proportional to e^{m (j - i)}."""
    r = _rng(12)
    s, d = 10, 8
    q, v = r.normal(size=(1, 2, s, d)), r.normal(size=(1, 2, s, d))
    k = r.normal(size=(1, 2, s, d))
    out = oracle.causal_attention(q, k, v)
    np.testing.assert_allclose(out[:, :, 0], v[:, :, 0], atol=1e-15)
    k0 = np.zeros_like(k)
    out = oracle.causal_attention(q, k0, v)
    cum = np.cumsum(v, axis=2) / np.arange(1, s + 1)[None, None, :, None]
    np.testing.assert_allclose(out, cum, atol=1e-13)
    m = oracle.alibi_slopes(2)
    out = oracle.causal_attention(q, k0, v, m)
    for a in range(2):
        for i in range(s):
            w = np.exp(m[a] * (np.arange(i + 1) - i))
            np.testing.assert_allclose(out[0, a, i], (w / w.sum()) @ v[0, a, :i + 1],
                                       atol=1e-13)


def test_alibi_shift_invariance():
    """Bias m(j - i) and bias m*j give the same softmax (row shift invariance)."""
    r = _rng(13)
    q, k, v = (r.normal(size=(1, 4, 12, 8)) for _ in range(3))
    m = oracle.alibi_slopes(4)
    out = oracle.causal_attention(q, k, v, m)
    s = 12
    i = np.arange(s)
    S = (q[0] @ np.swapaxes(k[0], -1, -2)) / math.sqrt(8) + m[:, None, None] * i[None, None, :]
    S = np.where(i[None, :] <= i[:, None], S, -np.inf)
    P = np.exp(S - S.max(-1, keepdims=True))
    P /= P.sum(-1, keepdims=True)
    np.testing.assert_allclose(out[0], P @ v[0], atol=1e-13)


# ----------------------------------------------------------------------------- activations

def test_activations_against_torch():
    z = np.linspace(-8, 8, 1001)
    np.testing.assert_allclose(oracle.silu(z), F.silu(torch.from_numpy(z)).numpy(), atol=1e-14)
    np.testing.assert_allclose(oracle.gelu_tanh(z),
                               F.gelu(torch.from_numpy(z), approximate="tanh").numpy(),
                               atol=1e-14)
    assert oracle.silu(np.zeros(1))[0] == 0.0 and oracle.gelu_tanh(np.zeros(1))[0] == 0.0
    # tanh-GELU is not erf-GELU: they differ visibly somewhere in [-8, 8]
    erf = F.gelu(torch.from_numpy(z)).numpy()
    assert np.abs(oracle.gelu_tanh(z) - erf).max() > 1e-4


# --------------------------------------------------------------------- fused QKV de-interleave

def test_split_fused_qkv_against_explicit_interleave():
    """Build the fused tensor row by row from known q/k/v weights in the per-head
    interleaved order (head a: q rows, then k rows, then v rows) and check the split
    recovers them; the naive [Q; K; V] block reading does not."""
    H, d, h = 3, 4, 5
    r = _rng(14)
    parts = [r.normal(size=(H * d, h)) for _ in range(3)]
    fused = np.zeros((3 * H * d, h))
    row = 0
    for a in range(H):
        for c in range(3):
            for e in range(d):
                fused[row] = parts[c][a * d + e]
                row += 1
    got = oracle.split_fused_qkv(fused, H, d)
    for c in range(3):
        assert np.array_equal(got[c], parts[c])
    blocks = np.split(fused, 3)
    assert not np.array_equal(blocks[0], parts[0])
    bias = fused[:, 0]
    gb = oracle.split_fused_qkv(bias, H, d)
    for c in range(3):
        assert np.array_equal(gb[c], parts[c][:, 0])


# ----------------------------------------------------------------------------- Q8_0

def test_q8_0_integer_blocks_are_exact():
    """A block of integers whose largest magnitude is 127 has scale 1 and codes equal to
    the integers; scaled by a power of two, the scale scales and the codes stay."""
    r = _rng(40)
    ints = r.integers(-127, 128, size=(3, 64)).astype(np.float64)
    ints[:, 0], ints[:, 32] = 127, -127                    # each block reaches 127
    for e in (0, -10, -6):
        w = (ints * 2.0 ** e).astype(np.float16)
        q, d = oracle.quantize_q8_0(w)
        assert np.array_equal(q, ints.astype(np.int8))
        assert np.all(d == np.float16(2.0 ** e))
        np.testing.assert_array_equal(oracle.dequantize_q8_0(q, d), w.astype(np.float64))


def test_q8_0_rounds_half_away_from_zero():
    w = np.zeros((1, 32), np.float16)
    w[0, :7] = [127, 2.5, -2.5, 0.5, -0.5, 1.5, -126.5]
    q, d = oracle.quantize_q8_0(w)
    assert d[0, 0] == 1
    assert list(q[0, :7]) == [127, 3, -3, 1, -1, 2, -127]


def test_q8_0_zero_block_and_sign_symmetry():
    r = _rng(41)
    w = (r.normal(size=(5, 96)) * 0.02).astype(np.float16)
    w[2, 32:64] = 0
    q, d = oracle.quantize_q8_0(w)
    assert d[2, 1] == 0 and not q[2, 32:64].any()
    qn, dn = oracle.quantize_q8_0(-w)
    assert np.array_equal(qn, -q) and np.array_equal(dn, d)


def test_q8_0_error_bound_and_range():
    """Every code lies in [-127, 127], every nonzero block uses +-127, and the decoded
    value is within d/2 plus the float16 rounding of the scale (127 |d - d16|)."""
    r = _rng(42)
    w = (r.normal(size=(64, 256)) * 0.02).astype(np.float16)
    q, d = oracle.quantize_q8_0(w)
    assert np.abs(q.astype(int)).max() <= 127
    assert np.all(np.abs(q.reshape(64, 8, 32).astype(int)).max(-1) == 127)
    err = np.abs(oracle.dequantize_q8_0(q, d) - w.astype(np.float64)).reshape(64, 8, 32).max(-1)
    d32 = np.abs(w.astype(np.float32)).reshape(64, 8, 32).max(-1) / np.float32(127)
    bound = 0.5 * d32 + 127 * np.abs(d32.astype(np.float64) - d.astype(np.float64))
    assert np.all(err <= bound * (1 + 1e-6))


def test_q8_0_model_weights_and_effect():
    """Only the projection matrices and the lm_head are replaced; the Q8_0 model's logits
    stay close to the float16 model's but are not equal."""
    from workloads import ModelConfig, synth_ids, synth_weights
    cfg = ModelConfig(name="tiny_q8", n_layers=2, hidden=256, n_heads=4, head_dim=64,
                      inter=704, vocab=512, batch=2, seq=16, seed=43)
    W = synth_weights(cfg)
    Wq = oracle.q8_0_weights(cfg, W)
    for k in W:
        base = k.split(".")[-1]
        changed = not np.array_equal(np.asarray(Wq[k], np.float64), W[k].astype(np.float64))
        assert changed == (base in oracle.Q8_MATRICES or k == "lm_head"), k
    ids = synth_ids(cfg)
    a = oracle.forward(cfg, W, ids)
    b = oracle.forward(cfg.with_(weight_format="q8_0"), W, ids)
    cos = (a * b).sum(-1) / np.linalg.norm(a, axis=-1) / np.linalg.norm(b, axis=-1)
    assert 0.99 < cos.min() and cos.min() < 1 - 1e-9
