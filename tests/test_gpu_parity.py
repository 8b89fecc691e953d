"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded
synthetic weights and ids.

Gates (per position): logit cosine >= 0.99999, argmax agreement wherever the oracle's
top-2 margin exceeds 1e-2, per-layer residual row-normwise max relative error <= 5e-3.
Small cases run the oracle in float64 on the whole batch; the full-size workloads run on
the GPU in the same launch configuration the benchmark times and are checked on sampled
batch rows and prefixes (causality makes a prefix of a row an exact sub-problem), with
the oracle in float32.
"""
import numpy as np
import pytest
import torch

import oracle

from workloads import CONFIGS, ModelConfig, synth_ids, synth_weights

from . import gpu_util as U

pytestmark = pytest.mark.gpu

# Small models spanning several GEMM / attention tiles with ragged tails.
RAGGED_SLM = ModelConfig(name="ragged_slm", n_layers=2, hidden=512, n_heads=8, head_dim=64,
                         inter=1408, vocab=1000, batch=3, seq=77, seed=21)
RAGGED_BLOOM = ModelConfig(name="ragged_bloom", n_layers=2, hidden=512, n_heads=8,
                           head_dim=64, inter=2048, vocab=777, batch=2, seq=150, rot_dim=0,
                           alibi=True, embed_norm=True, qkv_layout="fused", qkv_bias=True,
                           o_bias=True, mlp_bias=True, mlp_kind="gelu_tanh", seed=22)
RAGGED_OLMO = ModelConfig(name="ragged_olmo", n_layers=2, hidden=512, n_heads=4, head_dim=128,
                          inter=1024, vocab=900, batch=2, seq=131, norm_kind="rms",
                          norm_place="post", rot_dim=128, rope_theta=500000.0,
                          qk_norm="full_rms", qkv_bias=False, norm_eps=1e-6,
                          qk_norm_eps=1e-6, seed=23)
# StableLM-2-12B's block at small sizes: parallel residual, per-head Q/K LayerNorm, 2 key/value
# heads for 8 query heads (the K | V boundary, 640, is not a multiple of the GEMM tile).
RAGGED_SLM12 = RAGGED_SLM.with_(name="ragged_slm12_block", qkv_bias=False, n_kv_heads=2,
                                parallel_residual=True, qk_norm="head_ln", qk_norm_eps=1e-5,
                                seed=24)
# Learned absolute positions on a GPT-2-like block (LayerNorm, biases, tanh-GELU MLP).
RAGGED_POS = ModelConfig(name="ragged_learned_pos", n_layers=2, hidden=512, n_heads=8,
                         head_dim=64, inter=2048, vocab=1111, batch=3, seq=100, max_seq=128,
                         rot_dim=0, learned_pos=True, qkv_bias=True, o_bias=True,
                         mlp_bias=True, mlp_kind="gelu_tanh", seed=25)


def _parity_full(cfg, dtype=np.float64, tag=None, mask=None):
    W, ids = synth_weights(cfg), synth_ids(cfg)
    model = U.get_model(cfg, W)
    g, gres = U.run_gpu(model, ids, dump=True, mask=mask)
    r, rres = U.oracle_run(cfg, W, ids, dtype=dtype, mask=mask)
    return U.assert_parity(g.cpu().numpy(), r, gres.cpu().numpy(), np.stack(rres),
                           tag=tag or cfg.name)


def _pad_masks(b, s, seed):
    """Row 0 left-padded past the first 64-key tile, row 1 right-padded, row 2 with random
    holes, further rows alternating fully padded and unpadded."""
    r = np.random.default_rng(seed)
    m = np.ones((b, s), np.int32)
    m[0, :min(s - 1, 70)] = 0
    if b > 1:
        m[1, s - s // 4:] = 0
    if b > 2:
        m[2] = (r.random(s) > 0.3).astype(np.int32)
    for i in range(3, b):
        m[i] = 0 if i % 2 else 1
    return m


def test_c0_tiny_parity():
    _parity_full(CONFIGS["c0_tiny"])


@pytest.mark.parametrize("cfg", [RAGGED_SLM, RAGGED_BLOOM, RAGGED_OLMO], ids=lambda c: c.name)
def test_ragged_small_models(cfg):
    _parity_full(cfg)


# Five 2048-token rows with an MLP width of 5696: the down projection (K = 5696, 89 k-tiles
# of 64) runs 320 256x256 tiles on the persistent grid, so each CU moves on to a next tile
# after an odd k-tile count (the next tile's first k-tile then comes from the epilogue, not
# from the last refill slots as with the even counts of the other workloads); the gate/up
# GEMM (N = 11392 = 44.5 x 256) ends in a half-filled column tile.
BIG_ODD_K = ModelConfig(name="big_tiles_odd_k", n_layers=1, hidden=2048, n_heads=32,
                        head_dim=64, inter=5696, vocab=640, batch=5, seq=2048, seed=26)


def test_big_tiles_odd_k_tiles_and_ragged_columns():
    _parity_full(BIG_ODD_K, dtype=np.float32)


# The small models above have at most one 8-wave query block per CU, so their attention
# splits each query's key range between two halves of the block's waves; larger launches
# keep the unsplit schedule. Bloom-style (ALiBi) at 4 x 2100 (288 query blocks of 256)
# takes the unsplit one, with and without padding keys.
UNSPLIT_BLOOM = RAGGED_BLOOM.with_(name="unsplit_bloom", n_layers=1, batch=4, seq=2100,
                                   seed=90)


@pytest.mark.parametrize("padded", [False, True], ids=["plain", "padded"])
def test_unsplit_attention_alibi(padded):
    cfg = UNSPLIT_BLOOM
    mask = _pad_masks(cfg.batch, cfg.seq, 91) if padded else None
    _parity_full(cfg, mask=mask, tag=cfg.name + (" padded" if padded else ""))


@pytest.mark.parametrize("rot", [2, 4, 8, 16, 32, 64])
def test_rotary_spans(rot):
    """Every rotary span the fused QKV epilogue supports. In its transposed accumulator
    layout the partner of a rotated element is another register of the same lane (half 1,
    2, 8, 16), the same register of lane ^ 32 (half 4) or the neighbouring 32-column block
    (half 32, the whole 64-dim head)."""
    _parity_full(RAGGED_SLM.with_(rot_dim=rot, seed=30 + rot), tag=f"rot{rot}")


def test_rotary_partial_head128():
    """64 rotated dims of a 128-dim head: the blocks at head dims 64..127 pass unrotated."""
    _parity_full(RAGGED_SLM.with_(n_heads=4, head_dim=128, rot_dim=64, seed=37),
                 tag="rot64 hd128")


def test_qk_norm_with_partial_rotary():
    _parity_full(RAGGED_OLMO.with_(rot_dim=64, seed=31), tag="olmo rot64")


@pytest.mark.parametrize("rot,kv,hidden,heads", [
    (16, 0, 512, 4),     # whole-row path, rotary partner 2 lanes away
    (32, 0, 512, 4),     # whole-row path, partner 4 lanes away
    (64, 4, 1536, 12),   # whole-row path with grouped key/value heads (12 query, 4 kv)
    (64, 2, 512, 4),     # grouped heads, Q | K row of 768: two-read four-column path
    (128, 0, 768, 6),    # Q | K row of 1536: two-read four-column path
    (4, 0, 512, 4),      # rotary half-span 2: one column per thread
], ids=lambda v: str(v))
def test_qk_rms_norm_paths(rot, kv, hidden, heads):
    """Each path of the whole-row QK RMSNorm kernel: rows held in registers with the rotary
    partner taken by lane exchange (partner distances 2, 4 and grouped heads), the
    two-read path for rows that do not split into whole register groups, and the
    one-column path for rotary spans that are not a multiple of 8."""
    cfg = RAGGED_OLMO.with_(rot_dim=rot, n_kv_heads=kv, hidden=hidden, n_heads=heads,
                            seed=100 + rot + kv)
    _parity_full(cfg, tag=f"qk-rms rot{rot} kv{kv} h{hidden}")


def test_stablelm12_block_small():
    _parity_full(RAGGED_SLM12)


@pytest.mark.parametrize("kv", [1, 2, 4])
def test_grouped_kv_heads_fused_rope(kv):
    """Grouped key/value heads through the fused QKV rotary epilogue (no QK norm): the rotated
    columns end at (H + Hkv) d, inside a 256-column tile for kv 1 and 2."""
    _parity_full(RAGGED_SLM.with_(n_kv_heads=kv, seed=40 + kv), tag=f"kv{kv}")


def test_parallel_residual_layernorm_block():
    """Parallel block alone (one kv head per query head, no QK norm)."""
    _parity_full(RAGGED_SLM.with_(parallel_residual=True, seed=45), tag="parallel")


@pytest.mark.parametrize("rot", [0, 32, 64])
def test_head_layernorm_fused_rotary_spans(rot):
    """Per-head Q/K LayerNorm over 64-dim heads runs in the QKV GEMM epilogue; each rotary
    span it takes (none, half 16, half 32 = the whole head) against the oracle."""
    _parity_full(RAGGED_SLM12.with_(rot_dim=rot, seed=60 + rot), tag=f"head_ln rot{rot}")


def test_head_layernorm_head128_gqa():
    """Per-head Q/K LayerNorm over 128-dim heads (two values per lane), grouped heads."""
    _parity_full(RAGGED_SLM12.with_(n_heads=4, head_dim=128, n_kv_heads=2, rot_dim=32,
                                    seed=46), tag="head_ln hd128")


def test_head_layernorm_reading_negative_control():
    """The per-head LayerNorm model checked against an oracle that applies one RMSNorm to the
    whole Q and K rows (the OLMo-2 reading) must fail the gate."""
    cfg = RAGGED_SLM12
    W, ids = synth_weights(cfg), synth_ids(cfg)
    g, _ = U.run_gpu(U.get_model(cfg, W), ids)
    r = U.oracle_run(cfg.with_(qk_norm="full_rms"), W, ids, residuals=False)
    assert U.cosines(g.cpu().numpy(), r).min() < U.COS_MIN


def test_learned_positions_small():
    _parity_full(RAGGED_POS)


def test_learned_positions_full_table():
    """seq = max_seq: the last row of the position table is read."""
    _parity_full(RAGGED_POS.with_(batch=1, seq=128, seed=26), tag="pos seq=max_seq")


def test_learned_positions_negative_control():
    """The model checked against an oracle without its position rows must fail the gate."""
    cfg = RAGGED_POS
    W, ids = synth_weights(cfg), synth_ids(cfg)
    g, _ = U.run_gpu(U.get_model(cfg, W), ids)
    r = U.oracle_run(cfg.with_(learned_pos=False), W, ids, residuals=False)
    assert U.cosines(g.cpu().numpy(), r).min() < U.COS_MIN


@pytest.mark.parametrize("cfg", [RAGGED_SLM.with_(batch=4, seed=50), RAGGED_BLOOM.with_(batch=3),
                                 RAGGED_OLMO.with_(batch=3), RAGGED_SLM12.with_(batch=3),
                                 RAGGED_POS], ids=lambda c: c.name)
def test_padding_mask(cfg):
    """attention_mask with left, right and hole padding (and a fully padded row) on every
    block variant; all positions are compared (padding positions are defined too)."""
    _parity_full(cfg, mask=_pad_masks(cfg.batch, cfg.seq, 60), tag=cfg.name + " padded")


def test_padding_mask_negative_control():
    """A padded GPU run checked against the oracle without the mask must fail the gate."""
    cfg = RAGGED_SLM
    mask = _pad_masks(cfg.batch, cfg.seq, 61)
    W, ids = synth_weights(cfg), synth_ids(cfg)
    g, _ = U.run_gpu(U.get_model(cfg, W), ids, mask=mask)
    r = U.oracle_run(cfg, W, ids, residuals=False)
    assert U.cosines(g.cpu().numpy(), r).min() < U.COS_MIN


def test_all_ones_mask_is_bitwise_unpadded():
    cfg = RAGGED_SLM
    model = U.get_model(cfg)
    ids = synth_ids(cfg)
    a, _ = U.run_gpu(model, ids)
    b, _ = U.run_gpu(model, ids, mask=np.ones(ids.shape, np.int32))
    assert torch.equal(a, b)


@pytest.mark.parametrize("logits16", [False, True])
def test_next_token_probs(logits16):
    """GPU next-token probabilities against (a) the softmax of the GPU's own last-position
    logits on the host in float64 (the kernel's arithmetic, rel. 1e-5) and (b) the
    oracle's distribution (total variation <= 2.5e-3, from the logit gate)."""
    from dense_transformer_prefill_amd import PrefillModel, upload_weights
    cfg = RAGGED_SLM
    W, ids = synth_weights(cfg), synth_ids(cfg)
    model = PrefillModel(cfg, upload_weights(W),
                         logits_dtype=torch.float16 if logits16 else torch.float32)
    mask = _pad_masks(cfg.batch, cfg.seq, 62)
    g, _, p = U.run_gpu(model, ids, mask=mask, probs=True)
    model.close()
    p = p.cpu().numpy().astype(np.float64)
    last = g[:, -1].float().cpu().numpy().astype(np.float64)
    own = np.exp(last - last.max(-1, keepdims=True))
    own /= own.sum(-1, keepdims=True)
    assert np.abs(p - own).max() <= 1e-5 * own.max()
    ref = oracle.next_token_probs(U.oracle_run(cfg, W, ids, residuals=False, mask=mask))
    tv = 0.5 * np.abs(p - ref).sum(-1).max()
    print(f"next-token probs: max |p - softmax(own logits)| {np.abs(p - own).max():.2e}, "
          f"total variation vs oracle {tv:.2e}")
    assert tv <= 2.5e-3
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-5)


def test_q8_0_codes_bit_exact():
    """The library's Q8_0 encoder against the oracle's, code for code and scale for scale:
    random rows, integer blocks, half-way ties, zero blocks, float16 extremes and a
    packed-size weight matrix."""
    from dense_transformer_prefill_amd import quantize_q8_0
    r = np.random.default_rng(70)
    w = (r.normal(size=(64, 512)) * 0.02).astype(np.float16)
    w[0, :32] = r.integers(-127, 128, 32)
    w[0, 0] = 127
    w[1, :32] = 0
    w[1, 32:64] = [127, 2.5, -2.5, 0.5, -0.5, 1.5] + [0] * 26
    w[2, :32] = np.float16(65504)
    w[2, 32:64] = np.float16(6e-8)                        # float16 subnormals
    w[3] = (r.normal(size=512) * 1000).astype(np.float16)
    big = synth_weights(RAGGED_SLM)["layers.0.gate_w"]
    for m in (w, big):
        q, d = quantize_q8_0(torch.from_numpy(np.ascontiguousarray(m)).cuda())
        torch.cuda.synchronize()
        rq, rd = oracle.quantize_q8_0(m)
        assert np.array_equal(q.cpu().numpy(), rq)
        assert np.array_equal(d.cpu().numpy().view(np.uint16), rd.view(np.uint16))


@pytest.mark.parametrize("cfg", [RAGGED_SLM.with_(weight_format="q8_0", seed=71),
                                 RAGGED_BLOOM.with_(weight_format="q8_0", seed=72),
                                 RAGGED_OLMO.with_(weight_format="q8_0", seed=73)],
                         ids=lambda c: c.name)
def test_q8_0_models(cfg):
    """Q8_0 weights through packing, per-GEMM decoding and the float16 GEMMs, against the
    oracle's forward on the decoded weights."""
    _parity_full(cfg, tag=cfg.name + " q8_0")


@pytest.mark.parametrize("fmt", ["f16", "q8_0"])
def test_caller_workspace_matches_own(fmt):
    """tf_prefill_ex with a caller-provided workspace of exactly tf_workspace_size bytes
    (padding mask and, for Q8_0, the decoded-weight slice inside it) gives the same bits as
    the handle's own workspace; one byte short is rejected."""
    from dense_transformer_prefill_amd import TfError
    cfg = RAGGED_SLM.with_(weight_format=fmt, seed=80)
    model = U.get_model(cfg)
    ids = torch.from_numpy(synth_ids(cfg)).cuda()
    mask = torch.from_numpy(_pad_masks(cfg.batch, cfg.seq, 81)).cuda()
    a = model.prefill(ids, attention_mask=mask)
    n = model.workspace_bytes(cfg.batch, cfg.seq)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = model.prefill(ids, attention_mask=mask, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    with pytest.raises(TfError):
        model.prefill(ids, attention_mask=mask, workspace=ws[:n - 256])


@pytest.mark.parametrize("cfg", [CONFIGS["c0_tiny"], RAGGED_SLM], ids=lambda c: c.name)
def test_plain_tf_prefill_entry_point(cfg):
    """`tf_prefill(cfg, weights, ids, batch, seq, logits_out, stream)` called through ctypes
    directly: bit for bit what `tf_prefill_ex(..., opts=NULL)` and `tf_prefill_ex` with an
    all-default options struct give, and within the default gates of the oracle."""
    import ctypes as C
    from dense_transformer_prefill_amd import _abi as A
    W, ids_np = synth_weights(cfg), synth_ids(cfg)
    model = U.get_model(cfg, W)
    lib = model.lib
    ids = torch.from_numpy(ids_np).cuda()
    b, s = ids.shape
    outs = [torch.full((b, s, cfg.vocab), float("nan"), dtype=torch.float32, device="cuda")
            for _ in range(3)]
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = (C.byref(model.c_cfg), model.handle, C.c_void_p(ids.data_ptr()), b, s)
    A.check(lib.tf_prefill(*args, C.c_void_p(outs[0].data_ptr()), st))
    A.check(lib.tf_prefill_ex(*args, C.c_void_p(outs[1].data_ptr()), st, None))
    opts = A.TfPrefillOpts()
    A.check(lib.tf_prefill_ex(*args, C.c_void_p(outs[2].data_ptr()), st, C.byref(opts)))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    r = U.oracle_run(cfg, W, ids_np, residuals=False)
    U.assert_parity(outs[0].cpu().numpy(), r, tag=cfg.name + " tf_prefill")


def test_seq_one_and_batch_rows():
    cfg = RAGGED_SLM.with_(batch=5, seq=1)
    _parity_full(cfg, tag="seq1")


def test_deterministic_and_rows_independent():
    cfg = RAGGED_SLM
    model = U.get_model(cfg)
    ids = synth_ids(cfg)
    ids[2] = ids[0]
    a, _ = U.run_gpu(model, ids)
    b, _ = U.run_gpu(model, ids)
    assert torch.equal(a, b)
    assert torch.equal(a[2], a[0])


def test_empty_call_is_noop():
    cfg = RAGGED_SLM
    model = U.get_model(cfg)
    ids = torch.zeros((0, 5), dtype=torch.int32, device="cuda")
    out = model.prefill(ids)
    assert out.shape == (0, 5, cfg.vocab)


def test_out_of_range_id_poisons_only_its_batch_row():
    cfg = RAGGED_SLM.with_(batch=3, seq=9)
    model = U.get_model(cfg, key=(RAGGED_SLM, "default"))
    ids = synth_ids(cfg)
    ref, _ = U.run_gpu(model, ids)
    ids[1, 4] = cfg.vocab + 5
    ids[2, 0] = -3
    out, _ = U.run_gpu(model, ids)
    out, ref = out.cpu().numpy(), ref.cpu().numpy()
    assert np.array_equal(out[0], ref[0])
    assert np.isnan(out[1, 4:]).all() and np.isnan(out[2]).all()


def test_full_rope_negative_control():
    """A GPU run with the model's 16-dim rotary span compared against an oracle that
    rotates all 64 dims must fail the gate at positions >= 1 (p = 0 is unaffected)."""
    cfg = CONFIGS["c0_tiny"].with_(seq=48)
    W, ids = synth_weights(cfg), synth_ids(cfg)
    g, _ = U.run_gpu(U.get_model(cfg, W), ids)
    r = U.oracle_run(cfg.with_(rot_dim=64), W, ids, residuals=False)
    c = U.cosines(g.cpu().numpy(), r)
    print("full-rope control cosines: p0 %.8f, min(p>=1) %.6f" % (c[0], c[1:].min()))
    assert c[0] >= U.COS_MIN
    assert c[1:].min() < U.COS_MIN


def test_fused_qkv_block_reading_negative_control():
    """Reading the per-head interleaved fused QKV tensor as [Q; K; V] blocks must fail."""
    cfg = RAGGED_BLOOM
    W, ids = synth_weights(cfg), synth_ids(cfg)
    g, _ = U.run_gpu(U.get_model(cfg, W), ids)
    Wb = dict(W)
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        Wb[p + "q_w"], Wb[p + "k_w"], Wb[p + "v_w"] = np.split(W[p + "qkv_fused_w"], 3)
        Wb[p + "q_b"], Wb[p + "k_b"], Wb[p + "v_b"] = np.split(W[p + "qkv_fused_b"], 3)
    r = U.oracle_run(cfg.with_(qkv_layout="separate"), Wb, ids, residuals=False)
    assert U.cosines(g.cpu().numpy(), r).min() < U.COS_MIN


def test_norm_slot_swap_negative_control():
    """Post-attention norm loaded into the post-feedforward slot must fail the gate."""
    cfg = RAGGED_OLMO
    W, ids = synth_weights(cfg), synth_ids(cfg)
    g, _ = U.run_gpu(U.get_model(cfg, W), ids)
    Wc = dict(W)
    for l in range(cfg.n_layers):
        Wc[f"layers.{l}.post_ff_norm_w"] = W[f"layers.{l}.post_attn_norm_w"]
    r = U.oracle_run(cfg, Wc, ids, residuals=False)
    assert U.cosines(g.cpu().numpy(), r).min() < U.COS_MIN


def _mid_row_max_moves(cfg, W, ids, layer=0, margin=8.0):
    """(moves, largest |score|) of `layer`: moves counts the queries whose running score max
    (log2 domain, moved only when a later 64-key tile's max exceeds it by more than
    `margin`) moves after their first tile, from the oracle's own queries and keys."""
    dt = np.float64
    x = oracle.embed(cfg, W, ids, dt)
    for l in range(layer):
        x = oracle.block(cfg, W, l, x, dt)
    tr = {}
    oracle.block(cfg, W, layer, x, dt, trace=tr)
    q, k = tr["attention_queries"], tr["attention_keys"]
    t = (q @ k.transpose(0, 1, 3, 2)) / np.sqrt(cfg.head_dim) * np.log2(np.e)
    moves = 0
    for i in range(t.shape[2]):
        row = t[:, :, i, :i + 1]
        m = row[:, :, :64].max(-1)
        for j0 in range(64, i + 1, 64):
            tm = row[:, :, j0:j0 + 64].max(-1)
            mv = tm > m + margin
            moves += int(mv.sum())
            m = np.where(mv, tm, m)
    causal = np.tril(np.ones(t.shape[-2:], bool))
    return moves, float(np.abs(t[..., causal]).max())


# (model, weight slots scaled, factor): the StableLM form's Q/K projections (d = 64), and
# OLMo-2's Q/K RMSNorm gains (its norms undo a projection scale; d = 128, where each wave
# starts the next tile's score MFMAs before the current tile's softmax may move the max).
MID_ROW_CASES = {
    "slm": (RAGGED_SLM.with_(batch=2, seq=300, seed=71), ("q_w", "k_w", "q_b", "k_b"), 4.0),
    "olmo": (RAGGED_OLMO.with_(batch=2, seq=300, seed=73), ("q_norm_w", "k_norm_w"), 2.0),
}


FLOOR_FACTOR = 1.25   # the GPU's error may exceed the fp16-storage floor by this much


@pytest.mark.parametrize("case,padded", [("slm", False), ("slm", True), ("olmo", False)])
def test_running_max_moves_mid_row(case, padded):
    """Scaled query and key projections (or QK-norm gains) spread the scores (log2-domain
    std about 4.6 for the StableLM case), so a query's running max moves after its first
    key tile: the path that rescales the output and the row sum and restarts the score
    accumulators at the new max. The oracle confirms such moves occur (33 and 51); the GPU
    path must match it.

    Gates: with scores up to about 26-29 in the log2 domain (asserted <= 32), the fp16
    storage of q, k, v and P alone moves the result further from the float64 oracle than
    the default gates allow. The test measures that floor on this very input: the forward
    run in float64 with the library's fp16 roundings inserted (`tests/fp16_floor.py`), and
    gates the GPU's cosine gap and residual error at FLOOR_FACTOR times the floor's; argmax
    still exact. A fault in the rescale path itself mis-scales probabilities by 2^8 or more
    and fails them by far. `padded` runs the padding-mask kernel (row 0 left-padded past
    the first key tile, row 1 right-padded); the moves are counted on the unpadded rows."""
    from . import fp16_floor
    cfg, slots, factor = MID_ROW_CASES[case]
    W, ids = synth_weights(cfg), synth_ids(cfg)
    for l in range(cfg.n_layers):
        for n in slots:
            key = f"layers.{l}.{n}"
            W[key] = (W[key].astype(np.float32) * factor).astype(np.float16)
    moves, tmax = _mid_row_max_moves(cfg, W, ids)
    assert moves > 0 and tmax <= 32.0, (moves, tmax)
    mask = _pad_masks(cfg.batch, cfg.seq, 72) if padded else None
    model = U.get_model(cfg, W, key=(cfg, "qk scaled", factor))
    g, gres = U.run_gpu(model, ids, dump=True, mask=mask)
    r, rres = U.oracle_run(cfg, W, ids, mask=mask)
    e, eres = fp16_floor.forward(cfg, W, ids, attention_mask=mask)
    g, gres = g.cpu().numpy(), gres.cpu().numpy()
    assert np.isfinite(g).all()
    c, ce = U.cosines(g, r), U.cosines(e, r)
    nq, na = U.argmax_check(g, r)
    errs = [U.resid_err(gres[l], rres[l]) for l in range(len(rres))]
    floor = [U.resid_err(eres[l], rres[l]) for l in range(len(rres))]
    to_floor = [U.resid_err(gres[l], eres[l]) for l in range(len(rres))]
    gap, gap_floor = 1.0 - c.min(), 1.0 - ce.min()
    msg = (f"GPU: min cos {c.min():.8f} (gap {gap:.3e}), max residual rel err {max(errs):.3e}; "
           f"fp16-storage floor: gap {gap_floor:.3e}, residual {max(floor):.3e}; "
           f"GPU vs floor emulation: residual {max(to_floor):.3e}; argmax {na}/{nq}")
    print(msg, flush=True)
    assert gap <= FLOOR_FACTOR * gap_floor, msg
    assert max(errs) <= FLOOR_FACTOR * max(floor), msg
    assert na == nq, msg


def test_alibi_model_rotary_off_is_finite():
    cfg = RAGGED_BLOOM.with_(seq=300)
    g, _ = U.run_gpu(U.get_model(cfg, key=(RAGGED_BLOOM, "default")), synth_ids(cfg))
    assert torch.isfinite(g).all()


# ------------------------------------------------------------------ full-size workloads

def _sampled(name, rows, prefix, deep_row=None, dtype=np.float32, mask=None):
    """Full-size run on the GPU; oracle on sampled rows' prefixes (every position's logits
    and per-layer residuals), and on one whole row (`deep_row`) with logits at sampled
    positions up to the last one and residuals at every position. With a padding mask the
    prefix of a row and its mask is still an exact sub-problem."""
    cfg = CONFIGS[name]
    W, ids = synth_weights(cfg), synth_ids(cfg)
    model = U.get_model(cfg, W)
    g, gres = U.run_gpu(model, ids, dump=True, mask=mask)
    assert torch.isfinite(g).all()
    sub_mask = lambda r, n: None if mask is None else mask[r:r + 1, :n]
    for r in rows:
        sub = cfg.with_(batch=1, seq=prefix)
        ref, rres = U.oracle_run(sub, W, ids[r:r + 1, :prefix], dtype=dtype,
                                 mask=sub_mask(r, prefix))
        U.assert_parity(g[r:r + 1, :prefix].cpu().numpy(), ref,
                        gres[:, r:r + 1, :prefix].cpu().numpy(), np.stack(rres),
                        tag=f"{name} row {r} prefix {prefix}")
    if deep_row is not None:
        s = cfg.seq
        pos = sorted({0, 1, s // 4, s // 2, s - 2, s - 1} |
                     set(np.random.default_rng(s).integers(0, s, 10).tolist()))
        ref, rres = U.oracle_run(cfg.with_(batch=1), W, ids[deep_row:deep_row + 1], dtype=dtype,
                                 logit_positions=pos, mask=sub_mask(deep_row, s))
        U.assert_parity(g[deep_row:deep_row + 1, pos].cpu().numpy(), ref,
                        gres[:, deep_row:deep_row + 1].cpu().numpy(), np.stack(rres),
                        tag=f"{name} row {deep_row} all {s} positions, logits at {len(pos)}")
    del g, gres
    U.drop_models()


def test_c1_full_parity():
    cfg = CONFIGS["c1_stablelm2_s512"]
    _parity_full(cfg, dtype=np.float32)
    U.drop_models()


@pytest.mark.timeout(1200)
def test_c2_full_parity_every_position():
    """The benchmark workload (8 x 2048) checked at every (batch row, position): the float64
    oracle runs one whole batch row at a time (rows are independent sequences), and each
    row's 2048 logit vectors and 25 residual layers are gated like the small models'."""
    import time
    name = "c2_stablelm2_b8s2048"
    cfg = CONFIGS[name]
    W, ids = synth_weights(cfg), synth_ids(cfg)
    model = U.get_model(cfg, W)
    g, gres = U.run_gpu(model, ids, dump=True)
    assert torch.isfinite(g).all()
    worst_cos, worst_res, qual, agree = 1.0, 0.0, 0, 0
    for r in range(cfg.batch):
        t0 = time.time()
        ref, rres = U.oracle_run(cfg.with_(batch=1), W, ids[r:r + 1], dtype=np.float64)
        c, errs = U.assert_parity(g[r:r + 1].cpu().numpy(), ref,
                                  gres[:, r:r + 1].cpu().numpy(), np.stack(rres),
                                  tag=f"{name} row {r}, all {cfg.seq} positions "
                                      f"({time.time() - t0:.0f} s)")
        nq, na = U.argmax_check(g[r:r + 1].cpu().numpy(), ref)
        worst_cos, worst_res = min(worst_cos, c.min()), max(worst_res, max(errs))
        qual, agree = qual + nq, agree + na
        del ref, rres
    print(f"{name}: {cfg.batch * cfg.seq} positions, min cos {worst_cos:.8f}, "
          f"argmax {agree}/{qual}, max residual rel err {worst_res:.2e}", flush=True)
    del g, gres
    U.drop_models()


@pytest.mark.timeout(600)
def test_c2_share_full_parity():
    """One batch row of 2048 tokens (one GPU's share of the benchmark workload split
    data-parallel): its O and down projections run 128x128 tiles with split K, the
    others 256x256. Every position and residual layer against the float64 oracle."""
    _parity_full(CONFIGS["c2_share_b1s2048"])
    U.drop_models()


def test_c3_sampled_parity():
    _sampled("c3_bloom560m", rows=[1, 3], prefix=192, deep_row=2)


def test_c4_sampled_parity():
    """seq 4096 = max_seq: the longest rotary table row and attention span."""
    _sampled("c4_olmo2_1b", rows=[2], prefix=160, deep_row=1)


def test_c5_sampled_parity():
    """StableLM-2-12B's block at 1.6B sizes (8 key/value heads, parallel, per-head LN)."""
    _sampled("c5_slm12b_block_b8s2048", rows=[4], prefix=160, deep_row=6)


def test_c6_sampled_parity():
    """Learned absolute positions on GPT-2-small sizes, seq = max_seq = 1024."""
    _sampled("c6_learned_pos_b4s1024", rows=[3], prefix=160, deep_row=1)


def test_c2_padded_sampled_parity():
    """The benchmark workload with left padding of a different length in every row (row r
    starts at 200 r), checked on two rows' prefixes and one whole row."""
    cfg = CONFIGS["c2_stablelm2_b8s2048"]
    mask = np.ones((cfg.batch, cfg.seq), np.int32)
    for r in range(cfg.batch):
        mask[r, :200 * r] = 0
    _sampled("c2_stablelm2_b8s2048", rows=[0, 1], prefix=256, deep_row=3, mask=mask)



def test_c7_q8_sampled_parity():
    """The benchmark shape with Q8_0 weights."""
    _sampled("c7_stablelm2_q8_b8s2048", rows=[2], prefix=160, deep_row=4)
