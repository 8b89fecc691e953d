"""Helpers of the GPU parity tests: run the HIP path, run the oracle, compare with the
gates (per-position logit cosine, argmax where the oracle's top-2 margin is clear,
per-layer residual row-normwise relative error)."""
import numpy as np
import torch

import oracle
from workloads import synth_ids, synth_weights

COS_MIN = 0.99999        # per-position logit cosine
MARGIN = 1e-2            # argmax compared where oracle top1 - top2 > MARGIN
RESID_RTOL = 5e-3        # per-layer residual: max_row ||g - r||_inf / ||r||_inf

_model_cache = {}


def get_model(cfg, W=None, key=None):
    """Pack (once per key) the model of cfg on cuda:0."""
    from dense_transformer_prefill_amd import PrefillModel, upload_weights
    key = key or (cfg, "default")
    if key not in _model_cache:
        if W is None:
            W = synth_weights(cfg)
        dev = upload_weights(W)
        _model_cache[key] = PrefillModel(cfg, dev)
        del dev
        torch.cuda.synchronize()
    return _model_cache[key]


def drop_models():
    for m in _model_cache.values():
        m.close()
    _model_cache.clear()
    torch.cuda.empty_cache()


def run_gpu(model, ids_np, dump=False, mask=None, probs=False):
    """Logits (and the residual dump) of the HIP path; with probs=True also the
    next-token probabilities, as a third value."""
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).cuda()
    b, s = ids.shape
    res = None
    if dump:
        res = torch.empty((model.cfg.n_layers + 1, b, s, model.cfg.hidden),
                          dtype=torch.float32, device="cuda")
    am = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask, dtype=np.int32)).cuda()
    ntp = torch.empty((b, model.cfg.vocab), dtype=torch.float32, device="cuda") if probs else None
    out = model.prefill(ids, residual_dump=res, attention_mask=am, next_token_probs=ntp)
    torch.cuda.synchronize()
    return (out, res, ntp) if probs else (out, res)


def cosines(g, r):
    g = g.reshape(-1, g.shape[-1]).astype(np.float64)
    r = r.reshape(-1, r.shape[-1]).astype(np.float64)
    return (g * r).sum(-1) / (np.linalg.norm(g, axis=-1) * np.linalg.norm(r, axis=-1))


def argmax_check(g, r):
    """(qualifying positions, agreements) where the oracle's top-2 margin > MARGIN."""
    g = g.reshape(-1, g.shape[-1])
    r = r.reshape(-1, r.shape[-1]).astype(np.float64)
    top2 = np.partition(r, -2, axis=-1)[:, -2:]
    margin = top2[:, 1] - top2[:, 0]
    q = margin > MARGIN
    agree = np.argmax(g, -1) == np.argmax(r, -1)
    return int(q.sum()), int((agree & q).sum())


def resid_err(g, r):
    """max over rows of ||g - r||_inf / ||r||_inf (rows along the last axis)."""
    g = g.reshape(-1, g.shape[-1]).astype(np.float64)
    r = r.reshape(-1, r.shape[-1]).astype(np.float64)
    return float((np.abs(g - r).max(-1) / np.abs(r).max(-1)).max())


def assert_parity(g_logits, r_logits, g_res=None, r_res=None, tag=""):
    c = cosines(g_logits, r_logits)
    nq, na = argmax_check(g_logits, r_logits)
    msg = f"{tag}: min cos {c.min():.8f} mean {c.mean():.8f}; argmax {na}/{nq}"
    errs = []
    if g_res is not None:
        errs = [resid_err(g_res[l], r_res[l]) for l in range(len(r_res))]
        msg += f"; max residual rel err {max(errs):.2e} (layer {int(np.argmax(errs))})"
    print(msg, flush=True)
    assert np.isfinite(g_logits).all(), tag + ": non-finite logits"
    assert c.min() >= COS_MIN, msg
    assert na == nq, msg
    if errs:
        assert max(errs) <= RESID_RTOL, msg
    return c, errs


def oracle_run(cfg, W, ids, dtype=np.float64, residuals=True, logit_positions=None, mask=None):
    return oracle.forward(cfg, W, ids, dtype=dtype, residuals=residuals,
                          logit_positions=logit_positions, attention_mask=mask)
