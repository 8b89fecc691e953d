"""CPU checks of the fp16-storage emulation the GPU stress test takes its error floor from:
with its roundings switched off it is the float64 oracle (so the floor it measures comes
from the roundings alone), and with them on it moves the result by about fp16's relative
precision."""
import numpy as np
import pytest

from workloads import ModelConfig, synth_ids, synth_weights

from . import fp16_floor
from . import gpu_util as U

SLM = ModelConfig(name="floor_slm", n_layers=2, hidden=256, n_heads=4, head_dim=64, inter=512,
                  vocab=300, batch=2, seq=150, seed=91)
OLMO = ModelConfig(name="floor_olmo", n_layers=2, hidden=256, n_heads=2, head_dim=128,
                   inter=512, vocab=300, batch=2, seq=150, norm_kind="rms", norm_place="post",
                   rot_dim=128, rope_theta=500000.0, qk_norm="full_rms", qkv_bias=False,
                   norm_eps=1e-6, qk_norm_eps=1e-6, seed=92)


def _mask(cfg):
    m = np.ones((cfg.batch, cfg.seq), np.int32)
    m[0, :70] = 0          # a query block whose first key tile is all padding
    m[1, cfg.seq - 20:] = 0
    return m


@pytest.mark.parametrize("cfg", [SLM, OLMO], ids=lambda c: c.name)
@pytest.mark.parametrize("masked", [False, True])
def test_emulation_without_rounding_is_the_oracle(cfg, masked, monkeypatch):
    W, ids = synth_weights(cfg), synth_ids(cfg)
    # scale q and k up so the running max moves after the first key tile
    for l in range(cfg.n_layers):
        for n in ("q_w", "k_w"):
            W[f"layers.{l}.{n}"] = (W[f"layers.{l}.{n}"].astype(np.float32) * 4).astype(np.float16)
    mask = _mask(cfg) if masked else None
    r, rres = U.oracle_run(cfg, W, ids, mask=mask)
    monkeypatch.setattr(fp16_floor, "_h", lambda a: np.asarray(a, np.float64))
    e, eres = fp16_floor.forward(cfg, W, ids, attention_mask=mask)
    assert np.abs(e - r).max() <= 1e-10 * np.abs(r).max()
    assert max(U.resid_err(eres[l], rres[l]) for l in range(len(rres))) <= 1e-11


def test_emulation_rounds_at_fp16_precision():
    cfg = SLM
    W, ids = synth_weights(cfg), synth_ids(cfg)
    r, rres = U.oracle_run(cfg, W, ids)
    e, eres = fp16_floor.forward(cfg, W, ids)
    err = max(U.resid_err(eres[l], rres[l]) for l in range(len(rres)))
    assert 1e-5 < err < 5e-3, err
