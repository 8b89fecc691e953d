"""Thin torch-facing wrapper over the C ABI: device tensors in, device tensors out.

PyTorch only supplies device memory and the current HIP stream. Every step of the
forward runs in the library's HIP kernels; this module only marshals pointers.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import _abi as A


def _stream_ptr(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def upload_weights(W: dict, device="cuda") -> dict:
    """Copy a {name: float16 ndarray} dict to contiguous float16 device tensors."""
    out = {}
    for k, v in W.items():
        if k in out:
            continue
        t = torch.from_numpy(np.ascontiguousarray(v))
        assert t.dtype == torch.float16, k
        out[k] = t.to(device, non_blocking=False)
    return out


def quantize_q8_0(w: torch.Tensor, stream=None):
    """Q8_0 encoding of a contiguous float16 device matrix [rows, cols] (cols a multiple
    of 32) by the library: (int8 codes [rows, cols], float16 scales [rows, cols / 32])."""
    if w.dtype != torch.float16 or not w.is_cuda or w.dim() != 2 or not w.is_contiguous():
        raise ValueError("w must be a contiguous float16 device matrix")
    rows, cols = w.shape
    q = torch.empty((rows, cols), dtype=torch.int8, device=w.device)
    d = torch.empty((rows, cols // 32), dtype=torch.float16, device=w.device)
    lib = A.load()
    A.check(lib.tf_quantize_q8_0(C.c_void_p(w.data_ptr()), rows, cols, C.c_void_p(q.data_ptr()),
                                 C.c_void_p(d.data_ptr()), C.c_void_p(_stream_ptr(stream))))
    return q, d


class PrefillModel:
    """Packed weights of one model on the current GPU.

    cfg: object with the ModelConfig attribute names. weights: {name: float16 device
    tensor} using the slot names of `workloads.synth.weight_slots` (per-layer names are
    prefixed "layers.{l}."). The raw tensors may be freed after construction.
    """

    def __init__(self, cfg, weights: dict, logits_dtype=torch.float32, stream=None):
        self.lib = A.load()
        self.cfg = cfg
        self.logits_dtype = logits_dtype
        self.c_cfg = A.config_to_c(
            cfg, A.TF_LOGITS_F32 if logits_dtype == torch.float32 else A.TF_LOGITS_F16)
        A.check(self.lib.tf_config_validate(C.byref(self.c_cfg)))

        def ptr(name):
            t = weights.get(name)
            if t is None:
                return None
            if t.dtype != torch.float16 or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"weight {name} must be a contiguous float16 device tensor")
            return t.data_ptr()

        layers = (A.TfRawLayer * cfg.n_layers)()
        for l in range(cfg.n_layers):
            for slot in A.RAW_LAYER_SLOTS:
                setattr(layers[l], slot, ptr(f"layers.{l}.{slot}"))
        raw = A.TfRawWeights()
        raw.embed = ptr("embed")
        raw.embed_norm_w = ptr("embed_norm_w")
        raw.embed_norm_b = ptr("embed_norm_b")
        raw.layers = C.cast(layers, C.POINTER(A.TfRawLayer))
        raw.final_norm_w = ptr("final_norm_w")
        raw.final_norm_b = ptr("final_norm_b")
        raw.lm_head = ptr("lm_head")
        raw.pos_embed = ptr("pos_embed")
        handle = C.c_void_p()
        A.check(self.lib.tf_weights_pack(C.byref(self.c_cfg), C.byref(raw),
                                          C.c_void_p(_stream_ptr(stream)), C.byref(handle)))
        self.handle = handle

    def workspace_bytes(self, batch: int, seq: int) -> int:
        n = C.c_size_t()
        A.check(self.lib.tf_workspace_size(C.byref(self.c_cfg), batch, seq, C.byref(n)))
        return n.value

    def prefill(self, ids: torch.Tensor, out: torch.Tensor | None = None,
                residual_dump: torch.Tensor | None = None, timed_kernel: int = 0,
                workspace: torch.Tensor | None = None, stream=None,
                attention_mask: torch.Tensor | None = None,
                next_token_probs: torch.Tensor | None = None) -> torch.Tensor:
        """ids: int32 device tensor [batch, seq]. Returns logits [batch, seq, vocab].
        Without options this is `tf_prefill`; any option goes through `tf_prefill_ex`.

        attention_mask: optional int32 device tensor [batch, seq], zeros marking padding.
        next_token_probs: optional float32 device tensor [batch, vocab] that receives the
        softmax of the logits at position seq-1."""
        if ids.dtype != torch.int32 or not ids.is_cuda or ids.dim() != 2:
            raise ValueError("ids must be an int32 device tensor [batch, seq]")
        ids = ids.contiguous()
        b, s = ids.shape
        if out is None:
            out = torch.empty((b, s, self.cfg.vocab), dtype=self.logits_dtype, device=ids.device)
        elif (out.dtype != self.logits_dtype or tuple(out.shape) != (b, s, self.cfg.vocab)
              or not out.is_contiguous()):
            raise ValueError("out has the wrong dtype, shape or layout")
        if (residual_dump is None and workspace is None and not timed_kernel
                and attention_mask is None and next_token_probs is None):
            A.check(self.lib.tf_prefill(C.byref(self.c_cfg), self.handle,
                                        C.c_void_p(ids.data_ptr()), b, s,
                                        C.c_void_p(out.data_ptr()),
                                        C.c_void_p(_stream_ptr(stream))))
            return out
        opts = A.TfPrefillOpts()
        if residual_dump is not None:
            want = (self.cfg.n_layers + 1, b, s, self.cfg.hidden)
            if (residual_dump.dtype != torch.float32 or tuple(residual_dump.shape) != want
                    or not residual_dump.is_contiguous()):
                raise ValueError(f"residual_dump must be contiguous float32 {want}")
            opts.residual_dump = residual_dump.data_ptr()
        if workspace is not None:
            opts.workspace = workspace.data_ptr()
            opts.workspace_bytes = workspace.numel() * workspace.element_size()
        opts.timed_kernel = timed_kernel
        if attention_mask is not None:
            if (attention_mask.dtype != torch.int32 or not attention_mask.is_cuda
                    or tuple(attention_mask.shape) != (b, s) or not attention_mask.is_contiguous()):
                raise ValueError("attention_mask must be a contiguous int32 device tensor [batch, seq]")
            opts.attention_mask = attention_mask.data_ptr()
        if next_token_probs is not None:
            if (next_token_probs.dtype != torch.float32 or not next_token_probs.is_cuda
                    or tuple(next_token_probs.shape) != (b, self.cfg.vocab)
                    or not next_token_probs.is_contiguous()):
                raise ValueError("next_token_probs must be a contiguous float32 device tensor "
                                 "[batch, vocab]")
            opts.next_token_probs = next_token_probs.data_ptr()
        A.check(self.lib.tf_prefill_ex(C.byref(self.c_cfg), self.handle, C.c_void_p(ids.data_ptr()),
                                       b, s, C.c_void_p(out.data_ptr()),
                                       C.c_void_p(_stream_ptr(stream)), C.byref(opts)))
        return out

    def prefill_noalloc(self, ids: torch.Tensor, out: torch.Tensor, stream=None) -> torch.Tensor:
        """`tf_prefill_noalloc`: the forward on the library's fixed per-GPU workspace, with no
        allocation by the library (out must be given). Calls on one GPU must not overlap."""
        if ids.dtype != torch.int32 or not ids.is_cuda or ids.dim() != 2 or not ids.is_contiguous():
            raise ValueError("ids must be a contiguous int32 device tensor [batch, seq]")
        b, s = ids.shape
        if (out.dtype != self.logits_dtype or tuple(out.shape) != (b, s, self.cfg.vocab)
                or not out.is_contiguous()):
            raise ValueError("out has the wrong dtype, shape or layout")
        A.check(self.lib.tf_prefill_noalloc(C.byref(self.c_cfg), self.handle,
                                            C.c_void_p(ids.data_ptr()), b, s,
                                            C.c_void_p(out.data_ptr()),
                                            C.c_void_p(_stream_ptr(stream))))
        return out

    def timing(self, kernel: int):
        """(total milliseconds, launches) recorded for a kernel class since the last read."""
        ms, n = C.c_double(), C.c_int32()
        A.check(self.lib.tf_timing_read(self.handle, kernel, C.byref(ms), C.byref(n)))
        return ms.value, n.value

    def close(self):
        if getattr(self, "handle", None):
            self.lib.tf_weights_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
