"""tf_prefill_noalloc (the entry point for callers that cannot allocate) against tf_prefill:
called through the C ABI twice in a row, the second time with a smaller input, each output
bit for bit equal to tf_prefill's on the same handle and within the default gates of the
oracle; a call whose workspace exceeds the fixed array is rejected before any launch; and the
same entry point captured in a HIP graph replays bit for bit."""
import ctypes as C

import numpy as np
import pytest
import torch

from workloads import ModelConfig, synth_ids, synth_weights

from . import gpu_util as U

pytestmark = pytest.mark.gpu

CFG = ModelConfig(name="noalloc_slm", n_layers=2, hidden=512, n_heads=8, head_dim=64,
                  inter=1408, vocab=1000, batch=3, seq=150, seed=95)


def _noalloc(model, ids, out):
    from dense_transformer_prefill_amd import _abi as A
    b, s = ids.shape
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    return model.lib.tf_prefill_noalloc(C.byref(model.c_cfg), model.handle,
                                        C.c_void_p(ids.data_ptr()), b, s,
                                        C.c_void_p(out.data_ptr()), st)


def test_noalloc_matches_tf_prefill_twice_then_smaller():
    from dense_transformer_prefill_amd import _abi as A
    W = synth_weights(CFG)
    model = U.get_model(CFG, W, key=(CFG, "noalloc"))
    for b, s in [(3, 150), (2, 77)]:
        ids_np = synth_ids(CFG)[:b, :s]
        ids = torch.from_numpy(np.ascontiguousarray(ids_np)).cuda()
        want = model.prefill(ids)                     # tf_prefill, own workspace
        got = torch.full_like(want, float("nan"))
        A.check(_noalloc(model, ids, got))
        torch.cuda.synchronize()
        assert torch.equal(got, want), (b, s)
        r = U.oracle_run(CFG.with_(batch=b, seq=s), W, ids_np, residuals=False)
        U.assert_parity(got.cpu().numpy(), r, tag=f"noalloc b{b} s{s}")


def test_noalloc_rejects_a_workspace_beyond_its_array():
    from dense_transformer_prefill_amd import _abi as A
    model = U.get_model(CFG, key=(CFG, "noalloc"))
    b, s = 16, 4096                                   # needs more than the fixed array
    n = C.c_size_t()
    A.check(model.lib.tf_workspace_size(C.byref(model.c_cfg), b, s, C.byref(n)))
    assert n.value > A.NOALLOC_SCRATCH_BYTES
    ids = torch.zeros((b, s), dtype=torch.int32, device="cuda")
    out = torch.empty((1,), dtype=torch.float32, device="cuda")   # never written
    assert _noalloc(model, ids, out) == A.TF_ERR_INVALID_ARG
    assert "workspace" in model.lib.tf_last_error().decode()


def test_noalloc_forward_replays_from_a_captured_graph():
    """The no-allocation entry point captured in a HIP graph (torch.cuda.graph on the
    library's stream argument): three replays, each followed by eager calls of both entry
    points on the same GPU, each replay bit for bit equal to the eager tf_prefill."""
    from dense_transformer_prefill_amd import _abi as A
    W = synth_weights(CFG)
    model = U.get_model(CFG, W, key=(CFG, "noalloc"))
    ids = torch.from_numpy(synth_ids(CFG)).cuda()
    want = model.prefill(ids)
    out = torch.empty_like(want)
    A.check(_noalloc(model, ids, out))                # eager first call (takes the array's address)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        A.check(_noalloc(model, ids, out))
    torch.cuda.synchronize()
    other = torch.empty_like(want)
    for r in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), r
        model.prefill(ids, out=other)                 # eager work between the replays
        A.check(_noalloc(model, ids, other))
        torch.cuda.synchronize()
        assert torch.equal(other, want), r
