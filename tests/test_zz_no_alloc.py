"""moe_forward_noalloc (the entry point for callers that cannot allocate: the library's fixed per-device
scratch instead of a workspace) against moe_forward on the same inputs, bit for bit, on two calls in a row,
the second with a smaller batch; and its host-side refusal of batches beyond the scratch."""
import ctypes

import numpy as np
import pytest

import synth
from tests import _harness as H

pytestmark = pytest.mark.gpu


def _noalloc(moe, cfg, N, x, weights, y, idx, wt, counts):
    import torch

    st = moe.lib().moe_forward_noalloc(ctypes.byref(cfg), int(N), x.data_ptr(), ctypes.byref(weights), y.data_ptr(),
                                       idx.data_ptr(), wt.data_ptr(), counts.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream)
    return st


@pytest.mark.parametrize("name,sizes", [("glm5_decode", (32, 7)), ("tiny_fp32", (64, 13))])
def test_noalloc_matches_forward(name, sizes):
    import torch

    import sparse_moe_layer_gate_amd as moe

    w = synth.WORKLOADS[name]
    print(f"[noalloc] {name} N={sizes}", flush=True)
    _, _, dev = H.device_weights(w, generate_on_device=w.dtype == "bf16")
    x_all = H.to_device(synth.x_host(w.with_tokens(max(sizes))))
    cfg = moe.config_of(w)
    weights = moe.weights_struct(cfg, dev)
    moe.lib().moe_forward_noalloc.restype = ctypes.c_int
    for N in sizes:
        x = x_all[:N].contiguous()
        y = torch.empty_like(x)
        idx = torch.empty((N, w.k), dtype=torch.int32, device="cuda")
        wt = torch.empty((N, w.k), dtype=torch.float32, device="cuda")
        counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
        assert _noalloc(moe, cfg, N, x, weights, y, idx, wt, counts) == moe.MOE_OK
        torch.cuda.synchronize()
        y_ref, i_ref, w_ref, c_ref = H.gpu_forward(w, x, dev)
        assert np.array_equal(H.to_host(y), y_ref), N
        assert np.array_equal(H.to_host(idx), i_ref) and np.array_equal(H.to_host(wt), w_ref)
        assert np.array_equal(H.to_host(counts), c_ref)


def test_noalloc_refuses_batches_beyond_scratch():
    import torch

    import sparse_moe_layer_gate_amd as moe

    w = synth.WORKLOADS["glm5_decode"]
    cfg = moe.config_of(w)
    lim = moe.lib().moe_noalloc_scratch_bytes
    lim.restype = ctypes.c_size_t
    N = 1
    while moe.moe_workspace_size(cfg, N) <= lim():
        N *= 2
    fake = ctypes.c_void_p(4096)  # never dereferenced: the size check comes first
    ws = moe.MoeWeights(fake, fake, fake, fake, fake, fake, fake)
    assert moe.lib().moe_forward_noalloc(ctypes.byref(cfg), N, fake, ctypes.byref(ws), fake, None, None, None,
                                         None) == moe.MOE_ERR_WORKSPACE
    del torch
