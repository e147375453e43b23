"""HIP graph capture of the forward.  A forward launches kernels only (no
memset, copy or allocation), so it can be captured into a graph and replayed;
each replay runs after other eager work and a synchronization and must give
the eager output bit for bit.  Covers the workspace forward, the no-alloc
forward (the library's own workspace) and a chained MLP pair."""
import ctypes as C

import numpy as np
import pytest

import oracle as o
from diffusion_smooth_group_amd import svdq as S
from diffusion_smooth_group_amd import workloads as wl
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


def _layer(fmt, M=700, K=512, N=768, seed=960):
    spec = wl.small_spec("graph", M, K, N, o.BF16, fmt, 16, lora_rank=8, seed=(seed, 0))
    d = wl.generate(spec)
    Xd = S.bits_to_device(d["X"], S.BF16, G.device())
    lin = G.pack_gpu(d, fmt, 16, cap=24, absmax=G.calib_absmax_gpu(Xd, o.BF16))
    lin.attach_lora(d["lora_A"], d["lora_B"], 1.0)
    return lin, Xd


def _capture(fn):
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        fn()                                 # once eagerly on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            fn()
    torch.cuda.synchronize()
    return g


def _replays(g, Y, ref, eager):
    import torch
    for rep in range(3):
        Y.fill_(0)                           # eager fill outside the graph
        eager()                              # other eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(S.device_to_bits(Y), ref), f"replay {rep}"


@pytest.mark.parametrize("fmt,gelu", [(o.MXFP4, False), (o.MXFP4, True), (o.INT4, True), (o.INT8, False)])
def test_forward_graph_replays(fmt, gelu):
    import torch
    lin, Xd = _layer(fmt)
    M, N = Xd.shape[0], lin.N
    ref = S.device_to_bits(lin.forward(Xd, gelu=gelu))
    Y = torch.empty((M, N), dtype=Xd.dtype, device=Xd.device)
    ws = torch.empty_like(lin.workspace(M))
    g = _capture(lambda: lin.forward(Xd, gelu=gelu, Y=Y, ws=ws))
    other = torch.empty_like(Y)
    _replays(g, Y, ref, lambda: lin.forward(Xd, gelu=not gelu, Y=other))


def test_noalloc_forward_graph_replays():
    import torch
    lin, Xd = _layer(o.MXFP4, seed=961)
    M, N = Xd.shape[0], lin.N
    ref = S.device_to_bits(lin.forward(Xd, gelu=True))
    Y = torch.empty((M, N), dtype=Xd.dtype, device=Xd.device)
    lib = S.lib_handle()

    def run():
        rc = lib.svdq_linear_forward_noalloc(C.byref(lin.layer), S._t_ptr(Xd), M, Xd.stride(0), S._t_ptr(Y),
                                             Y.stride(0), S.FLAG_GELU, S._stream())
        assert rc == 0

    g = _capture(run)
    other = torch.empty_like(Y)
    _replays(g, Y, ref, lambda: lin.forward(Xd, Y=other))


@pytest.mark.parametrize("fmt", [o.MXFP4, o.INT4])
def test_chained_pair_graph_replays(fmt):
    import torch
    fc1 = wl.small_spec("graph_fc1", 300, 256, 512, o.BF16, fmt, 16, seed=(962, 0))
    fc2 = wl.small_spec("graph_fc2", 300, 512, 256, o.BF16, fmt, 16, x_dist="gelu_of_fc1", seed=(962, 1))
    d1 = wl.generate(fc1)
    d2 = wl.generate(fc2, fc1_inputs=d1)
    dev = G.device()
    X = S.bits_to_device(d1["X"], S.BF16, dev)
    lin1 = G.pack_gpu(d1, fmt, 16, absmax=G.calib_absmax_gpu(X, o.BF16))
    lin2 = G.pack_gpu(d2, fmt, 16, absmax=G.calib_absmax_gpu(S.bits_to_device(d2["X"], S.BF16, dev), o.BF16))
    M = X.shape[0]
    need = S._SZ(0)
    S._call("svdq_chain_workspace_size", C.byref(lin1.layer), C.byref(lin2.layer), M, C.byref(need))
    ws1 = torch.empty(need.value, dtype=torch.uint8, device=dev)
    ws2 = torch.empty_like(lin2.workspace(M))
    Y2 = torch.empty((M, lin2.N), dtype=X.dtype, device=dev)

    def pair():
        lin1.forward_chain(lin2, X, gelu=True, ws=ws1, ws_next=ws2)
        lin2.gemm(M, Y2, ws2)

    pair()
    torch.cuda.synchronize()
    ref = S.device_to_bits(Y2)
    g = _capture(pair)
    other = torch.empty((M, lin1.N), dtype=X.dtype, device=dev)
    _replays(g, Y2, ref, lambda: lin1.forward(X, Y=other))
