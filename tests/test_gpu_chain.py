"""GPU parity of epilogue chaining: an MLP's fc1 -> GELU -> fc2 where fc2's
activation pass (smoothing, 4-bit group quantization, down-projection) runs
in fc1's GEMM epilogue, for MXFP4 and for INT4 pairs.

Gates: fc2's activation codes and scales bit-identical to what fc2's own
activation kernel writes for fc1's stored output (which itself passes the
oracle's bit-exact code gate); T within one 16-bit rounding of that; fc1's
and fc2's outputs against the oracle's composition of the two layers (fc2
evaluated on the oracle's own rounded fc1 output) with the usual output gate.
"""
import numpy as np
import pytest

import oracle as o
from diffusion_smooth_group_amd import svdq as S
from diffusion_smooth_group_amd import workloads as wl
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


def _pair_small(M, K, H, dtype, rank, lora, seed, fmt=o.MXFP4):
    fc1 = wl.small_spec(f"chain_fc1_{M}x{K}x{H}", M, K, H, dtype, fmt, rank, seed=(300 + seed, 0))
    fc2 = wl.small_spec(f"chain_fc2_{M}x{H}x{K}", M, H, K, dtype, fmt, rank, lora_rank=lora,
                        x_dist="gelu_of_fc1", seed=(300 + seed, 1))
    d1 = wl.generate(fc1)
    return d1, wl.generate(fc2, fc1_inputs=d1)


def _pack(d, rank, lora, fmt=o.MXFP4):
    dev = G.device()
    dt = d["dtype"]
    # calibration on the layer's own (unquantized) input sample
    am = G.calib_absmax_gpu(S.bits_to_device(d["X"], G.DTS[dt], dev), dt)
    lin = G.pack_gpu(d, fmt, rank, cap=rank + lora, absmax=am)
    if lora:
        lin.attach_lora(d["lora_A"], d["lora_B"], 1.0)
    return lin


def _run_pair(d1, d2, rank, lora, rows=None, cols=None, store_y1=True, fmt=o.MXFP4):
    import torch
    dev = G.device()
    dt = d1["dtype"]
    M = d1["X"].shape[0]
    lin1 = _pack(d1, rank, 0, fmt)
    lin2 = _pack(d2, rank, lora, fmt)
    X = S.bits_to_device(d1["X"], G.DTS[dt], dev)
    # unchained on the GPU: fc1 stores Y1, fc2's activation kernel reads it
    Y1u = lin1.forward(X, gelu=True)
    ws2u = torch.empty_like(lin2.workspace(M))
    lin2.quantize_activations(Y1u, ws=ws2u)
    torch.cuda.synchronize()
    ref = lin2.workspace_export(M, ws=ws2u)
    # chained
    Y1c = torch.full_like(Y1u, 0.0) if store_y1 else None
    ws2c = torch.empty_like(ws2u)
    lin1.forward_chain(lin2, X, gelu=True, Y=Y1c, ws_next=ws2c)
    Y2c = torch.empty((M, lin2.N), dtype=X.dtype, device=dev)
    lin2.gemm(M, Y2c, ws2c)
    torch.cuda.synchronize()
    got = lin2.workspace_export(M, ws=ws2c)
    assert np.array_equal(got["codes"], ref["codes"]), "chained activation codes"
    assert np.array_equal(got["scales"], ref["scales"]), "chained activation scales"
    Tg, Tr = o.decode16(got["T"], dt), o.decode16(ref["T"], dt)
    if Tr.size:
        tol = np.abs(Tr).max() * (2.0 ** -7 if dt == o.BF16 else 2.0 ** -10) + 1e-30
        assert np.abs(Tg - Tr).max() <= tol, "chained down-projection T"
    if store_y1:
        assert np.array_equal(S.device_to_bits(Y1c), S.device_to_bits(Y1u)), "chained fc1 output"
    # oracle composition on sampled tokens: fc1 over all of its columns, then fc2
    rows = np.arange(M) if rows is None else rows
    ex1, ex2 = lin1.export(), lin2.export()
    layer1 = G.oracle_layer_from_export(ex1, d1["W"], dt, fmt, rank, d1["bias"])
    Y1r = o.forward(layer1, np.ascontiguousarray(d1["X"][rows]), gelu=True)
    if store_y1:
        G.compare_outputs(S.device_to_bits(Y1c)[rows], Y1r, dt, what="chained fc1")
    cols_all = np.arange(lin2.N) if cols is None else cols
    layer2 = G.oracle_layer_from_export(ex2, d2["W"], dt, fmt, rank, d2["bias"], cols)
    Y2r = o.forward(layer2, Y1r)
    return G.compare_outputs(S.device_to_bits(Y2c)[np.ix_(rows, cols_all)], Y2r, dt, what="chained fc2")


@pytest.mark.parametrize("fmt", [o.MXFP4, o.INT4])
@pytest.mark.parametrize("dtype", [o.BF16, o.F16])
def test_chain_small_full_parity(dtype, fmt):
    # ragged tokens (200 of a 256-row tile), fc1 N = 640 (a half-filled last
    # 256-column tile for MXFP4; five 128-column tiles for INT4), fc2 with
    # rank 16 + LoRA 16
    d1, d2 = _pair_small(200, 256, 640, dtype, 16, 16, seed=1, fmt=fmt)
    _run_pair(d1, d2, 16, 16, fmt=fmt)


@pytest.mark.parametrize("fmt", [o.MXFP4, o.INT4])
def test_chain_without_storing_fc1_output(fmt):
    d1, d2 = _pair_small(96, 384, 512, o.BF16, 16, 0, seed=2, fmt=fmt)
    _run_pair(d1, d2, 16, 0, store_y1=False, fmt=fmt)


@pytest.mark.parametrize("fmt", [o.MXFP4, o.INT4])
def test_chain_next_rank_zero(fmt):
    # fc2 without a low-rank branch: no partials, no T
    d1, d2 = _pair_small(64, 256, 384, o.BF16, 0, 0, seed=3, fmt=fmt)
    _run_pair(d1, d2, 0, 0, fmt=fmt)


def test_chain_int4_wide_branch():
    # INT4 pair, fc2 with rank 64 + LoRA 32 (three 32-rank chunks of T, six
    # 16-column tiles per partial), 300 tokens over two 256-row workspace tiles
    d1, d2 = _pair_small(300, 384, 768, o.BF16, 64, 32, seed=5, fmt=o.INT4)
    _run_pair(d1, d2, 64, 32, fmt=o.INT4)


def test_chain_rejects_mismatched_layers():
    import torch
    d1, d2 = _pair_small(32, 256, 384, o.BF16, 16, 0, seed=4)
    lin1 = _pack(d1, 16, 0)
    lin2 = _pack(d2, 16, 0)
    X = S.bits_to_device(d1["X"], S.BF16, G.device())
    with pytest.raises(S.SvdqError) as e:
        lin2.forward_chain(lin2, S.bits_to_device(d2["X"], S.BF16, G.device()))   # 384 -> 256 into K = 384
    assert e.value.code == 2
    d3 = dict(d2)
    lin3 = G.pack_gpu(d3, o.INT4, 16)
    with pytest.raises(S.SvdqError) as e:
        lin1.forward_chain(lin3, X)      # MXFP4 into INT4: mixed pairs are not chained
    assert e.value.code == 3
    # a first-layer workspace one byte short of the chained size
    need = S._SZ(0)
    S._call("svdq_chain_workspace_size", S.C.byref(lin1.layer), S.C.byref(lin2.layer), 32, S.C.byref(need))
    ws = torch.empty(need.value - 1, dtype=torch.uint8, device=G.device())
    with pytest.raises(S.SvdqError) as e:
        lin1.forward_chain(lin2, X, ws=ws)
    assert e.value.code == 4


@pytest.mark.parametrize("fmt", [o.MXFP4, o.INT4])
def test_chain_flux_mlp_pair_sampled(fmt):
    fc1, fc2 = wl.config_shapes(3)
    d1 = wl.generate(fc1)
    d2 = wl.generate(fc2, fc1_inputs=d1)
    rows = wl.random_rows(fc1.M, 24, 71)
    cols = np.sort(np.random.default_rng(72).choice(fc2.N, size=256, replace=False))
    _run_pair(d1, d2, 32, 0, rows=rows, cols=cols, fmt=fmt)
