"""The GEMM trace (SVDQ_FLAG_TRACE) and the clock / matrix-rate probes:
tracing leaves every output bit unchanged, records one entry per GEMM
workgroup with consistent counters, and the probes report physically
possible values (the dense FP4 rate can not exceed the chip's peak at the
clock the probe itself measured)."""
import ctypes as C

import numpy as np
import pytest

import oracle as o
from diffusion_smooth_group_amd import svdq as S
from diffusion_smooth_group_amd import workloads as wl
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt,gelu", [(o.MXFP4, False), (o.MXFP4, True), (o.INT4, False), (o.INT8, True)])
def test_trace_keeps_outputs_and_records_every_workgroup(fmt, gelu):
    import torch
    spec = wl.small_spec("trace", 700, 512, 768, o.BF16, fmt, 16, lora_rank=8, seed=(950, 0))
    d = wl.generate(spec)
    Xd = S.bits_to_device(d["X"], S.BF16, G.device())
    lin = G.pack_gpu(d, fmt, 16, cap=24, absmax=G.calib_absmax_gpu(Xd, o.BF16))
    lin.attach_lora(d["lora_A"], d["lora_B"], 1.0)
    Y0 = lin.forward(Xd, gelu=gelu)
    ws = lin.workspace(700)
    Y1 = torch.empty_like(Y0)
    lib = S.lib_handle()
    flags = S.FLAG_TRACE | (S.FLAG_GELU if gelu else 0)
    rc = lib.svdq_linear_forward(C.byref(lin.layer), S._t_ptr(Xd), 700, 512, S._t_ptr(Y1), 768, S._t_ptr(ws),
                                 ws.numel(), flags, S._stream())
    assert rc == 0
    rec, hz = S.trace_read()
    torch.cuda.synchronize()
    assert np.array_equal(S.device_to_bits(Y0), S.device_to_bits(Y1))
    assert hz > 0 and len(rec) > 0
    r = rec.astype(np.int64)
    assert np.all(r[:, 2] > r[:, 0]) and np.all(r[:, 3] > r[:, 1])
    mhz = (r[:, 3] - r[:, 1]).sum() / (r[:, 2] - r[:, 0]).sum() * hz * 1e-6
    assert 100.0 < mhz < 3000.0
    # workgroups of the launch: the tile grid of the format's GEMM
    Mp = -(-700 // 256) * 256
    expect = {o.INT4: (768 // 128) * (Mp // 128), o.INT8: -(-768 // 256) * (Mp // 256),
              o.MXFP4: (-(-768 // 192) * -(-Mp // 192)) if gelu else (-(-768 // 256) * (Mp // 256))}[fmt]
    assert len(rec) == expect


def test_probes_are_physical():
    clk = S.probe_clock()
    assert 100.0 < clk < 3000.0
    for rnd in (True, False):
        tf, mhz = S.probe_mfma_rate(rnd, 500)
        assert 100.0 < mhz < 3000.0
        # dense FP4: 4096 flops per SIMD per clock, 1024 SIMDs
        assert 0.0 < tf <= 4096 * 1024 * mhz * 1e6 * 1e-12 * 1.02, (tf, mhz)


@pytest.mark.parametrize("fmt", [o.MXFP4, o.INT4])
def test_kernel_timing_records_each_launch(fmt):
    # svdq_timing_start / stop: every kernel of the timed forwards is
    # recorded in launch order with its kind, outputs stay bit-identical,
    # and the kernels' durations fit inside the wall time of the loop
    import torch
    spec = wl.small_spec("timing", 600, 512, 768, o.BF16, fmt, 16, seed=(951, 0))
    d = wl.generate(spec)
    Xd = S.bits_to_device(d["X"], S.BF16, G.device())
    lin = G.pack_gpu(d, fmt, 16, absmax=G.calib_absmax_gpu(Xd, o.BF16))
    Y0 = lin.forward(Xd, gelu=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    S.timing_start(5)                   # room for two forwards and one more kernel
    e0.record()
    Ys = [lin.forward(Xd, gelu=True) for _ in range(3)]
    e1.record()
    torch.cuda.synchronize()
    kinds, us = S.timing_stop()
    assert list(kinds) == [S.KERNEL_ACT, S.KERNEL_GEMM] * 2 + [S.KERNEL_ACT]   # capacity 5: the rest untimed
    assert np.all(us > 0.0)
    assert us.sum() <= e0.elapsed_time(e1) * 1e3
    for Y in Ys:
        assert np.array_equal(S.device_to_bits(Y), S.device_to_bits(Y0))
    # stopped: nothing more is recorded
    lin.forward(Xd, gelu=True)
    torch.cuda.synchronize()
    kinds, us = S.timing_stop()
    assert len(kinds) == 0
