"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and evaluate the oracle on the same seeded inputs (given the library's
exported factors, because a truncated SVD is not unique)."""
from __future__ import annotations

import numpy as np

import oracle as o
from diffusion_smooth_group_amd import svdq as S
from diffusion_smooth_group_amd import workloads as wl

FMTS = {o.INT4: S.FMT_INT4_G64, o.MXFP4: S.FMT_MXFP4_G32, o.INT8: S.FMT_INT8_W8A8}
DTS = {o.F16: S.F16, o.BF16: S.BF16}

# Output gate (floating point): relative Frobenius error <= 5e-3 and
# max |dY| <= 1e-2 max |Y| against the oracle's float64 forward.
REL_FRO = 5e-3
REL_MAX = 1e-2


def device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def calib_absmax_gpu(Xd, dtype):
    """Per-channel max |X| with the library's calibration kernel."""
    import torch
    a = S.activation_absmax(Xd, DTS[dtype])
    torch.cuda.synchronize()
    return a.cpu().numpy()


def pack_gpu(d, fmt, rank, cap=None, absmax=None, refine=0):
    dt = d["dtype"]
    lin = S.SVDQLinear.pack(d["W"], DTS[dt], absmax, rank, FMTS[fmt], d["bias"], rank_capacity=cap,
                            refine_iters=refine)
    return lin


def oracle_layer_from_export(ex, W_bits, dtype, fmt, rank, bias_bits, cols=None):
    """Oracle layer for the library's lambda / 16-bit factors; with `cols`
    only those output columns (every step is column-local on the weight side)."""
    W = W_bits if cols is None else np.ascontiguousarray(W_bits[:, cols])
    L2q = ex["L2q"] if cols is None else np.ascontiguousarray(ex["L2q"][:, cols])
    pf = o.pack_from_factors(W, dtype, ex["lam"], ex["L1x"][:, :rank], L2q[:rank], fmt)
    bias = None
    if bias_bits is not None:
        bias = bias_bits if cols is None else bias_bits[cols]
    return {"dtype": dtype, "fmt": fmt, "lam": ex["lam"], "invlam": ex["invlam"], "L1x": ex["L1x"],
            "L2q": L2q, "qw": pf["qw"], "sw": pf["sw"], "bias": bias}


def compare_outputs(Y_gpu_bits, Y_ref_bits, dtype, what=""):
    Yg = o.decode16(Y_gpu_bits, dtype)
    Yr = o.decode16(Y_ref_bits, dtype)
    assert np.all(np.isfinite(Yg)), f"{what}: non-finite GPU output"
    fro = np.linalg.norm(Yg - Yr) / max(np.linalg.norm(Yr), 1e-30)
    mx = np.abs(Yg - Yr).max() / max(np.abs(Yr).max(), 1e-30)
    assert fro <= REL_FRO, f"{what}: relative Frobenius error {fro:.3e} > {REL_FRO}"
    assert mx <= REL_MAX, f"{what}: max error {mx:.3e} of max|Y| > {REL_MAX}"
    return fro, mx


def run_layer_case(d, fmt, rank, lora=False, gelu=False, rows=None, cols=None, cap=None, alpha=1.0,
                   check_codes=True, unfused=False, refine=0):
    """Pack on the GPU, run the forward, and compare with the oracle.
    rows / cols: sample of outputs evaluated by the oracle (None = all)."""
    import torch
    dev = device()
    dt = d["dtype"]
    M, K = d["X"].shape
    Xd = S.bits_to_device(d["X"], DTS[dt], dev)
    absmax = calib_absmax_gpu(Xd, dt)
    ref_absmax = o.activation_absmax(o.decode16(d["X"], dt))
    assert np.array_equal(absmax.view(np.uint32), ref_absmax.view(np.uint32)), "calibration absmax"
    lin = pack_gpu(d, fmt, rank, cap=cap if cap is not None else (rank + (d["lora_A"].shape[1] if lora else 0)),
                   absmax=absmax, refine=refine)
    if lora:
        lin.attach_lora(d["lora_A"], d["lora_B"], alpha)
    Y = lin.forward(Xd, gelu=gelu, unfused=unfused)
    torch.cuda.synchronize()
    Yb = S.device_to_bits(Y)
    ex = lin.export()
    rows_sampled = rows is not None
    if rows is None:
        rows = np.arange(M)
    if cols is None:
        cols_sel = None
        cols = np.arange(d["W"].shape[1])
    else:
        cols_sel = cols
    layer = oracle_layer_from_export(ex, d["W"], dt, fmt, rank, d["bias"], cols_sel)
    Xr = np.ascontiguousarray(d["X"][rows])
    Yr, parts = o.forward(layer, Xr, gelu=gelu, return_parts=True)
    fro, mx = compare_outputs(Yb[np.ix_(rows, cols)], Yr, dt, what=f"{d['spec'].name} {fmt}")
    if check_codes:
        wx = lin.workspace_export(M)
        assert np.array_equal(wx["codes"][rows].astype(np.int64), np.asarray(parts["qx"], np.int64)), "activation codes"
        assert np.array_equal(wx["scales"][rows], parts["sx"]), "activation scales"
        Tg = o.decode16(wx["T"][rows], dt)
        Tr = o.decode16(parts["T"], dt)
        if Tr.size:
            # T is rounded to 16 bits once from an fp32 (GPU) / fp64 (oracle) sum
            tol = np.abs(Tr).max() * (2.0 ** -7 if dt == o.BF16 else 2.0 ** -10) + 1e-30
            assert np.abs(Tg - Tr).max() <= tol, "down-projection T"
        if rows_sampled:
            # the activation pass is row-local and cheap to evaluate: codes,
            # scales and T on many more rows than the output sample (every
            # row where the oracle's quantizer is fast enough)
            wide = np.arange(M) if (fmt != o.MXFP4 and M * K <= (1 << 26)) else \
                np.union1d(rows, wl.random_rows(M, min(M, 1024), 97))
            Xw = o.decode16(np.ascontiguousarray(d["X"][wide]), dt)
            qa, sa, _ = o.quantize_activations(Xw, ex["invlam"], fmt)
            assert np.array_equal(wx["codes"][wide].astype(np.int64), np.asarray(qa, np.int64)), \
                f"activation codes ({len(wide)} rows)"
            assert np.array_equal(wx["scales"][wide], sa), f"activation scales ({len(wide)} rows)"
            Ta = o.decode16(o.down_projection(Xw, o.decode16(layer["L1x"], dt), dt), dt)
            Tw = o.decode16(wx["T"][wide], dt)
            if Ta.size:
                tol = np.abs(Ta).max() * (2.0 ** -7 if dt == o.BF16 else 2.0 ** -10) + 1e-30
                assert np.abs(Tw - Ta).max() <= tol, f"down-projection T ({len(wide)} rows)"
    return lin, {"fro": fro, "max": mx, "Y": Yb}
