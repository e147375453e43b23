"""The C-ABI library on the host (no GPU): symbols, error paths, and the
offline pack against the oracle.

Bit-exact gates (given the library's own factors, since a truncated SVD is
not unique): lambda, 1/lambda, the 16-bit rounding of the factors, the
residual codes and scales.  The library's SVD is checked against the
Eckart-Young-Mirsky optimum computed by the oracle's LAPACK SVD.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle as o
from diffusion_smooth_group_amd import svdq as S
from diffusion_smooth_group_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "svdq.h")
FMTS = {o.INT4: S.FMT_INT4_G64, o.MXFP4: S.FMT_MXFP4_G32, o.INT8: S.FMT_INT8_W8A8}
DTS = {o.F16: S.F16, o.BF16: S.BF16}


def _declared():
    txt = open(HDR).read()
    return sorted(set(re.findall(r"^(?:svdq_status|const char\*)\s+(svdq_\w+)\s*\(", txt, re.M)))


def test_library_exports_every_declared_symbol():
    lib = S.lib_handle()
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert lib.svdq_status_string(0) == b"ok"
    assert lib.svdq_status_string(6) == b"HIP runtime error"


def test_packed_size_and_shape_errors():
    assert S.packed_size(3072, 12288, 32, S.FMT_INT4_G64, S.BF16) > 3072 * 12288 // 2
    for args, code in [((100, 128, 32, 0, 0), 2), ((128, 100, 32, 0, 0), 2), ((128, 128, 129, 0, 0), 1),
                       ((128, 128, 32, 5, 0), 1), ((128, 128, 32, 0, 7), 1), ((0, 128, 32, 0, 0), 2)]:
        with pytest.raises(S.SvdqError) as e:
            S.packed_size(*args)
        assert e.value.code == code


def _inputs(K=256, N=384, M=64, dtype=o.BF16, seed=0, w_out=2):
    spec = wl.small_spec("t", M, K, N, dtype, o.INT4, 8, x_outliers=3, w_outliers=w_out, seed=(seed, 0))
    return wl.generate(spec)


def test_pack_error_paths():
    d = _inputs()
    W = d["W"]
    a = o.activation_absmax(o.decode16(d["X"], o.BF16))
    with pytest.raises(S.SvdqError) as e:          # rank above capacity
        S.pack_weights_host(W, S.BF16, a, 40, 32, S.FMT_INT4_G64)
    assert e.value.code == 1
    with pytest.raises(S.SvdqError) as e:          # K not a multiple of 128
        S.pack_weights_host(W[:200], S.BF16, a[:200], 8, 8, S.FMT_INT4_G64)
    assert e.value.code == 2
    Wn = W.copy()
    Wn[3, 5] = 0x7FC0                               # NaN weight
    with pytest.raises(S.SvdqError) as e:
        S.pack_weights_host(Wn, S.BF16, a, 8, 8, S.FMT_INT4_G64)
    assert e.value.code == 5
    an = a.copy()
    an[0] = np.inf
    with pytest.raises(S.SvdqError) as e:
        S.pack_weights_host(W, S.BF16, an, 8, 8, S.FMT_INT4_G64)
    assert e.value.code == 5
    # blob too small
    L = S.svdq_layer()
    blob = np.zeros(1024, np.uint8)
    rc = S.lib_handle().svdq_pack_weights_host(S._np_ptr(W), 256, 384, 384, S.BF16, S._np_ptr(a), 8, 8, 0, None,
                                               S._np_ptr(blob), blob.size, C.byref(L))
    assert rc == 4
    # null weight pointer
    rc = S.lib_handle().svdq_pack_weights_host(None, 256, 384, 384, S.BF16, None, 8, 8, 0, None,
                                               S._np_ptr(blob), blob.size, C.byref(L))
    assert rc == 1


def test_lora_capacity_and_forward_arg_errors():
    d = _inputs()
    L, blob = S.pack_weights_host(d["W"], S.BF16, None, 8, 16, S.FMT_MXFP4_G32)
    A = np.zeros((256, 9), np.uint16)
    B = np.zeros((9, 384), np.uint16)
    with pytest.raises(S.SvdqError) as e:
        S.attach_lora(L, A, B)
    assert e.value.code == 4
    lib = S.lib_handle()
    # forward on a host blob is refused before any launch
    ws = np.zeros(1 << 20, np.uint8)
    rc = lib.svdq_linear_forward(C.byref(L), S._np_ptr(ws), 16, 256, S._np_ptr(ws), 384, S._np_ptr(ws), ws.size, 0,
                                 None)
    assert rc == 1
    assert lib.svdq_workspace_size(C.byref(L), -1, C.byref(C.c_size_t())) == 1
    assert S.workspace_size(L, 1) >= 256 * 256 // 2
    # chaining also needs device layers; nothing is launched
    assert lib.svdq_chain_workspace_size(C.byref(L), C.byref(L), 16, C.byref(C.c_size_t())) == 1
    rc = lib.svdq_linear_forward_chain(C.byref(L), C.byref(L), S._np_ptr(ws), 16, 256, None, 0, S._np_ptr(ws),
                                       ws.size, S._np_ptr(ws), ws.size, 0, None)
    assert rc == 1


def test_kernel_timing_argument_checks():
    # no GPU call is made on these paths
    lib = S.lib_handle()
    assert lib.svdq_timing_start(0) == 1
    assert lib.svdq_timing_start((1 << 20) + 1) == 1
    n = C.c_int(-1)
    assert lib.svdq_timing_stop(None, None, 0, C.byref(n)) == 0 and n.value == 0   # stop without start
    assert lib.svdq_timing_stop(None, None, 1, C.byref(n)) == 1
    assert lib.svdq_timing_stop(None, None, -1, C.byref(n)) == 1
    assert lib.svdq_timing_stop(None, None, 0, None) == 1


@pytest.mark.parametrize("dtype", [o.F16, o.BF16])
@pytest.mark.parametrize("fmt", [o.INT4, o.MXFP4, o.INT8])
@pytest.mark.parametrize("KN", [(256, 384), (640, 256)])
def test_host_pack_bit_exact_given_factors(dtype, fmt, KN):
    K, N = KN
    d = _inputs(K=K, N=N, dtype=dtype, seed=K + N)
    X = o.decode16(d["X"], dtype)
    a = o.activation_absmax(X)
    r = 16
    L, blob = S.pack_weights_host(d["W"], DTS[dtype], a, r, 32, FMTS[fmt], d["bias"])
    ex = S.layer_export(L)
    lam, invlam = o.smoothing_factors(a, o.weight_channel_absmax(o.decode16(d["W"], dtype)))
    assert np.array_equal(ex["lam"].view(np.uint32), lam.view(np.uint32))
    assert np.array_equal(ex["invlam"].view(np.uint32), invlam.view(np.uint32))
    # 16-bit factors are the one-step rounding of the library's fp64 factors
    L1, L2, sg, lam2 = S.svd_factors(d["W"], DTS[dtype], a, r)
    assert np.array_equal(lam2.view(np.uint32), lam.view(np.uint32))
    l1x, l2q = o.runtime_factors(L1, L2, invlam, dtype)
    assert np.array_equal(ex["L1x"], l1x) and np.array_equal(ex["L2q"], l2q)
    # residual codes and scales, recomputed by the oracle from the library's factors
    pf = o.pack_from_factors(d["W"], dtype, ex["lam"], ex["L1x"], ex["L2q"], fmt)
    assert np.array_equal(ex["codes"].astype(np.int64), pf["qw"].astype(np.int64))
    assert ex["scales"].shape == pf["sw"].shape
    assert np.array_equal(np.ascontiguousarray(ex["scales"]).view(np.uint8), np.ascontiguousarray(pf["sw"]).view(np.uint8))
    assert np.array_equal(ex["bias"], o.decode16(d["bias"], dtype).astype(np.float32))


@pytest.mark.parametrize("KN,r", [((256, 384), 16), ((640, 256), 32), ((384, 384), 48), ((128, 1024), 64)])
def test_library_svd_reaches_eckart_young_mirsky(KN, r):
    K, N = KN
    d = _inputs(K=K, N=N, seed=3 * K + N, w_out=3)
    X = o.decode16(d["X"], o.BF16)
    a = o.activation_absmax(X)
    L1, L2, sg, lam = S.svd_factors(d["W"], S.BF16, a, r)
    What = o.smoothed_weight(o.decode16(d["W"], o.BF16), lam)
    _, _, s_ref = o.truncated_svd(What, r)
    assert np.allclose(sg, s_ref[:r], rtol=1e-9)
    Rr = What - L1 @ L2
    spec = np.linalg.norm(Rr, 2)
    assert abs(spec / s_ref[r] - 1) < 1e-6
    assert abs(np.sum(Rr ** 2) / np.sum(s_ref[r:] ** 2) - 1) < 1e-8


def test_svd_rank_deficient_and_repeated_singular_values():
    # exact repeated singular values (orthogonal columns of equal norm) and rank < r
    K, N, r = 128, 256, 8
    W = np.zeros((K, N), np.float32)
    for i in range(5):
        W[i, 3 * i] = 0.5            # five equal singular values, rank 5 < r
    Wb = wl.f32_to_bits16(W, o.F16)
    L1, L2, sg, lam = S.svd_factors(Wb, S.F16, None, r)
    assert np.allclose(sg[:5], 0.5, rtol=1e-12) and np.all(sg[5:] == 0)
    assert np.allclose(L1 @ L2, W.astype(np.float64), atol=1e-12)


def test_lora_attach_detach_and_copy_on_host():
    d = _inputs(K=256, N=384, dtype=o.F16, seed=9)
    a = o.activation_absmax(o.decode16(d["X"], o.F16))
    L, blob = S.pack_weights_host(d["W"], S.F16, a, 16, 40, S.FMT_INT4_G64)
    ex0 = S.layer_export(L)
    rng = np.random.default_rng(1)
    A = wl.f32_to_bits16((rng.standard_normal((256, 20)) * 0.02).astype(np.float32), o.F16)
    B = wl.f32_to_bits16((rng.standard_normal((20, 384)) * 0.02).astype(np.float32), o.F16)
    S.attach_lora(L, A, B, 0.75)
    assert L.rank_active == 36
    ex1 = S.layer_export(L)
    ref = o.attach_lora({"dtype": o.F16, "L1x": ex0["L1x"], "L2q": ex0["L2q"]}, A, B, 0.75)
    assert np.array_equal(ex1["L1x"], ref["L1x"]) and np.array_equal(ex1["L2q"], ref["L2q"])
    assert np.array_equal(ex1["codes"], ex0["codes"]) and np.array_equal(ex1["scales"], ex0["scales"])
    # the blob moves by copying its bytes
    blob2 = np.zeros_like(blob)
    L2 = S.layer_copy(L, S._np_ptr(blob2), blob2.size, False)
    ex2 = S.layer_export(L2)
    for k in ex1:
        assert np.array_equal(ex1[k], ex2[k])
    S.detach_lora(L)
    assert L.rank_active == 16
    ex3 = S.layer_export(L)
    assert np.array_equal(ex3["L1x"], ex0["L1x"]) and np.array_equal(ex3["L2q"], ex0["L2q"])
    # re-attach a smaller LoRA after a larger one: stale slots are cleared
    S.attach_lora(L, A[:, :4], B[:4], 1.0)
    assert L.rank_active == 20
    raw_l1 = np.zeros((256, 20), np.uint16)
    assert np.array_equal(S.layer_export(L)["L1x"][:, 16:], A[:, :4])


def test_config1_full_pack_matches_oracle():
    """The 256 x 1152 -> 1152 fp16 INT4 layer at its full size."""
    spec = wl.config_shapes(1)[0]
    d = wl.generate(spec)
    X = o.decode16(d["X"], o.F16)
    a = o.activation_absmax(X)
    L, blob = S.pack_weights_host(d["W"], S.F16, a, 32, 32, S.FMT_INT4_G64)
    ex = S.layer_export(L)
    pf = o.pack_from_factors(d["W"], o.F16, ex["lam"], ex["L1x"], ex["L2q"], o.INT4)
    assert np.array_equal(ex["codes"].astype(np.int64), pf["qw"].astype(np.int64))
    assert np.array_equal(ex["scales"], pf["sw"])
    ref = o.pack(d["W"], o.F16, a, 32, o.INT4)
    # same split quality as LAPACK (the bases may differ in sign / degenerate directions)
    What = o.smoothed_weight(o.decode16(d["W"], o.F16), ref["lam"])
    L1, L2, sg, _ = S.svd_factors(d["W"], S.F16, a, 32)
    assert abs(np.linalg.norm(What - L1 @ L2, 2) / ref["sigma"][32] - 1) < 1e-6


# ------------------------------------------------ low-rank split refinement
@pytest.mark.parametrize("fmt", [o.INT4, o.MXFP4])
def test_refined_pack_against_oracle(fmt):
    K, N, dt, r = 256, 384, o.BF16, 16
    d = _inputs(K=K, N=N, dtype=dt, seed=70, w_out=3)
    a = o.activation_absmax(o.decode16(d["X"], dt))
    # zero rounds: byte for byte the plain pack, and its error is the oracle's
    L0, b0 = S.pack_weights_host(d["W"], DTS[dt], a, r, 32, FMTS[fmt], d["bias"])
    e0 = np.zeros(1, np.float64)
    L1, b1 = S.pack_weights_host(d["W"], DTS[dt], a, r, 32, FMTS[fmt], d["bias"], refine_iters=0, errors=e0)
    assert np.array_equal(b0, b1)
    ex = S.layer_export(L1)
    ref0 = o.split_error(d["W"], dt, ex["lam"], ex["L1x"], ex["L2q"], ex["codes"], ex["scales"], fmt)
    assert abs(e0[0] - ref0) <= 1e-9 * ref0
    # three rounds: the packed split is the one with the smallest reported
    # error, its codes follow from its factors, and its error is the oracle's
    it = 3
    errs = np.zeros(it + 1, np.float64)
    L3, b3 = S.pack_weights_host(d["W"], DTS[dt], a, r, 32, FMTS[fmt], d["bias"], refine_iters=it, errors=errs)
    ex3 = S.layer_export(L3)
    pf = o.pack_from_factors(d["W"], dt, ex3["lam"], ex3["L1x"], ex3["L2q"], fmt)
    assert np.array_equal(ex3["codes"].astype(np.int64), pf["qw"].astype(np.int64))
    assert np.array_equal(ex3["scales"], pf["sw"])
    ref3 = o.split_error(d["W"], dt, ex3["lam"], ex3["L1x"], ex3["L2q"], ex3["codes"], ex3["scales"], fmt)
    assert abs(errs.min() - ref3) <= 1e-9 * ref3
    assert abs(errs[0] - ref0) <= 1e-9 * ref0
    assert errs.min() < errs[0]
    # the oracle's own refinement (LAPACK SVD) follows the same trajectory
    # up to the SVDs' last bits: same one-shot error, best error within 2%
    orc = o.refine_split(d["W"], dt, a, r, fmt, it)
    oerr = [x["err"] for x in orc["rounds"]]
    assert abs(oerr[0] - errs[0]) <= 1e-3 * oerr[0]
    assert abs(min(oerr) - errs.min()) <= 2e-2 * min(oerr)


def test_refine_iters_bounds():
    d = _inputs()
    a = o.activation_absmax(o.decode16(d["X"], o.BF16))
    for bad in (-1, 17):
        with pytest.raises(S.SvdqError) as e:
            S.pack_weights_host(d["W"], S.BF16, a, 8, 8, S.FMT_INT4_G64, refine_iters=bad)
        assert e.value.code == 1
