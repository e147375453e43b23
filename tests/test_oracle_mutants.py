"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case swaps one oracle function for a plausible wrong variant (a
dropped term, a wrong rounding rule, a flipped orientation, a transposed
operand) and checks that at least one pin then fails.
"""
import numpy as np
import pytest

import oracle
import oracle.svdquant as osq
from tests import test_oracle_quant as tq
from tests import test_oracle_split as ts
from tests import test_oracle_gelu_lora as tg


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(osq, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _expect_fail(*pins):
    failed = 0
    for pin, args in pins:
        try:
            pin(*args)
        except AssertionError:
            failed += 1
    assert failed > 0, "planted mistake went unnoticed"


def test_mutant_int4_round_half_away(monkeypatch):
    orig = osq.quant_int4_g64

    def bad(v):
        q, s = orig(v)
        s32 = s.view(np.float16).astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            r = (np.asarray(v, np.float32) / s32[..., None]).astype(np.float32)
        qa = np.clip(np.sign(r) * np.floor(np.abs(r) + 0.5), -7, 7)
        qa = np.where(s32[..., None] == 0, 0, np.nan_to_num(qa))
        return qa.astype(np.int8), s
    _patch(monkeypatch, "quant_int4_g64", bad)
    _expect_fail((tq.test_int4_worked_example, ()), (tq.test_int4_against_scalar_restatement, (1.0,)))


def test_mutant_mxfp4_floor_scale(monkeypatch):
    orig = osq.quant_mxfp4_g32

    def bad(v):
        v = np.asarray(v, np.float32)
        m = np.max(np.abs(v), -1).astype(np.float32)
        t = (m / np.float32(6)).astype(np.float32)
        e = ((t.view(np.uint32) >> 23) & 0xFF).astype(np.int64)   # floor exponent, no round-up
        u = np.ldexp(v, (127 - e)[..., None].astype(np.int32)).astype(np.float32)
        idx = osq._e2m1_nearest_even(np.abs(u))
        return (idx | (np.signbit(v).astype(np.uint8) << 3)).astype(np.uint8), e.astype(np.uint8)
    _patch(monkeypatch, "quant_mxfp4_g32", bad)
    _expect_fail((tq.test_mxfp4_worked_examples, ("mxfp4_g32_scale_up.txt",)),
                 (tq.test_mxfp4_scale_is_smallest_power_of_two_covering, ()))


def test_mutant_residual_drops_lambda(monkeypatch):
    def bad(W, lam, L1x, L2q):
        W = np.asarray(W, np.float64); lam64 = np.asarray(lam, np.float64)
        s = np.asarray(L1x, np.float64) @ np.asarray(L2q, np.float64)
        return (lam64[:, None] * W - s).astype(np.float32)
    _patch(monkeypatch, "residual", bad)
    _expect_fail((ts.test_residual_reconstructs_to_fp32_rounding, ()))


def test_mutant_svd_drops_sigma(monkeypatch):
    def bad(W_hat, r):
        U, S, Vt = np.linalg.svd(W_hat, full_matrices=False)
        return U[:, :r].copy(), Vt[:r].copy(), S
    _patch(monkeypatch, "truncated_svd", bad)
    _expect_fail((ts.test_eckart_young_mirsky, ((128, 96),)))


def test_mutant_smoothing_inverted(monkeypatch):
    orig = osq.smoothing_factors

    def bad(a, w):
        lam, inv = orig(a, w)
        return inv, lam
    _patch(monkeypatch, "smoothing_factors", bad)
    _expect_fail((ts.test_smoothing_balances_channel_maxima, ()))


def test_mutant_forward_drops_up_projection(monkeypatch):
    def bad(Y_main, T, L2q, bias, gelu):
        Y = np.asarray(Y_main, np.float64)
        if bias is not None:
            Y = Y + np.asarray(bias, np.float64)[None, :]
        return Y
    _patch(monkeypatch, "output_epilogue_f64", bad)
    _expect_fail((ts.test_brute_force_tiny, (oracle.INT4, 64, oracle.F16)))


def test_mutant_mx_scales_wrong_axis(monkeypatch):
    orig = osq.dequant_weight

    def bad(q, s, fmt):
        if fmt != oracle.MXFP4:
            return orig(q, s, fmt)
        s2 = np.ascontiguousarray(s[::-1])       # group scales applied to the wrong K-groups
        return orig(q, s2, fmt)
    _patch(monkeypatch, "dequant_weight", bad)
    _expect_fail((ts.test_brute_force_tiny, (oracle.MXFP4, 128, oracle.BF16)))


def test_mutant_int4_partial_sign(monkeypatch):
    orig = osq.int4_group_partials

    def bad(qx, qw):
        P = orig(qx, qw)
        P[-1] = -P[-1]                            # wrong sign on one group
        return P
    _patch(monkeypatch, "int4_group_partials", bad)
    _expect_fail((ts.test_brute_force_tiny, (oracle.INT4, 128, oracle.F16)),
                 (ts.test_rank0_unit_lambda_is_naive_w4a4, ()))


_GELU_PINS = ((tg.test_gelu_closed_values, ()), (tg.test_gelu_matches_quadrature_of_the_density, ()),
              (tg.test_gelu_odd_part_is_identity, ()), (tg.test_gelu_slope_at_zero_and_derivative, ()),
              (tg.test_gelu_tails, ()))


def test_mutant_gelu_tanh_form(monkeypatch):
    def bad(x):
        x = np.asarray(x, np.float64)
        return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))
    _patch(monkeypatch, "gelu_erf", bad)
    _expect_fail(*_GELU_PINS)


def test_mutant_gelu_wrong_sqrt2(monkeypatch):
    from scipy.special import erf

    def bad(x):
        x = np.asarray(x, np.float64)
        return 0.5 * x * (1.0 + erf(x / 2.0))
    _patch(monkeypatch, "gelu_erf", bad)
    _expect_fail(*_GELU_PINS)


def _lora_pins():
    return tuple((tg.test_lora_adds_exactly_its_own_product_on_raw_x, (a,)) for a in (1.0, 0.3, -1.7)) + \
        ((tg.test_lora_leaves_residual_and_branch_untouched, ()),)


def test_mutant_lora_alpha_on_a(monkeypatch):
    def bad(layer, A_bits, B_bits, alpha=1.0):
        dt = layer["dtype"]
        A, B = osq.decode16(A_bits, dt), osq.decode16(B_bits, dt)
        out = dict(layer)
        out["L1x"] = np.concatenate([layer["L1x"], osq.round16(float(alpha) * A, dt)], axis=1)
        out["L2q"] = np.concatenate([layer["L2q"], osq.round16(B, dt)], axis=0)
        return out
    _patch(monkeypatch, "attach_lora", bad)
    _expect_fail(*_lora_pins())


def test_mutant_lora_on_smoothed_input(monkeypatch):
    def bad(layer, A_bits, B_bits, alpha=1.0):
        dt = layer["dtype"]
        A, B = osq.decode16(A_bits, dt), osq.decode16(B_bits, dt)
        out = dict(layer)
        Ah = np.asarray(layer["invlam"], np.float64)[:, None] * A     # LoRA applied to X_hat
        out["L1x"] = np.concatenate([layer["L1x"], osq.round16(Ah, dt)], axis=1)
        out["L2q"] = np.concatenate([layer["L2q"], osq.round16(float(alpha) * B, dt)], axis=0)
        return out
    _patch(monkeypatch, "attach_lora", bad)
    _expect_fail(*_lora_pins())
