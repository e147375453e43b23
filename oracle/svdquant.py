"""SVDQuant linear layer, restated step by step in float64 (CPU oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Citations name sections of the SVDQuant paper, "SVDQuant: Absorbing Outliers
by Low-Rank Components for 4-Bit Diffusion Models", as read in its translated
article on developer.volcengine.com ([SVDQuant §n]).  The extracted text lost
every display formula; where a step had to be reconstructed the reading is
stated next to it.

Notation (orientation of the paper's §3 / §4.1): X is M x K (tokens x input
channels), W is K x N, lambda has K entries, L1 is K x r, L2 is r x N,
R is K x N, group size G runs along K.

Every public function is pinned by tests/test_oracle_*.py against closed
forms, invariants, worked examples, an independent textbook W4A4 routine and
brute force on tiny inputs.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Tuple

import numpy as np

INT4 = "int4_g64"
MXFP4 = "mxfp4_g32"
INT8 = "int8_w8a8"    # the 8-bit setting: per-token activations, per-channel weights
F16 = "f16"
BF16 = "bf16"
GROUP = {INT4: 64, MXFP4: 32}

# E2M1 magnitudes indexed by the 3 low code bits (OCP microscaling FP4:
# 1 sign, 2 exponent, 1 mantissa bit; 0b000 = 0, 0b001 = 0.5 subnormal).
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
INT4_QMAX = 7      # signed b-bit integer: 2^(b-1) - 1 [SVDQuant §3]
INT8_QMAX = 127    # the same rule for b = 8
E2M1_QMAX = 6.0    # largest 4-bit float magnitude with 1 mantissa, 2 exponent bits [SVDQuant §3]
FP16_MAX = 65504.0

__all__ = [
    "INT4", "MXFP4", "INT8", "F16", "BF16", "GROUP", "E2M1_GRID",
    "decode16", "round16", "round_sig",
    "activation_absmax", "weight_channel_absmax", "smoothing_factors",
    "smoothed_weight", "truncated_svd", "runtime_factors", "residual",
    "quant_int4_g64", "quant_mxfp4_g32", "dequant_int4", "dequant_mxfp4", "quant_int8_row", "dequant_int8",
    "quantize_groups", "dequantize_groups",
    "quantize_weight", "quantize_activations", "dequant_weight", "dequant_activations",
    "down_projection", "int4_group_partials", "main_product", "gelu_erf", "output_epilogue",
    "output_epilogue_f64",
    "pack", "pack_from_factors", "attach_lora", "forward",
    "quantization_error", "prop41_bound", "lowrank_overhead", "packed_bytes",
    "split_error", "refine_split",
]


# ---------------------------------------------------------------------------
# 16-bit storage types
# ---------------------------------------------------------------------------
def decode16(bits: np.ndarray, dtype: str) -> np.ndarray:
    """fp16 / bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    if dtype == F16:
        return b.view(np.float16).astype(np.float64)
    if dtype == BF16:
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


_FMT16 = {  # (significand bits incl. hidden, min normal exponent, max finite)
    F16: (11, -14, 65504.0),
    BF16: (8, -126, float((2.0 - 2.0 ** -7) * 2.0 ** 127)),
}


def round_sig(x: np.ndarray, p: int, emin: int, vmax: float) -> np.ndarray:
    """Round float64 values to a binary format with p significand bits,
    minimum normal exponent emin (gradual underflow below it) and largest
    finite value vmax; round to nearest, ties to even; overflow -> +-inf.
    The rounding is done directly from float64 (no intermediate fp32)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    fin = np.isfinite(x) & (x != 0)
    ax = np.abs(x[fin])
    _, e2 = np.frexp(ax)                  # ax = f * 2^e2, f in [0.5, 1)
    e = np.maximum(e2.astype(np.int64) - 1, emin)   # exponent of the leading bit
    q = np.ldexp(1.0, (e - (p - 1)).astype(np.int64))   # quantum at that exponent
    r = np.rint(ax / q) * q               # ax/q is an exact scaling; rint is half-even
    r = np.where(r > vmax, np.inf, r)
    out[fin] = np.copysign(r, x[fin])
    nf = ~np.isfinite(x)
    out[nf] = x[nf]
    zero = (x == 0)
    out[zero] = x[zero]                   # keeps the sign of zero
    return out


def round16(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> fp16/bf16 bit patterns, round to nearest even (one rounding)."""
    p, emin, vmax = _FMT16[dtype]
    r = round_sig(x, p, emin, vmax)
    if dtype == F16:
        # exact after round_sig, so the conversion below does not round again
        return r.astype(np.float16).view(np.uint16)
    r32 = r.astype(np.float32)            # exact: bf16 values are fp32 values
    u = r32.view(np.uint32)
    out = (u >> 16).astype(np.uint16)
    out[np.isnan(r32)] = 0x7FC0
    return out


# ---------------------------------------------------------------------------
# O1  smoothing factors  [SVDQuant §4.2, "Migrate outliers from activations
#     to weights", Fig. 4]
# ---------------------------------------------------------------------------
def activation_absmax(X: np.ndarray) -> np.ndarray:
    """Per input channel max |X[:, j]| (the calibration statistic), fp32."""
    return np.max(np.abs(np.asarray(X, dtype=np.float64)), axis=0).astype(np.float32)


def weight_channel_absmax(W: np.ndarray) -> np.ndarray:
    """Per input channel max_n |W[j, n]|, fp32 (exact for 16-bit weights)."""
    return np.max(np.abs(np.asarray(W, dtype=np.float64)), axis=1).astype(np.float32)


def smoothing_factors(act_absmax: np.ndarray, w_absmax: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """lambda_j = sqrt(max|X_j| / max|W_j|) in fp32 (correctly rounded divide,
    then sqrt) and its fp32 reciprocal.

    The paper divides the input by a per-channel factor and multiplies the
    weight by it (§4.2); its formula was lost in extraction.  Reading: the
    square-root balance of the two channel maxima (migration strength 1/2).
    A channel with a zero maximum on either side, or whose ratio is not a
    positive finite fp32 number, keeps lambda = 1.
    """
    a = np.asarray(act_absmax, dtype=np.float32)
    w = np.asarray(w_absmax, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        ratio = (a / w).astype(np.float32)
        lam = np.sqrt(ratio).astype(np.float32)
    ok = (a > 0) & (w > 0) & np.isfinite(ratio) & (ratio > 0) & np.isfinite(lam) & (lam > 0)
    lam = np.where(ok, lam, np.float32(1.0)).astype(np.float32)
    with np.errstate(over="ignore"):
        invlam = (np.float32(1.0) / lam).astype(np.float32)
    return lam, invlam


# ---------------------------------------------------------------------------
# O2, O3  smoothed weight and its truncated SVD  [SVDQuant §4.2, Eq. 5,
#         "Absorb magnified weight outliers with a low-rank branch", Fig. 5]
# ---------------------------------------------------------------------------
def smoothed_weight(W: np.ndarray, lam: np.ndarray) -> np.ndarray:
    """W_hat = diag(lambda) W in float64 (exact for 16-bit W and fp32 lambda)."""
    return np.asarray(lam, dtype=np.float64)[:, None] * np.asarray(W, dtype=np.float64)


def truncated_svd(W_hat: np.ndarray, r: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """L1 = U_r Sigma_r (K x r), L2 = V_r^T (r x N): the rank-r split that
    minimises the residual norm (Eckart-Young-Mirsky, §4.2).  Also returns
    all singular values.  Sigma goes into L1 (the garbled placement read as
    L1 = U Sigma, L2 = V^T)."""
    U, S, Vt = np.linalg.svd(np.asarray(W_hat, dtype=np.float64), full_matrices=False)
    r = int(r)
    L1 = U[:, :r] * S[None, :r]
    L2 = Vt[:r, :].copy()
    return L1, L2, S


# ---------------------------------------------------------------------------
# O4  runtime 16-bit factors; O5 residual  [SVDQuant §4.2 Eq. 5: the 16-bit
#     low-rank branch and the 4-bit residual]
# ---------------------------------------------------------------------------
def runtime_factors(L1: np.ndarray, L2: np.ndarray, invlam: np.ndarray, dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """L1x = round16(diag(1/lambda) L1), L2q = round16(L2) (bit patterns).

    X_hat L1 = X diag(1/lambda) L1, so folding 1/lambda into L1 lets the
    runtime multiply the raw 16-bit activations (one rounding fewer)."""
    L1x = round16(np.asarray(invlam, dtype=np.float64)[:, None] * np.asarray(L1, dtype=np.float64), dtype)
    L2q = round16(np.asarray(L2, dtype=np.float64), dtype)
    return L1x, L2q


def residual(W: np.ndarray, lam: np.ndarray, L1x: np.ndarray, L2q: np.ndarray) -> np.ndarray:
    """R = fl32(W_hat - diag(lambda) (L1x L2q)) with the low-rank product
    summed in float64 over k ascending (each term exact), so the residual
    absorbs the 16-bit rounding of the factors.  Order, stated exactly:
        s = 0; for k: s = s + L1x[:, k] * L2q[k, :]
        R = fl32(lambda * W - lambda * s)
    """
    W = np.asarray(W, dtype=np.float64)
    lam64 = np.asarray(lam, dtype=np.float64)
    L1x = np.asarray(L1x, dtype=np.float64)
    L2q = np.asarray(L2q, dtype=np.float64)
    K, N = W.shape
    s = np.zeros((K, N), dtype=np.float64)
    for k in range(L1x.shape[1]):
        s += np.multiply.outer(L1x[:, k], L2q[k, :])
    What = lam64[:, None] * W
    d = lam64[:, None] * s
    return (What - d).astype(np.float32)


# ---------------------------------------------------------------------------
# O6  group quantizers  [SVDQuant §3 quantizer Q(x) = round(x / s),
#     s = max|x| / q_max; §5.1 implementation details: symmetric per-group,
#     INT4 group 64 with 16-bit scales, FP4 group 32 with 8-bit (MX) scales]
# ---------------------------------------------------------------------------
def quant_int4_g64(v: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """v: fp32 [..., 64].  Returns (codes int8 in [-7, 7], fp16 scale bits).

    s = fp16_rne(min(fl32(max|v| / 7), 65504));
    q = clamp(rint_half_even(fl32(v / fp32(s))), -7, 7), q = 0 if s == 0.
    """
    v = np.asarray(v, dtype=np.float32)
    assert v.shape[-1] == 64
    m = np.max(np.abs(v), axis=-1).astype(np.float32)
    s = (m / np.float32(INT4_QMAX)).astype(np.float32)
    s = np.minimum(s, np.float32(FP16_MAX)).astype(np.float32)
    sh = s.astype(np.float16)
    s32 = sh.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (v / s32[..., None]).astype(np.float32)
    q = np.clip(np.rint(ratio), -INT4_QMAX, INT4_QMAX)
    q = np.where(s32[..., None] == 0, 0.0, q)
    q = np.nan_to_num(q, nan=0.0)
    return q.astype(np.int8), sh.view(np.uint16)


def dequant_int4(q: np.ndarray, s_bits: np.ndarray) -> np.ndarray:
    s = np.asarray(s_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    return np.asarray(q, dtype=np.float64) * s[..., None]


def _e2m1_nearest_even(a: np.ndarray) -> np.ndarray:
    """Index into E2M1_GRID of the nearest magnitude, ties to the even index
    (even mantissa bit), saturating above 6.  a >= 0, float32."""
    a = np.minimum(np.asarray(a, dtype=np.float64), E2M1_QMAX)
    flat = a.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    even = (np.arange(8) % 2 == 0)
    step = 1 << 20
    for i in range(0, flat.size, step):
        blk = flat[i:i + step]
        d = np.abs(blk[:, None] - E2M1_GRID[None, :])
        dmin = d.min(axis=1, keepdims=True)
        cand = d == dmin
        has_even = (cand & even[None, :]).any(axis=1)
        pick_even = np.argmax(cand & even[None, :], axis=1)
        pick_any = np.argmax(cand, axis=1)
        out[i:i + step] = np.where(has_even, pick_even, pick_any)
    return out.reshape(a.shape)


def quant_mxfp4_g32(v: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """v: fp32 [..., 32].  Returns (E2M1 codes uint8 0..15, e8m0 scale bytes).

    Scale: t = fl32(max|v| / 6); e = biased exponent of t, plus one if t is
    not a power of two, so 2^(e-127) >= t (reading: round the scale up, so
    |v| / scale <= 6 and no element clips); e = 0 for t = 0; e <= 254.
    Element: u = v * 2^(127 - e) (exact), magnitude rounded to nearest E2M1
    value, ties to even, saturating at 6; sign bit = sign of v (so -0 -> 0x8).
    """
    v = np.asarray(v, dtype=np.float32)
    assert v.shape[-1] == 32
    m = np.max(np.abs(v), axis=-1).astype(np.float32)
    t = (m / np.float32(E2M1_QMAX)).astype(np.float32)
    tb = t.view(np.uint32)
    e = ((tb >> 23) & 0xFF).astype(np.int64)
    e = e + ((tb & 0x7FFFFF) != 0)
    e = np.where(t == 0, 0, e)
    e = np.minimum(e, 254)
    u = np.ldexp(v, (127 - e)[..., None].astype(np.int32)).astype(np.float32)
    idx = _e2m1_nearest_even(np.abs(u))
    sign = np.signbit(v).astype(np.uint8)
    codes = (idx | (sign << 3)).astype(np.uint8)
    return codes, e.astype(np.uint8)


def dequant_mxfp4(codes: np.ndarray, e: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_GRID[c & 7]
    val = np.where((c >> 3) & 1, -mag, mag)
    return val * np.ldexp(1.0, np.asarray(e, dtype=np.int64) - 127)[..., None]


def quant_int8_row(v: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """v: fp32 [..., L], one scale for the whole last axis (a token's row of
    X_hat, or an output channel's column of R) [SVDQuant §5.1 implementation
    details: the 8-bit setting quantizes activations per token, dynamically,
    and weights per channel].  Returns (codes int8 in [-127, 127], fp32 scales
    [..., 1]).

    s = fl32(max|v| / 127) (reading: fp32 scale; the pages fix 16-bit scales
    only for the INT4 groups); q = clamp(rint_half_even(fl32(v / s)),
    -127, 127), q = 0 if s == 0.
    """
    v = np.asarray(v, dtype=np.float32)
    m = np.max(np.abs(v), axis=-1).astype(np.float32)
    s = (m / np.float32(INT8_QMAX)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (v / s[..., None]).astype(np.float32)
    q = np.clip(np.rint(ratio), -INT8_QMAX, INT8_QMAX)
    q = np.where(s[..., None] == 0, 0.0, q)
    q = np.nan_to_num(q, nan=0.0)
    return q.astype(np.int8), s[..., None]


def dequant_int8(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    return np.asarray(q, dtype=np.float64) * np.asarray(s, dtype=np.float64)


def quantize_groups(v32: np.ndarray, fmt: str):
    """Quantize the last axis of v32 in consecutive groups along it (INT8:
    one group spanning the whole axis)."""
    if fmt == INT8:
        return quant_int8_row(v32)
    G = GROUP[fmt]
    *lead, K = v32.shape
    assert K % G == 0, "K must be a multiple of the group size"
    g = v32.reshape(*lead, K // G, G)
    if fmt == INT4:
        q, s = quant_int4_g64(g)
    elif fmt == MXFP4:
        q, s = quant_mxfp4_g32(g)
    else:
        raise ValueError(fmt)
    return q.reshape(*lead, K), s


def dequantize_groups(q: np.ndarray, s: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == INT8:
        return dequant_int8(q, s)
    G = GROUP[fmt]
    *lead, K = q.shape
    g = q.reshape(*lead, K // G, G)
    d = dequant_int4(g, s) if fmt == INT4 else dequant_mxfp4(g, s)
    return d.reshape(*lead, K)


def quantize_weight(R: np.ndarray, fmt: str) -> Tuple[np.ndarray, np.ndarray]:
    """Quantize the residual per output column n, groups along K.
    Returns codes [K, N] (int8 INT4 values, uint8 E2M1 codes, int8 INT8
    values) and scales [K/G, N] (fp16 bits, e8m0 bytes; INT8: fp32 [1, N])."""
    q, s = quantize_groups(np.ascontiguousarray(np.asarray(R, dtype=np.float32).T), fmt)
    return np.ascontiguousarray(q.T), np.ascontiguousarray(s.T)


def dequant_weight(q: np.ndarray, s: np.ndarray, fmt: str) -> np.ndarray:
    return np.ascontiguousarray(dequantize_groups(np.ascontiguousarray(q.T), np.ascontiguousarray(s.T), fmt).T)


def quantize_activations(X: np.ndarray, invlam: np.ndarray, fmt: str):
    """x_hat = fl32(fp32(x) * (1/lambda_k)) (one fp32 multiply), then the
    group quantizer along K for every token.  Returns (codes [M,K],
    scales [M,K/G], x_hat fp32)."""
    x32 = np.asarray(X, dtype=np.float64).astype(np.float32)
    xh = (x32 * np.asarray(invlam, dtype=np.float32)[None, :]).astype(np.float32)
    q, s = quantize_groups(xh, fmt)
    return q, s, xh


def dequant_activations(q, s, fmt):
    return dequantize_groups(q, s, fmt)


# ---------------------------------------------------------------------------
# O8  down-projection, O9 4-bit product, O10 epilogue  [SVDQuant §4.2 Eq. 5;
#     §4.3: the down-projection shares its input with the quantizer, the
#     up-projection shares its output with the 4-bit product, Fig. 6b]
# ---------------------------------------------------------------------------
def down_projection(X: np.ndarray, L1x: np.ndarray, dtype: str) -> np.ndarray:
    """T = round16(X L1x) (16-bit branch; product in float64). Bit patterns."""
    return round16(np.asarray(X, dtype=np.float64) @ np.asarray(L1x, dtype=np.float64), dtype)


def int4_group_partials(qx: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """P[g, m, n] = sum_{k in group g} qx[m,k] qw[k,n]: exact integers (int32
    range), the quantity an integer matrix unit accumulates per group."""
    qx = np.asarray(qx, dtype=np.int64)
    qw = np.asarray(qw, dtype=np.int64)
    M, K = qx.shape
    G = GROUP[INT4]
    out = np.empty((K // G, M, qw.shape[1]), dtype=np.int64)
    for g in range(K // G):
        a = qx[:, g * G:(g + 1) * G].astype(np.float64)   # |sum| <= 64*49: exact in float64
        b = qw[g * G:(g + 1) * G, :].astype(np.float64)
        out[g] = np.rint(a @ b).astype(np.int64)
    return out


def main_product(qx, sx, qw, sw, fmt: str) -> np.ndarray:
    """Q(X_hat) Q(R) in float64.
    INT4:  sum_g s_x[m,g] s_w[g,n] P_g[m,n]   (P_g exact integers)
    MXFP4: sum_b 2^(e_x + e_w - 254) sum_{k in b} e2m1(qx) e2m1(qw); both
           dequantized operands are exact in float64, so this is their product.
    INT8:  s_x[m] s_w[n] P[m,n], P = sum_k qx[m,k] qw[k,n] exact (|P| <= K 127^2
           < 2^53, so the float64 matrix product of the integer codes is exact).
    """
    if fmt == INT8:
        P = np.asarray(qx, dtype=np.float64) @ np.asarray(qw, dtype=np.float64)
        return (np.asarray(sx, dtype=np.float64).reshape(-1, 1) * np.asarray(sw, dtype=np.float64).reshape(1, -1)) * P
    if fmt == INT4:
        P = int4_group_partials(qx, qw).astype(np.float64)
        sxf = np.asarray(sx, dtype=np.uint16).view(np.float16).astype(np.float64)   # [M, Gs]
        swf = np.asarray(sw, dtype=np.uint16).view(np.float16).astype(np.float64)   # [Gs, N]
        Y = np.zeros((qx.shape[0], qw.shape[1]), dtype=np.float64)
        for g in range(P.shape[0]):
            Y += (sxf[:, g:g + 1] * swf[g:g + 1, :]) * P[g]
        return Y
    if fmt == MXFP4:
        xd = dequant_activations(qx, sx, fmt)
        wd = dequant_weight(qw, sw, fmt)
        return xd @ wd
    raise ValueError(fmt)


def gelu_erf(x: np.ndarray) -> np.ndarray:
    """x * Phi(x), the erf form of GELU (float64)."""
    from scipy.special import erf
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def output_epilogue_f64(Y_main: np.ndarray, T: np.ndarray, L2q: np.ndarray, bias: Optional[np.ndarray],
                        gelu: bool) -> np.ndarray:
    """Y_main + T L2q + bias [-> GELU] in float64 (before the output rounding)."""
    Y = np.asarray(Y_main, dtype=np.float64) + np.asarray(T, dtype=np.float64) @ np.asarray(L2q, dtype=np.float64)
    if bias is not None:
        Y = Y + np.asarray(bias, dtype=np.float64)[None, :]
    if gelu:
        Y = gelu_erf(Y)
    return Y


def output_epilogue(Y_main: np.ndarray, T: np.ndarray, L2q: np.ndarray, bias: Optional[np.ndarray],
                    gelu: bool, dtype: str) -> np.ndarray:
    """Y = round16(Y_main + T L2q + bias [-> GELU]) (float64 until the one rounding)."""
    return round16(output_epilogue_f64(Y_main, T, L2q, bias, gelu), dtype)


# ---------------------------------------------------------------------------
# Whole layer: offline pack, LoRA attach, forward
# ---------------------------------------------------------------------------
def pack_from_factors(W_bits, dtype, lam, L1x_bits, L2q_bits, fmt) -> Dict[str, np.ndarray]:
    """Residual and its codes given lambda and the 16-bit factors (so another
    implementation's split can be checked code for code)."""
    W = decode16(W_bits, dtype)
    L1x = decode16(L1x_bits, dtype)
    L2q = decode16(L2q_bits, dtype)
    R = residual(W, lam, L1x, L2q)
    qw, sw = quantize_weight(R, fmt)
    return {"R": R, "qw": qw, "sw": sw}


def pack(W_bits, dtype, act_absmax, r: int, fmt: str, bias_bits=None) -> Dict[str, object]:
    """Offline post-training quantization of one linear layer [SVDQuant §4.2]:
    smoothing factors -> W_hat -> rank-r SVD -> 16-bit factors -> residual
    -> group-quantized residual."""
    W = decode16(W_bits, dtype)
    lam, invlam = smoothing_factors(act_absmax, weight_channel_absmax(W))
    What = smoothed_weight(W, lam)
    L1, L2, S = truncated_svd(What, r)
    L1x, L2q = runtime_factors(L1, L2, invlam, dtype)
    pf = pack_from_factors(W_bits, dtype, lam, L1x, L2q, fmt)
    return {
        "dtype": dtype, "fmt": fmt, "rank": r,
        "lam": lam, "invlam": invlam, "L1": L1, "L2": L2, "sigma": S,
        "L1x": L1x, "L2q": L2q, "R": pf["R"], "qw": pf["qw"], "sw": pf["sw"],
        "bias": None if bias_bits is None else np.asarray(bias_bits, dtype=np.uint16),
    }


# ---------------------------------------------------------------------------
# O10  iterative refinement of the low-rank split  [SVDQuant §4.2, closing
#      remark on the low-rank branch: decompose again with the quantized
#      residual taken out, adjust the residual, repeat, keep the smallest
#      error]
# ---------------------------------------------------------------------------
def split_error(W_bits, dtype, lam, L1x_bits, L2q_bits, qw, sw, fmt) -> float:
    """err = ||W_hat - diag(lambda) L1x L2q - deq(Q(R))||_F^2 in float64: how
    far the packed layer (16-bit low-rank branch plus dequantized residual)
    is from the smoothed weight.  Reading: the pages name "the error" without
    a formula; the weight-space Frobenius error is the quantity the split
    itself minimises."""
    W = decode16(W_bits, dtype)
    What = smoothed_weight(W, lam)
    lam64 = np.asarray(lam, dtype=np.float64)
    lr = lam64[:, None] * (decode16(L1x_bits, dtype) @ decode16(L2q_bits, dtype))
    D = What - lr - dequant_weight(qw, sw, fmt)
    return float(np.sum(D * D))


def refine_split(W_bits, dtype, act_absmax, r: int, fmt: str, iters: int) -> Dict[str, object]:
    """Round 0 is the one-shot split of W_hat.  Round i >= 1 splits
    B_i = W_hat - deq(Q(R_{i-1})) at rank r (B_i's truncated SVD), rounds the
    factors to 16 bits, re-derives R_i = fl32(W_hat - diag(lambda) L1x L2q)
    and its codes.  Returns every round's (L1x, L2q, qw, sw, err) and the index
    of the smallest err."""
    W = decode16(W_bits, dtype)
    lam, invlam = smoothing_factors(act_absmax, weight_channel_absmax(W))
    What = smoothed_weight(W, lam)
    rounds = []
    B = What
    for i in range(int(iters) + 1):
        L1, L2, _ = truncated_svd(B, r)
        L1x, L2q = runtime_factors(L1, L2, invlam, dtype)
        pf = pack_from_factors(W_bits, dtype, lam, L1x, L2q, fmt)
        err = split_error(W_bits, dtype, lam, L1x, L2q, pf["qw"], pf["sw"], fmt)
        rounds.append({"L1x": L1x, "L2q": L2q, "qw": pf["qw"], "sw": pf["sw"], "err": err})
        B = What - dequant_weight(pf["qw"], pf["sw"], fmt)
    best = int(np.argmin([x["err"] for x in rounds]))
    return {"lam": lam, "invlam": invlam, "rounds": rounds, "best": best}


def attach_lora(layer: Dict[str, object], A_bits, B_bits, alpha: float = 1.0) -> Dict[str, object]:
    """Concatenate a LoRA into the low-rank branch without touching the
    residual [SVDQuant §5.2, integrating LoRA; §1: no re-quantization]:
    L1x <- [L1x | A], L2q <- [L2q ; round16(alpha B)].  LoRA acts on the raw
    (unsmoothed) input, as a LoRA of the original layer does."""
    dt = layer["dtype"]
    A = decode16(A_bits, dt)
    B = decode16(B_bits, dt)
    out = dict(layer)
    out["L1x"] = np.concatenate([layer["L1x"], round16(A, dt)], axis=1)
    out["L2q"] = np.concatenate([layer["L2q"], round16(float(alpha) * B, dt)], axis=0)
    return out


def forward(layer: Dict[str, object], X_bits, gelu: bool = False, return_parts: bool = False):
    """Y = X_hat L1 L2 + Q(X_hat) Q(R) (+ bias) for rows X_bits [M, K]
    [SVDQuant §4.2 Eq. 5].  Every step is row-local, so any subset of rows
    can be evaluated on its own."""
    dt, fmt = layer["dtype"], layer["fmt"]
    X = decode16(X_bits, dt)
    qx, sx, xh = quantize_activations(X, layer["invlam"], fmt)
    T = down_projection(X, decode16(layer["L1x"], dt), dt)
    Ym = main_product(qx, sx, layer["qw"], layer["sw"], fmt)
    bias = None if layer.get("bias") is None else decode16(layer["bias"], dt)
    Y64 = output_epilogue_f64(Ym, decode16(T, dt), decode16(layer["L2q"], dt), bias, gelu)
    Y = round16(Y64, dt)
    if return_parts:
        return Y, {"qx": qx, "sx": sx, "xhat": xh, "T": T, "Ymain": Ym, "Y64": Y64}
    return Y


# ---------------------------------------------------------------------------
# Error analysis  [SVDQuant §4.1, Problem Formulation, Prop. 4.1]
# ---------------------------------------------------------------------------
def quantization_error(X: np.ndarray, W: np.ndarray, Xq: np.ndarray, Wq: np.ndarray) -> float:
    """E(X, W) = ||X W - Q(X) Q(W)||_F (dequantized operands)."""
    return float(np.linalg.norm(np.asarray(X) @ np.asarray(W) - np.asarray(Xq) @ np.asarray(Wq)))


def prop41_bound(X, W, Xq, Wq) -> float:
    """Upper bound from the four quantities Prop. 4.1 names (||X||, ||W|| and
    their quantization errors); the inequality itself was lost in
    extraction.  Reading (triangle inequality + submultiplicativity):
        E <= ||X||_F ||W - Q(W)||_F + ||X - Q(X)||_F (||W||_F + ||W - Q(W)||_F)
    """
    nX = np.linalg.norm(X)
    nW = np.linalg.norm(W)
    eX = np.linalg.norm(np.asarray(X) - np.asarray(Xq))
    eW = np.linalg.norm(np.asarray(W) - np.asarray(Wq))
    return float(nX * eW + eX * (nW + eW))


def lowrank_overhead(K: int, N: int, r: int) -> float:
    """Extra parameters / compute of the low-rank branch relative to the
    layer: (K + N) r / (K N)  [SVDQuant §4.2, after Eq. 5]."""
    return (K + N) * r / (K * N)


def packed_bytes(K: int, N: int, r: int, fmt: str) -> int:
    """Bytes of one packed layer: 4-bit residual codes, group scales, the two
    16-bit factors and lambda, 1/lambda (fp32 each)."""
    G = GROUP[fmt]
    scale_bytes = 2 if fmt == INT4 else 1
    return K * N // 2 + (K // G) * N * scale_bytes + 2 * r * (K + N) + 8 * K
