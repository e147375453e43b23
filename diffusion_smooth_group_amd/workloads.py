"""Seeded synthetic inputs for the SVDQuant linear.

This module only draws random numbers and encodes them as 16-bit floats.
It holds none of the method's arithmetic (no smoothing, no SVD, no
quantization), so both the CPU oracle and the HIP path can consume the
exact same bytes.

The shapes and value distributions stand in for the FLUX.1 / SDXL
activations and weights that the SVDQuant paper calibrates and evaluates on
(SVDQuant: Absorbing Outliers by Low-Rank Components for 4-Bit Diffusion
Models, §5.1 Setups: FLUX.1, SDXL; implementation details: rank 32, INT4
group 64, FP4 group 32).  Those models and prompt sets are not available,
so every tensor here is synthetic.

Recipe (per linear shape):
  rng = numpy.random.default_rng([config_seed, shape_index])
  draws, in this order: X, activation outlier channels, W, weight outlier
  rows, bias, LoRA A, LoRA B.  Samples are float64, scaled, cast to fp32
  (round to nearest even) and then to fp16 / bf16 (round to nearest even).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

F16 = "f16"
BF16 = "bf16"
INT4 = "int4_g64"
MXFP4 = "mxfp4_g32"


# --------------------------------------------------------------------------
# 16-bit encodings (input plumbing: float32 -> storage bits)
# --------------------------------------------------------------------------
def f32_to_bits16(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Encode float32 values as fp16 or bf16 bit patterns, round to nearest even."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == F16:
        return x32.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        u = x32.view(np.uint32).astype(np.uint64)
        nan = np.isnan(x32)
        r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        r[nan] = 0x7FC0
        return r
    raise ValueError(dtype)


def bits16_to_f32(b: np.ndarray, dtype: str) -> np.ndarray:
    """Decode fp16 / bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    if dtype == F16:
        return b.view(np.float16).astype(np.float32)
    if dtype == BF16:
        return (b.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


def _to16(x64: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bits16(np.asarray(x64, dtype=np.float64).astype(np.float32), dtype)


# --------------------------------------------------------------------------
# Shapes
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class LinearSpec:
    name: str
    M: int
    K: int
    N: int
    dtype: str
    formats: tuple            # quantization formats exercised on this shape
    rank: int                 # SVD rank r
    lora_rank: int            # extra LoRA rank concatenated into the low-rank branch (0 = none)
    x_dist: str               # "gauss002" | "student_t3" | "gelu_of_fc1"
    x_outliers: int           # number of outlier activation channels
    x_outlier_scale: float
    w_outliers: int           # number of outlier weight rows (input channels)
    w_outlier_scale: float
    bias: bool
    seed: tuple               # (config seed, shape index)


def _pct1(k: int) -> int:
    return int(round(0.01 * k))


def config_shapes(cfg: int) -> List[LinearSpec]:
    """The five synthetic workloads (1-based config number)."""
    out: List[LinearSpec] = []
    if cfg == 1:
        out.append(LinearSpec("single_256x1152x1152", 256, 1152, 1152, F16, (INT4,), 32, 0,
                              "gauss002", 8, 20.0, 8, 10.0, False, (1, 0)))
    elif cfg == 2:
        out.append(LinearSpec("flux_qkv_4608x3072x9216", 4608, 3072, 9216, BF16, (INT4,), 32, 0,
                              "student_t3", _pct1(3072), 30.0, 0, 1.0, True, (2, 0)))
    elif cfg == 3:
        out.append(LinearSpec("flux_fc1_4608x3072x12288", 4608, 3072, 12288, BF16, (MXFP4, INT4), 32, 0,
                              "student_t3", _pct1(3072), 30.0, 0, 1.0, True, (3, 0)))
        out.append(LinearSpec("flux_fc2_4608x12288x3072", 4608, 12288, 3072, BF16, (MXFP4, INT4), 32, 0,
                              "gelu_of_fc1", 0, 1.0, 0, 1.0, True, (3, 1)))
    elif cfg == 4:
        shapes = [(8192, 640, 640), (8192, 640, 5120), (2048, 1280, 1280), (2048, 1280, 10240)]
        for i, (m, k, n) in enumerate(shapes):
            out.append(LinearSpec(f"sdxl_{m}x{k}x{n}", m, k, n, F16, (INT4,), 32, 16,
                                  "gauss002", 8, 20.0, 8, 10.0, True, (4, i)))
    elif cfg == 5:
        lin = [("qkv", 3072, 9216), ("proj", 3072, 3072), ("fc1", 3072, 12288),
               ("fc2", 12288, 3072), ("adaln", 3072, 18432)]
        i = 0
        for m in (4608, 16896):
            for nm, k, n in lin:
                out.append(LinearSpec(f"flux_block_{nm}_{m}x{k}x{n}", m, k, n, BF16, (MXFP4, INT4), 32, 16,
                                      "student_t3", _pct1(k), 30.0, _pct1(k), 10.0, True, (5, i)))
                i += 1
    else:
        raise ValueError(cfg)
    return out


def with_rows(spec: LinearSpec, M: int) -> LinearSpec:
    """Same layer and seed, different token count (for small parity cases)."""
    return dataclasses.replace(spec, M=M)


def small_spec(name, M, K, N, dtype, fmt, rank, lora_rank=0, x_dist="student_t3",
               x_outliers=None, w_outliers=None, bias=True, seed=(99, 0)) -> LinearSpec:
    """A reduced-size layer with the same recipe (oracle-sized parity cases)."""
    xo = _pct1(K) if x_outliers is None else x_outliers
    wo = _pct1(K) if w_outliers is None else w_outliers
    return LinearSpec(name, M, K, N, dtype, (fmt,), rank, lora_rank, x_dist, max(xo, 1), 30.0,
                      wo, 10.0, bias, seed)


# --------------------------------------------------------------------------
# Generation
# --------------------------------------------------------------------------
def _gelu_erf64(x: np.ndarray) -> np.ndarray:
    from scipy.special import erf
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def generate(spec: LinearSpec, fc1_inputs: Optional[Dict[str, np.ndarray]] = None) -> Dict[str, object]:
    """Draw one layer's inputs.  Returns 16-bit bit patterns (uint16 arrays).

    keys: X [M,K], W [K,N], bias [N] or None, lora_A [K,rL] or None,
          lora_B [rL,N] or None, dtype, spec.
    For x_dist == "gelu_of_fc1" (the MLP pair's second linear) X is
    bf16(GELU(X1 @ W1 + b1)) of the first linear's inputs, the exact
    (unquantized) product computed in float32: the hidden activations of an
    MLP.  Pass the first linear's generate() result as fc1_inputs, or it is
    regenerated here.
    """
    rng = np.random.default_rng(list(spec.seed))
    M, K, N = spec.M, spec.K, spec.N
    # X
    if spec.x_dist == "gauss002":
        X = rng.standard_normal((M, K)) * 0.02
    elif spec.x_dist == "student_t3":
        X = rng.standard_t(3.0, size=(M, K))
    elif spec.x_dist == "gelu_of_fc1":
        X = None
    else:
        raise ValueError(spec.x_dist)
    # activation outlier channels
    if X is not None and spec.x_outliers > 0:
        idx = rng.choice(K, size=spec.x_outliers, replace=False)
        X[:, idx] *= spec.x_outlier_scale
    # W
    W = rng.standard_normal((K, N)) * 0.02
    if spec.w_outliers > 0:
        widx = rng.choice(K, size=spec.w_outliers, replace=False)
        W[widx, :] *= spec.w_outlier_scale
    bias = rng.standard_normal(N) * 0.02 if spec.bias else None
    A = B = None
    if spec.lora_rank > 0:
        A = rng.standard_normal((K, spec.lora_rank)) * 0.02
        B = rng.standard_normal((spec.lora_rank, N)) * 0.02
    dt = spec.dtype
    if X is None:
        if fc1_inputs is None:
            fc1_spec = dataclasses.replace(spec, K=N, N=K, x_dist="student_t3",
                                           x_outliers=_pct1(N), x_outlier_scale=30.0,
                                           seed=(spec.seed[0], spec.seed[1] - 1))
            fc1_inputs = generate(fc1_spec)
        x1 = bits16_to_f32(fc1_inputs["X"], dt)
        w1 = bits16_to_f32(fc1_inputs["W"], dt)
        h = x1 @ w1
        if fc1_inputs["bias"] is not None:
            h = h + bits16_to_f32(fc1_inputs["bias"], dt)[None, :]
        Xb = f32_to_bits16(_gelu_erf64(h.astype(np.float64)).astype(np.float32), dt)
        assert Xb.shape == (M, K), (Xb.shape, M, K)
    else:
        Xb = _to16(X, dt)
    return {
        "X": Xb,
        "W": _to16(W, dt),
        "bias": None if bias is None else _to16(bias, dt),
        "lora_A": None if A is None else _to16(A, dt),
        "lora_B": None if B is None else _to16(B, dt),
        "dtype": dt,
        "spec": spec,
    }


def random_rows(M: int, count: int, seed: int = 12345) -> np.ndarray:
    """Sorted sample of row indices (used to check large outputs row by row)."""
    rng = np.random.default_rng(seed)
    count = min(count, M)
    return np.sort(rng.choice(M, size=count, replace=False))
