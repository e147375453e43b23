"""Pins for the oracle's 8-bit setting (per-token dynamic activation scales,
per-output-channel weight scales, q_max = 127) [SVDQuant §5.1 implementation
details], checked against closed forms, the nearest-integer property in
exact arithmetic, locality invariants and brute force on tiny inputs."""
import numpy as np

import oracle as o


def test_int8_closed_form_values():
    # max |v| = 127 gives s = 1 exactly, so the codes are rint(v) (ties to even)
    v = np.array([127.0, -63.5, 0.5, -0.5, 1.5, 2.5, 0.0, -127.0, 3.25, -100.49], np.float32)
    q, s = o.quant_int8_row(v)
    assert s.shape == (1,) and s[0] == np.float32(1.0)
    assert q.tolist() == [127, -64, 0, 0, 2, 2, 0, -127, 3, -100]
    # an all-zero row: scale 0, codes 0
    q0, s0 = o.quant_int8_row(np.zeros((2, 64), np.float32))
    assert not q0.any() and not s0.any() and s0.shape == (2, 1)


def test_int8_codes_are_nearest_integers():
    rng = np.random.default_rng(3)
    v = (rng.standard_t(3.0, size=(64, 300)) * rng.uniform(1e-3, 1e3, size=(64, 1))).astype(np.float32)
    q, s = o.quant_int8_row(v)
    q = q.astype(np.int64)
    s64 = s.astype(np.float64)
    # the row maximum lands on +-127; no code exceeds 127
    i = np.argmax(np.abs(v), axis=1)
    assert np.array_equal(np.abs(q[np.arange(64), i]), np.full(64, 127))
    assert np.abs(q).max() <= 127
    # q is the nearest integer to the exact ratio v / s (float64), except
    # where that ratio lies within one float32 ulp of a half-integer
    t = v.astype(np.float64) / s64
    frac = np.abs(t - np.floor(t) - 0.5)
    clear = frac > 4 * np.spacing(np.abs(t).astype(np.float32)).astype(np.float64)
    assert np.array_equal(q[clear], np.rint(t[clear]).astype(np.int64))
    # dequantized error at most half a step
    assert np.all(np.abs(v - q * s64) <= 0.5 * s64 * (1 + 1e-6))


def test_int8_per_token_and_per_channel_locality():
    rng = np.random.default_rng(4)
    X = o.round16(rng.standard_normal((40, 256)) * np.exp(rng.uniform(-3, 3, size=(1, 256))), o.BF16)
    invlam = rng.uniform(0.1, 10.0, size=256).astype(np.float32)
    q, s, _ = o.quantize_activations(o.decode16(X, o.BF16), invlam, o.INT8)
    assert q.shape == (40, 256) and s.shape == (40, 1)
    q2, s2, _ = o.quantize_activations(o.decode16(X[7:19], o.BF16), invlam, o.INT8)
    assert np.array_equal(q2, q[7:19]) and np.array_equal(s2, s[7:19])      # dynamic per token
    R = (rng.standard_normal((256, 96)) * rng.uniform(1e-3, 1.0, size=(1, 96))).astype(np.float32)
    qw, sw = o.quantize_weight(R, o.INT8)
    assert qw.shape == (256, 96) and sw.shape == (1, 96)
    qw2, sw2 = o.quantize_weight(R[:, 10:30], o.INT8)
    assert np.array_equal(qw2, qw[:, 10:30]) and np.array_equal(sw2, sw[:, 10:30])   # per channel
    # the channel scale is the column maximum over 127
    assert np.array_equal(sw[0], (np.abs(R).max(axis=0) / np.float32(127)).astype(np.float32))


def test_int8_main_product_brute_force():
    rng = np.random.default_rng(5)
    M, K, N = 5, 128, 7
    qx = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    qw = rng.integers(-127, 128, size=(K, N)).astype(np.int8)
    sx = rng.uniform(1e-3, 1.0, size=(M, 1)).astype(np.float32)
    sw = rng.uniform(1e-3, 1.0, size=(1, N)).astype(np.float32)
    Y = o.main_product(qx, sx, qw, sw, o.INT8)
    for m in range(M):
        for n in range(N):
            P = sum(int(qx[m, k]) * int(qw[k, n]) for k in range(K))      # exact integer
            assert Y[m, n] == float(sx[m, 0]) * float(sw[0, n]) * P


def test_int8_layer_is_far_closer_to_the_exact_product_than_4_bit():
    # the same layer, same smoothing and rank: 8-bit codes leave a much
    # smaller error against the unquantized X W than 4-bit groups do
    rng = np.random.default_rng(6)
    M, K, N = 64, 256, 128
    X = o.round16(rng.standard_t(3.0, size=(M, K)), o.BF16)
    W = o.round16(rng.standard_normal((K, N)) * 0.02, o.BF16)
    a = o.activation_absmax(o.decode16(X, o.BF16))
    exact = o.decode16(X, o.BF16) @ o.decode16(W, o.BF16)
    err = {}
    for fmt in (o.INT8, o.INT4):
        layer = o.pack(W, o.BF16, a, 16, fmt)
        Y = o.decode16(o.forward(layer, X), o.BF16)
        err[fmt] = np.linalg.norm(Y - exact) / np.linalg.norm(exact)
    assert err[o.INT8] < 0.02
    assert err[o.INT8] < 0.25 * err[o.INT4]


def test_int8_rank_zero_forward_is_w8a8_brute_force():
    rng = np.random.default_rng(7)
    M, K, N = 3, 128, 4
    X = o.round16(rng.standard_normal((M, K)), o.F16)
    W = o.round16(rng.standard_normal((K, N)) * 0.05, o.F16)
    a = o.activation_absmax(o.decode16(X, o.F16))
    layer = o.pack(W, o.F16, a, 0, o.INT8)
    Y = o.decode16(o.forward(layer, X), o.F16)
    # rank 0: Y = round16(sum_k qx qw sx sw), with every code and scale checked
    # against its definition element by element
    lam = layer["lam"].astype(np.float64)
    What = o.decode16(W, o.F16) * lam[:, None]
    for n in range(N):
        col = What[:, n].astype(np.float32)
        s = np.float32(np.abs(col).max() / np.float32(127))
        assert layer["sw"][0, n] == s
    for m in range(M):
        xh = (o.decode16(X[m], o.F16).astype(np.float32) * layer["invlam"]).astype(np.float32)
        sxm = np.float32(np.abs(xh).max() / np.float32(127))
        qx = [int(np.clip(np.rint(np.float32(x / sxm)), -127, 127)) for x in xh]
        for n in range(N):
            P = sum(qx[k] * int(layer["qw"][k, n]) for k in range(K))
            ref = float(sxm) * float(layer["sw"][0, n]) * P
            assert abs(Y[m, n] - ref) <= 2.0 ** -10 * abs(ref) + 1e-12
