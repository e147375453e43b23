"""GPU parity: the HIP path through the C ABI against the oracle.

Gates: activation codes and scales bit-exact; INT4 per-group int32 products
bit-exact; the calibration maxima bit-exact; Y within relative Frobenius
5e-3 and max |dY| <= 1e-2 max |Y|.  Small layers are compared on every
output; the full-size workloads on sampled rows x columns, evaluated one
block at a time by the oracle.
"""
import numpy as np
import pytest

import oracle as o
from diffusion_smooth_group_amd import svdq as S
from diffusion_smooth_group_amd import workloads as wl
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


def _small(M, K, N, dtype, fmt, rank, lora=0, seed=0, x_dist="student_t3", bias=True):
    spec = wl.small_spec(f"small_{M}x{K}x{N}", M, K, N, dtype, fmt, rank, lora_rank=lora, x_dist=x_dist,
                         bias=bias, seed=(100 + seed, 0))
    return wl.generate(spec)


@pytest.mark.parametrize("fmt", [o.MXFP4, o.INT4])
@pytest.mark.parametrize("dtype", [o.BF16, o.F16])
def test_small_layer_full_parity(fmt, dtype):
    d = _small(200, 384, 256, dtype, fmt, 16, seed=1)          # ragged M (not a multiple of 16)
    G.run_layer_case(d, fmt, 16)


@pytest.mark.parametrize("fmt", [o.MXFP4, o.INT4])
def test_lora_gelu_and_ragged(fmt):
    d = _small(77, 512, 384, o.BF16, fmt, 32, lora=16, seed=2)
    G.run_layer_case(d, fmt, 32, lora=True, gelu=True, alpha=0.5)


def test_mxfp4_many_tiles_full_parity():
    # 4096 x 4096 outputs = 256 GEMM tiles of 256 x 256 (one per CU), every output checked
    d = _small(4096, 256, 4096, o.BF16, o.MXFP4, 16, lora=16, seed=30)
    G.run_layer_case(d, o.MXFP4, 16, lora=True, gelu=True)


def test_mxfp4_more_tiles_than_cus_full_parity():
    # 17 x 16 = 272 tiles of 256 x 256: more than the 256 compute units, so
    # a second round of workgroups runs; ragged tokens (4300 of a 4352-row
    # workspace), GELU, LoRA, every output checked
    d = _small(4300, 256, 4096, o.BF16, o.MXFP4, 16, lora=16, seed=33)
    G.run_layer_case(d, o.MXFP4, 16, lora=True, gelu=True)


def test_mxfp4_staggered_uneven_split_full_parity():
    # 17 x 48 = 816 tiles of 256 x 256, more than three rounds on 256 CUs:
    # the launch staggers the odd XCDs and gives them 96 tiles against the
    # even XCDs' 108, with workgroups past an XCD's count running no tile;
    # ragged tokens (4300 of 4352), LoRA, every output checked
    d = _small(4300, 256, 12288, o.BF16, o.MXFP4, 16, lora=16, seed=36)
    G.run_layer_case(d, o.MXFP4, 16, lora=True)


@pytest.mark.parametrize("rank,lora", [(0, 0), (32, 0), (32, 16)])
@pytest.mark.parametrize("K", [640, 3072])
def test_mxfp4_activation_many_workgroups_full_parity(K, rank, lora):
    # 8300 tokens (528 activation workgroups of 16 on an 8448-row workspace):
    # more than two per compute unit on a 256-CU device, where the MXFP4
    # activation kernel requests whole chunks of steps; K = 640 gives waves
    # one or two steps (padding steps in every chunk), K = 3072 six; rank 0,
    # 32 and 48 cover the kernel's three chunk shapes; every output checked
    d = _small(8300, K, 256, o.BF16, o.MXFP4, rank, lora=lora, seed=35)
    G.run_layer_case(d, o.MXFP4, rank, lora=lora > 0)


@pytest.mark.parametrize("dtype", [o.BF16, o.F16])
@pytest.mark.parametrize("rank,lora", [(0, 0), (32, 0), (32, 16)])
def test_activation_two_tile_workgroups_full_parity(dtype, rank, lora):
    # 4300 tokens = 272 16-token tiles on a 4352-row workspace and K = 8192:
    # more tiles than compute units on a 256-CU device and a long K, so each
    # MXFP4 activation workgroup takes two tiles (one L1x fragment load per
    # step for 32 tokens); ragged last tile; rank 0, 32 and 48 (the two ring
    # depths); every code, scale, T row and output checked
    d = _small(4300, 8192, 128, dtype, o.MXFP4, rank, lora=lora, seed=37)
    G.run_layer_case(d, o.MXFP4, rank, lora=lora > 0)


@pytest.mark.parametrize("M", [4097, 8192])
def test_activation_two_tile_workgroup_edges(M):
    # the two-tile form at its edges: 4097 tokens (one real row in the last
    # pair of tiles, the rest repeating it) and 8192 tokens (512 tiles, the
    # largest count before the chunked one-tile form takes over on 256 CUs);
    # K = 8192, rank 32, every code, scale, T row and output checked
    d = _small(M, 8192, 128, o.BF16, o.MXFP4, 32, seed=38)
    G.run_layer_case(d, o.MXFP4, 32)


@pytest.mark.parametrize("dtype", [o.BF16, o.F16])
def test_int4_many_tiles_full_parity(dtype):
    # 17 x 32 = 544 INT4 GEMM tiles of 128 x 128, more than two per compute
    # unit; ragged tokens (2100 of a 2304-row workspace), GELU, LoRA, every
    # output checked
    d = _small(2100, 256, 4096, dtype, o.INT4, 16, lora=16, seed=34)
    G.run_layer_case(d, o.INT4, 16, lora=True, gelu=True)


@pytest.mark.parametrize("K", [128, 256, 384])
@pytest.mark.parametrize("fmt", [o.MXFP4, o.INT4])
def test_short_k_wide_low_rank(fmt, K):
    # fewer 128-deep K steps than the activation kernel has waves, with a
    # rank-48 branch (rank 16 + LoRA 32) whose T tiles every wave finalizes
    d = _small(48, K, 256, o.BF16, fmt, 16, lora=32, seed=20 + K)
    G.run_layer_case(d, fmt, 16, lora=True)


@pytest.mark.parametrize("fmt", [o.MXFP4, o.INT4])
@pytest.mark.parametrize("dtype", [o.BF16, o.F16])
def test_unfused_lowrank_baseline(fmt, dtype):
    # the separate-pass low-rank branch (Y rounded after the 4-bit GEMM and
    # again after T L2 is added) meets the same gates against the oracle,
    # with LoRA columns, GELU after the sum and a ragged token count
    d = _small(150, 512, 384, dtype, fmt, 32, lora=16, seed=60)
    G.run_layer_case(d, fmt, 32, lora=True, gelu=True, unfused=True)


def test_unfused_lowrank_qkv_sampled():
    spec = wl.config_shapes(2)[0]
    d = wl.generate(spec)
    rows, cols = _sample(spec.M, spec.N, 61)
    G.run_layer_case(d, o.INT4, 32, rows=rows, cols=cols, unfused=True)
    d5 = wl.generate(wl.config_shapes(5)[0])
    rows, cols = _sample(d5["spec"].M, d5["spec"].N, 62)
    G.run_layer_case(d5, o.MXFP4, 32, lora=True, rows=rows, cols=cols, unfused=True)


@pytest.mark.parametrize("fmt", [o.MXFP4, o.INT4])
@pytest.mark.parametrize("K", [256, 1024])
def test_branch_wider_than_64(fmt, K):
    # rank 64 + LoRA 32: six 16-rank chunks, three low-rank pipeline steps
    # in the MXFP4 GEMM (the third one is requested by the last K step)
    d = _small(96, K, 256, o.BF16, fmt, 64, lora=32, seed=70 + K)
    G.run_layer_case(d, fmt, 64, lora=True)


@pytest.mark.parametrize("K", [128, 384, 640, 1536])
@pytest.mark.parametrize("dtype", [o.BF16, o.F16])
def test_gelu_gemm_paired_tiles(K, dtype):
    # the MXFP4 GEMM with a GELU epilogue (192 x 192 tiles, two workgroups
    # per compute unit): fewer K steps than stages (K = 128, 384), the
    # steady-state loop (K = 640, 1536), a 96-wide branch (three low-rank
    # steps, some requested by the last K steps), ragged tokens and a partial
    # last column tile (640 = 3 x 192 + 64), every output checked
    d = _small(500, K, 640, dtype, o.MXFP4, 64, lora=32, seed=90 + K)
    G.run_layer_case(d, o.MXFP4, 64, lora=True, gelu=True, alpha=0.75)


@pytest.mark.parametrize("fmt", [o.MXFP4, o.INT4])
def test_refined_pack_forward(fmt):
    # a pack whose low-rank split was refined (device blob written through
    # svdq_pack_weights_ex) meets the same gates
    d = _small(130, 512, 384, o.BF16, fmt, 16, lora=16, seed=80)
    lin, _ = G.run_layer_case(d, fmt, 16, lora=True, gelu=True, refine=2)
    e = lin.refine_errors
    assert e is not None and e.shape == (3,) and np.all(np.isfinite(e)) and e.min() <= e[0]


@pytest.mark.parametrize("M", [1, 17, 256, 300])
def test_token_counts(M):
    d = _small(M, 256, 128, o.F16, o.INT4, 8, seed=3 + M)
    G.run_layer_case(d, o.INT4, 8)


@pytest.mark.parametrize("fmt", [o.INT4, o.MXFP4])
def test_tiny_values_subnormal_scales(fmt):
    # X and W scaled by 2^-14 (exact in bf16), the bias by 2^-28: the INT4
    # group scales absmax / 7 land in fp16's subnormal range on both sides,
    # which the scale products must keep (no flush to zero)
    d = dict(_small(96, 512, 256, o.BF16, fmt, 16, seed=7))
    for key, sc in (("X", 2.0 ** -14), ("W", 2.0 ** -14), ("bias", 2.0 ** -28)):
        d[key] = o.round16(o.decode16(d[key], o.BF16) * sc, o.BF16)
    lin, res = G.run_layer_case(d, fmt, 16)
    if fmt == o.INT4:
        sx = o.decode16(lin.workspace_export(96)["scales"], o.F16)
        assert np.mean((sx > 0) & (sx < 2.0 ** -14)) > 0.5, "most activation scales should be fp16 subnormals"


def test_rank_zero_is_w4a4():
    d = _small(64, 256, 256, o.BF16, o.MXFP4, 0, seed=5)
    G.run_layer_case(d, o.MXFP4, 0, cap=0)


def test_int4_group_partials_bit_exact():
    import torch
    d = _small(96, 512, 256, o.BF16, o.INT4, 16, seed=6)
    Xd = S.bits_to_device(d["X"], S.BF16, G.device())
    lin = G.pack_gpu(d, o.INT4, 16, absmax=G.calib_absmax_gpu(Xd, o.BF16))
    lin.forward(Xd)
    P = lin.int4_group_partials(96, 16, 64, 32, 96, 2, 5).cpu().numpy()
    torch.cuda.synchronize()
    wx = lin.workspace_export(96)
    ex = lin.export()
    ref = o.int4_group_partials(wx["codes"][16:80], ex["codes"][:, 32:128])
    assert np.array_equal(P.astype(np.int64), ref[2:7])
    # the activation codes themselves match the oracle bit for bit
    q, s, _ = o.quantize_activations(o.decode16(d["X"], o.BF16), ex["invlam"], o.INT4)
    assert np.array_equal(wx["codes"].astype(np.int64), q.astype(np.int64)) and np.array_equal(wx["scales"], s)


def test_lora_attach_detach_on_device():
    import torch
    d = _small(64, 256, 256, o.F16, o.MXFP4, 16, lora=16, seed=7)
    Xd = S.bits_to_device(d["X"], S.F16, G.device())
    lin = G.pack_gpu(d, o.MXFP4, 16, cap=48, absmax=G.calib_absmax_gpu(Xd, o.F16))
    Y0 = S.device_to_bits(lin.forward(Xd))
    lin.attach_lora(d["lora_A"], d["lora_B"], 1.0)
    Y1 = S.device_to_bits(lin.forward(Xd))
    lin.detach_lora()
    Y2 = S.device_to_bits(lin.forward(Xd))
    torch.cuda.synchronize()
    assert np.array_equal(Y0, Y2)
    assert not np.array_equal(Y0, Y1)
    # LoRA's contribution equals X A B within 16-bit rounding
    dY = o.decode16(Y1, o.F16) - o.decode16(Y0, o.F16)
    ref = o.decode16(d["X"], o.F16) @ o.decode16(d["lora_A"], o.F16) @ o.decode16(d["lora_B"], o.F16)
    assert np.linalg.norm(dY - ref) / np.linalg.norm(ref) < 0.05


def test_zero_input_and_noop():
    import torch
    d = _small(32, 256, 128, o.BF16, o.INT4, 8, seed=8)
    d["X"] = np.zeros_like(d["X"])
    lin, r = G.run_layer_case(d, o.INT4, 8)
    assert np.array_equal(o.decode16(r["Y"], o.BF16), o.decode16(d["bias"], o.BF16)[None, :].repeat(32, 0))
    Y = torch.full((4, 128), 7.0, dtype=torch.bfloat16, device=G.device())
    Xd = S.bits_to_device(d["X"][:0], S.BF16, G.device())
    lin.forward(Xd, Y=Y[:0])              # M = 0 is a no-op
    torch.cuda.synchronize()
    assert float(Y.float().sum()) == 7.0 * 4 * 128


def test_workspace_reuse_smaller_second_call():
    import torch
    d = _small(160, 256, 256, o.BF16, o.MXFP4, 16, seed=9)
    lin, r1 = G.run_layer_case(d, o.MXFP4, 16)
    d2 = dict(d)
    d2["X"] = np.ascontiguousarray(d["X"][:40])
    Xd = S.bits_to_device(d2["X"], S.BF16, G.device())
    Y = lin.forward(Xd)
    torch.cuda.synchronize()
    assert np.array_equal(S.device_to_bits(Y), r1["Y"][:40])


# ------------------------------------------------------- full-size workloads
ROWS = 48
COLS = 384


def _sample(M, N, seed):
    rows = wl.random_rows(M, ROWS, seed)
    cols = np.sort(np.random.default_rng(seed + 1).choice(N, size=min(COLS, N), replace=False))
    return rows, cols


def test_config1_full():
    spec = wl.config_shapes(1)[0]
    d = wl.generate(spec)
    G.run_layer_case(d, o.INT4, 32)
    d["bias"] = wl.f32_to_bits16((np.random.default_rng(11).standard_normal(spec.N) * 0.02).astype(np.float32), o.F16)
    G.run_layer_case(d, o.INT4, 32)


def test_config2_flux_qkv_sampled():
    spec = wl.config_shapes(2)[0]
    d = wl.generate(spec)
    rows, cols = _sample(spec.M, spec.N, 21)
    G.run_layer_case(d, o.INT4, 32, rows=rows, cols=cols)


@pytest.mark.parametrize("fmt", [o.MXFP4, o.INT4])
def test_config3_flux_mlp_pair_sampled(fmt):
    fc1, fc2 = wl.config_shapes(3)
    d1 = wl.generate(fc1)
    rows, cols = _sample(fc1.M, fc1.N, 31)
    G.run_layer_case(d1, fmt, 32, gelu=True, rows=rows, cols=cols)
    d2 = wl.generate(fc2, fc1_inputs=d1)
    rows, cols = _sample(fc2.M, fc2.N, 32)
    G.run_layer_case(d2, fmt, 32, rows=rows, cols=cols)


@pytest.mark.parametrize("idx", [0, 1, 2, 3])
def test_config4_sdxl_lora_sampled(idx):
    spec = wl.config_shapes(4)[idx]
    d = wl.generate(spec)
    rows, cols = _sample(spec.M, spec.N, 40 + idx)
    G.run_layer_case(d, o.INT4, 32, lora=True, rows=rows, cols=cols)


@pytest.mark.parametrize("idx", list(range(10)))
def test_config5_flux_block_sweep_sampled(idx):
    spec = wl.config_shapes(5)[idx]
    d = wl.generate(spec)
    for j, fmt in enumerate((o.MXFP4, o.INT4)):
        rows, cols = _sample(spec.M, spec.N, 50 + 2 * idx + j)
        G.run_layer_case(d, fmt, 32, lora=True, rows=rows, cols=cols)
