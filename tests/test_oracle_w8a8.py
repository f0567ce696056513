"""Pins of the per-block W8A8 linear layer in the oracle: brute-force
scalar loops, a power-of-two closed form, the quantization error bound
against the unquantized product, and the outlier behaviour that motivates
per-block scales (Vidu S1 blog, section "Infra")."""

import numpy as np

from oracle import w8a8, codecs


def _bf16(x):
    return codecs.round_to(np.asarray(x, np.float32), "bf16").astype(np.float32)


def test_quantizers_match_a_scalar_loop():
    rng = np.random.default_rng(90)
    X = _bf16(rng.standard_normal((3, 256)) * 2)
    X[1, 128:] = 0                                  # an all-zero group
    xq, dx = w8a8.quantize_act(X)
    for m in range(3):
        for g in range(2):
            blk = X[m, 128 * g:128 * g + 128]
            amax = np.float32(max(abs(float(v)) for v in blk))
            if amax == 0:
                assert dx[m, g] == 0 and not xq[m, 128 * g:128 * g + 128].any()
                continue
            assert dx[m, g] == np.float32(amax / np.float32(127))
            inv = np.float32(np.float32(127) / amax)
            for k in range(128):
                c = np.rint(np.float32(blk[k] * inv))
                assert xq[m, 128 * g + k] == int(max(-127, min(127, c)))
    W = _bf16(rng.standard_normal((256, 128)))
    wq, dw = w8a8.quantize_weight(W)
    assert dw.shape == (2, 1)
    for nb in range(2):
        amax = np.abs(W[128 * nb:128 * nb + 128]).max()
        assert dw[nb, 0] == np.float32(amax / np.float32(127))


def test_power_of_two_blocks_are_exact():
    """Blocks whose entries are integers in [-127, 127] times 2^e with one
    entry at +-127 2^e quantize to exactly those integers, so the quantized
    GEMM equals X W^T exactly."""
    rng = np.random.default_rng(91)
    M, N, K = 5, 256, 256
    X = rng.integers(-127, 128, (M, K)).astype(np.float64)
    X[:, ::128] = 127
    X *= 2.0 ** rng.integers(-4, 4, (M, 1))
    W = rng.integers(-127, 128, (N, K)).astype(np.float64)
    W[::128, ::128] = -127
    W[128:] *= 0.25
    xq, dx = w8a8.quantize_act(X.astype(np.float32))
    wq, dw = w8a8.quantize_weight(W.astype(np.float32))
    y, _ = w8a8.gemm_exact(xq, dx, wq, dw)
    np.testing.assert_array_equal(y, X @ W.T)


def test_gemm_matches_brute_force_and_bias():
    rng = np.random.default_rng(92)
    M, N, K = 3, 128, 256
    X = _bf16(rng.standard_normal((M, K)))
    W = _bf16(rng.standard_normal((N, K)))
    bias = _bf16(rng.standard_normal(N))
    xq, dx = w8a8.quantize_act(X)
    wq, dw = w8a8.quantize_weight(W)
    y, mag = w8a8.gemm_exact(xq, dx, wq, dw, bias)
    for m in range(M):
        for n in (0, 77, 127):
            ref = float(bias[n])
            for kb in range(2):
                s = sum(int(xq[m, k]) * int(wq[n, k]) for k in range(128 * kb, 128 * kb + 128))
                ref += float(dx[m, kb]) * float(dw[0, kb]) * s
            assert abs(y[m, n] - ref) <= 1e-12 * mag[m, n]


def test_quantization_error_within_the_rounding_bound():
    """|Y_q - X W^T| <= sum_k (|x| dw/2 + |w| dx/2 + dx dw/4): each code is
    within half a step of its value."""
    rng = np.random.default_rng(93)
    M, N, K = 16, 256, 384
    X = _bf16(rng.standard_normal((M, K)))
    W = _bf16(rng.standard_normal((N, K)) * 0.05)
    xq, dx = w8a8.quantize_act(X)
    wq, dw = w8a8.quantize_weight(W)
    y, _ = w8a8.gemm_exact(xq, dx, wq, dw)
    ref = w8a8.linear_fp64(X, W)
    DX = np.repeat(dx, 128, axis=1).astype(np.float64)                   # [M, K]
    DW = np.repeat(np.repeat(dw, 128, axis=0), 128, axis=1).astype(np.float64)  # [N, K]
    bound = (np.abs(X) @ DW.T) / 2 + (DX @ np.abs(W).T) / 2 + (DX @ DW.T) / 4
    assert (np.abs(y - ref) <= bound * (1 + 1e-9)).all()
    cos = (y * ref).sum() / np.sqrt((y * y).sum() * (ref * ref).sum())
    assert cos > 0.9999


def test_per_block_scales_contain_channel_outliers():
    """One activation channel x100: per-block scales keep the other groups'
    precision; a single per-tensor scale loses it."""
    rng = np.random.default_rng(94)
    M, N, K = 64, 128, 512
    X = _bf16(rng.standard_normal((M, K)))
    X[:, 7] *= 100
    W = _bf16(rng.standard_normal((N, K)))
    xq, dx = w8a8.quantize_act(X)
    wq, dw = w8a8.quantize_weight(W)
    y, _ = w8a8.gemm_exact(xq, dx, wq, dw)
    ref = w8a8.linear_fp64(X, W)
    xt, dt = w8a8.quant_tiles(X, M, K)        # one scale for the whole tensor
    yt, _ = w8a8.gemm_exact(xt, np.repeat(dt, M, axis=0).repeat(K // 128, axis=1), wq, dw)
    e_blk = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    e_ten = np.linalg.norm(yt - ref) / np.linalg.norm(ref)
    assert e_blk * 3 < e_ten
