"""Pins of the block-sparse reading in the oracle: a (128-query block,
64-key block) tile dropped by the caller's block mask is skipped, as sparse
attention built on SageAttention does (Vidu S1 blog, section "Infra";
TurboDiffusion digests).  Each pin fixes the result by something other than
the oracle's own code: brute-force softmax over the kept keys, a closed form,
or the same emulation run on inputs with the dropped keys deleted."""

import math

import numpy as np
import pytest

from oracle import attention, quant, emulate
from oracle.constants import PV_16, PV_FP8, BK, BQ


def _rnd16(x):
    from oracle import codecs
    return codecs.round_to(np.asarray(x, np.float32), "bf16").astype(np.float32)


def _mask(rng, B, H, Nq, Nkv, density):
    return (rng.random((B, H, -(-Nq // BQ), -(-Nkv // BK))) < density).astype(np.uint8)


def test_fp64_block_mask_equals_brute_force_softmax():
    rng = np.random.default_rng(70)
    B, H, Nq, Nkv, d, F = 1, 2, 200, 300, 8, 100
    Q, K, V = (rng.standard_normal((B, H, n, d)) for n in (Nq, Nkv, Nkv))
    M = _mask(rng, B, H, Nq, Nkv, 0.5)
    M[0, 0, 0, :] = 0                       # a tile with nothing kept
    kv, qp = [280], [80]
    rows = np.array([0, 5, 127, 128, 150, 199])
    out = attention.attention_fp64(Q, K, V, 0.4, frame_len=F, kv_len=kv, q_pos0=qp, rows=rows, block_mask=M)
    for h in range(H):
        for r, i in enumerate(rows):
            keys = [j for j in range(Nkv) if j < kv[0] and j // F <= (qp[0] + i) // F and M[0, h, i // BQ, j // BK]]
            if not keys:
                assert not out[0, h, r].any()
                continue
            s = [0.4 * sum(Q[0, h, i, c] * K[0, h, j, c] for c in range(d)) for j in keys]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            ref = [sum(wk * V[0, h, j, c] for wk, j in zip(w, keys)) / sum(w) for c in range(d)]
            np.testing.assert_allclose(out[0, h, r], ref, rtol=0, atol=1e-12)
    assert not out[0, 0, :3].any()          # rows 0, 5, 127 of the empty tile


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8])
def test_all_kept_mask_is_the_dense_path(pv_mode):
    rng = np.random.default_rng(71)
    Q = _rnd16(rng.standard_normal((1, 2, 200, 32)))
    K = _rnd16(rng.standard_normal((1, 2, 330, 32)) + 1.0)
    V = _rnd16(rng.standard_normal((1, 2, 330, 32)))
    ones = np.ones((1, 2, 2, 6), np.uint8)
    a, _ = emulate.emulate_from_inputs(Q, K, V, pv_mode, "bf16", kv_len=[320])
    b, _ = emulate.emulate_from_inputs(Q, K, V, pv_mode, "bf16", kv_len=[320], block_mask=ones)
    assert np.array_equal(a, b)
    c = emulate.emulate_block_sparse(Q, K, V, pv_mode, "bf16", ones, 1, kv_len=[320])[0]
    assert np.array_equal(a, c)
    r1 = attention.attention_fp64(Q, K, V, kv_len=[320])
    r2 = attention.attention_fp64(Q, K, V, kv_len=[320], block_mask=ones)
    np.testing.assert_allclose(r1, r2, rtol=0, atol=1e-15)


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8])
def test_q_zero_is_the_mean_over_kept_keys(pv_mode):
    """Q = 0: every visible p is 1, so a row is the mean of V^ over its kept,
    visible keys (0 when there are none); fixes the mask count."""
    rng = np.random.default_rng(72)
    B, H, Nq, Nkv, d, F = 1, 2, 256, 640, 16, 128
    Q = np.zeros((B, H, Nq, d), np.float32)
    K = _rnd16(rng.standard_normal((B, H, Nkv, d)))
    V = _rnd16(rng.standard_normal((B, H, Nkv, d)))
    M = _mask(rng, B, H, Nq, Nkv, 0.4)
    M[0, 1, 1, :] = 0
    kv, qp = [600], [300]
    o64, _ = emulate.emulate_from_inputs(Q, K, V, pv_mode, "bf16", frame_len=F, kv_len=kv, q_pos0=qp,
                                         block_mask=M)
    if pv_mode == PV_FP8:
        vc, ve, _ = quant.quantize_v_fp8(V, kv)
        Vh = quant.dequant_v_fp8(vc, ve)
    else:
        Vh = V.astype(np.float64)
    for h in range(H):
        for i in range(0, Nq, 7):
            end = min(kv[0], ((qp[0] + i) // F + 1) * F)
            keys = [j for j in range(end) if M[0, h, i // BQ, j // BK]]
            ref = Vh[0, h, keys].mean(axis=0) if keys else np.zeros(d)
            np.testing.assert_allclose(o64[0, h, i], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8])
def test_dropped_key_blocks_are_as_if_deleted(pv_mode):
    """The same key blocks dropped for every query tile, with the mean and
    channel shifts frozen, give bit-identical outputs to the emulation on K
    and V with those 64-key blocks deleted: skipped chunks change neither the
    running max nor the sums."""
    rng = np.random.default_rng(73)
    Nq, nkb, d = 256, 10, 32
    Q = _rnd16(rng.standard_normal((1, 2, Nq, d)))
    K = _rnd16(rng.standard_normal((1, 2, nkb * BK, d)) * 1.5 + 0.5)
    V = _rnd16(rng.standard_normal((1, 2, nkb * BK, d)))
    mu = quant.k_mean(K)
    a = quant.channel_shift(Q, K, mu)
    keep = np.array([1, 0, 1, 1, 0, 0, 1, 0, 1, 1], bool)
    M = np.broadcast_to(keep.astype(np.uint8), (1, 2, 2, nkb)).copy()
    sparse, _ = emulate.emulate_from_inputs(Q, K, V, pv_mode, "bf16", mu=mu, shift=a, block_mask=M)
    idx = np.concatenate([np.arange(k * BK, k * BK + BK) for k in np.nonzero(keep)[0]])
    dense, _ = emulate.emulate_from_inputs(Q, K[:, :, idx], V[:, :, idx], pv_mode, "bf16", mu=mu, shift=a)
    assert np.array_equal(sparse, dense)
    # and dropping one more block changes the result
    M2 = M.copy()
    M2[..., 2] = 0
    other, _ = emulate.emulate_from_inputs(Q, K, V, pv_mode, "bf16", mu=mu, shift=a, block_mask=M2)
    assert not np.array_equal(sparse, other)


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8])
def test_sparse_splits_are_the_dense_grid(pv_mode):
    """KV splits under a block mask cut the batch's chunk grid exactly as
    without one: with every tile kept, the split emulation is bit-identical
    to the dense emulation over the same split ranges."""
    rng = np.random.default_rng(74)
    Q = _rnd16(rng.standard_normal((2, 1, 200, 32)))
    K = _rnd16(rng.standard_normal((2, 1, 900, 32)))
    V = _rnd16(rng.standard_normal((2, 1, 900, 32)))
    kv = [900, 517]
    ones = np.ones((2, 1, 2, -(-900 // BK)), np.uint8)
    for S in (2, 3, 5):
        sparse = emulate.emulate_block_sparse(Q, K, V, pv_mode, "bf16", ones, S, kv_len=kv)[0]
        dense = emulate.emulate_from_inputs(Q, K, V, pv_mode, "bf16", kv_len=kv,
                                            splits=[emulate.split_ranges(k, S) for k in kv])[0]
        assert np.array_equal(sparse, dense)
        assert emulate.split_ranges(517, S) == [(s * 9 // S, (s + 1) * 9 // S) for s in range(S)]


def test_sparse_split_emulation_within_p_rounding():
    """Split work items over a tile's kept list keep their own running max;
    the merged result stays within P's rounding of the unsplit one."""
    rng = np.random.default_rng(75)
    Q = _rnd16(rng.standard_normal((1, 2, 256, 32)))
    K = _rnd16(rng.standard_normal((1, 2, 1280, 32)))
    V = _rnd16(rng.standard_normal((1, 2, 1280, 32)))
    M = _mask(rng, 1, 2, 256, 1280, 0.5)
    o1 = emulate.emulate_block_sparse(Q, K, V, PV_16, "bf16", M, 1)[0]
    o3 = emulate.emulate_block_sparse(Q, K, V, PV_16, "bf16", M, 3)[0]
    assert np.abs(o3 - o1).max() <= 2 * 2 * 2.0 ** -8 * np.abs(V).max()
    assert not np.array_equal(o1, o3)
