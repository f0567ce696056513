"""GPU edge cases through the C ABI: degenerate values, the scheme's special
cases with closed forms, and the largest batch and split counts.

* Q = 0: every code and scale of Q is 0, so every score is 0 and every
  visible key gets the same weight: each output row is the mean of V^ (V in
  16-bit mode, its FP8 reconstruction otherwise) over the row's visible keys,
  rounded to the output type.
* V constant along the keys: the output is that constant exactly (the row
  sums l are taken from the same rounded weights that multiply V^).
* K blocks equal to the mean: their smoothed codes and scale are 0, so their
  scores are 0; checked against the emulation.
* B = SAGE_MAX_BATCH with ragged frames, and kv_splits = SAGE_MAX_SPLITS.
* Inputs of very large and very small magnitude.
* The largest key length the kernel addresses (a head's 16-bit V^T just under
  2^31 bytes): its last key block dominates every row, so every output row is
  that block's V row.
"""

import numpy as np
import pytest
import torch

import bit_quantized_attention_sage_amd as sage
from oracle import quant, attention, codecs
from oracle.constants import PV_16, PV_FP8
from gpu_util import run_gpu, host, check_quantized, emulate_like_gpu, assert_close, cosine, ulp16

pytestmark = pytest.mark.gpu


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16)


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8])
def test_zero_queries_average_the_visible_values(lib, pv_mode):
    B, H, Nq, Nkv, d, F = 2, 2, 300, 900, 128, 150
    kv, qp = [900, 640], [600, 300]
    q = torch.zeros((B, H, Nq, d), dtype=torch.bfloat16)
    k, v = _rand((B, H, Nkv, d), 31), _rand((B, H, Nkv, d), 32)
    for b in range(B):
        k[b, :, kv[b]:] = 0
        v[b, :, kv[b]:] = 0
    out, views, desc, _, _ = run_gpu(q.cuda(), k.cuda(), v.cuda(), pv_mode, F, kv, qp)
    assert not views["q_codes"].cpu().numpy().any() and not views["q_scale"].cpu().numpy().any()
    V = host(v)
    if pv_mode == PV_FP8:
        vc, ve, _ = quant.quantize_v_fp8(V, kv)
        V = quant.dequant_v_fp8(vc, ve)
    ref = np.empty((B, H, Nq, d))
    for b in range(B):
        for i in range(Nq):
            end = min(kv[b], ((qp[b] + i) // F + 1) * F)
            ref[b, :, i] = V[b, :, :end].mean(axis=1)
    og = host(out)
    # the mean in float32 from rounded weights that are all equal: within
    # float32 accumulation of it, then the output rounding
    err = np.abs(og - ref)
    bound = 0.5 * ulp16(ref, "bf16") * (1 + 2.0 ** -8) + 1e-5 * np.abs(V).max()
    print(f"  max |O - mean V| {err.max():.3e}", flush=True)
    assert (err <= bound).all()


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8])
def test_constant_values_pass_through(lib, pv_mode):
    """O = sum p~ c / sum p~ = c: the float32 sums differ from exact by far
    less than half a bf16 spacing (or, in FP8 mode, c's e4m3 reconstruction,
    itself a bf16 value), so the rounded output is the constant itself."""
    B, H, Nq, Nkv, d = 1, 2, 200, 777, 128
    q, k = _rand((B, H, Nq, d), 41), _rand((B, H, Nkv, d), 42, 2.0)
    c = _rand((1, H, 1, d), 43)
    v = c.expand(B, H, Nkv, d).contiguous()
    out, _, _, _, _ = run_gpu(q.cuda(), k.cuda(), v.cuda(), pv_mode)
    C = host(c)
    if pv_mode == PV_FP8:
        vc, ve, _ = quant.quantize_v_fp8(np.broadcast_to(C, (B, H, Nkv, d)).copy())
        C = quant.dequant_v_fp8(vc, ve)[:, :, :1].astype(np.float32)
        C = codecs.round_to(C, "bf16")
    np.testing.assert_array_equal(host(out), np.broadcast_to(C, (B, H, Nq, d)))


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8])
def test_key_blocks_at_the_mean_have_zero_codes(lib, pv_mode):
    B, H, Nq, Nkv, d = 1, 2, 256, 640, 128
    q, k, v = _rand((B, H, Nq, d), 51), _rand((B, H, Nkv, d), 52), _rand((B, H, Nkv, d), 53)
    mu = torch.from_numpy(np.full((B, H, d), 0.5, np.float32))
    k[:, :, 128:256] = 0.5                  # two whole 64-key blocks equal to the (given) mean
    out, views, desc, _, _ = run_gpu(q.cuda(), k.cuda(), v.cuda(), pv_mode, k_mean_in=mu.cuda())
    Q, K, V = host(q), host(k), host(v)
    check_quantized(views, Q, K, V, pv_mode, "bf16", None, mu_in=mu.numpy())
    assert not views["k_codes"].cpu().numpy()[:, :, 128:256].any()
    assert not views["k_scale"].cpu().numpy()[:, :, 2:4].any()
    o64, aux = emulate_like_gpu(Q, K, V, pv_mode, "bf16", desc, mu=mu.numpy())
    assert_close(host(out), o64, aux, "bf16", pv_mode)


def test_max_batch_ragged_frames(lib):
    B, H, Nq, Nkv, d, F = sage.SAGE_MAX_BATCH, 1, 40, 400, 64, 50
    rng = np.random.default_rng(61)
    kv = [int(x) for x in rng.integers(Nq, Nkv + 1, B)]
    qp = [int(rng.integers(0, x - Nq + 1)) for x in kv]
    q, k, v = _rand((B, H, Nq, d), 62), _rand((B, H, Nkv, d), 63), _rand((B, H, Nkv, d), 64)
    for b in range(B):
        k[b, :, kv[b]:] = 0
        v[b, :, kv[b]:] = 0
    q, k, v = q.to(torch.float16), k.to(torch.float16), v.to(torch.float16)
    out, views, desc, _, _ = run_gpu(q.cuda(), k.cuda(), v.cuda(), PV_16, F, kv, qp)
    Q, K, V = host(q), host(k), host(v)
    check_quantized(views, Q, K, V, PV_16, "f16", kv)
    o64, aux = emulate_like_gpu(Q, K, V, PV_16, "f16", desc, F, kv, qp)
    print(f"  B={B}", flush=True)
    assert_close(host(out), o64, aux, "f16", PV_16)


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8])
def test_max_splits(lib, pv_mode):
    B, H, Nq, Nkv, d = 1, 2, 130, 3000, 128
    q, k, v = _rand((B, H, Nq, d), 71), _rand((B, H, Nkv, d), 72), _rand((B, H, Nkv, d), 73)
    out, _, desc, _, _ = run_gpu(q.cuda(), k.cuda(), v.cuda(), pv_mode, kv_splits=sage.SAGE_MAX_SPLITS)
    assert sage.sage_attn_kv_splits(desc) == sage.SAGE_MAX_SPLITS
    Q, K, V = host(q), host(k), host(v)
    o64, aux = emulate_like_gpu(Q, K, V, pv_mode, "bf16", desc)
    assert_close(host(out), o64, aux, "bf16", pv_mode)


@pytest.mark.parametrize("scale_qk,scale_v", [(30.0, 1e-3), (1e-3, 400.0)])
def test_extreme_magnitudes(lib, scale_qk, scale_v):
    """Large scores (a nearly one-hot softmax, exercising the lazy running
    max) and tiny ones (nearly uniform), with V far from unit scale."""
    B, H, Nq, Nkv, d = 1, 2, 200, 900, 128
    q, k = _rand((B, H, Nq, d), 81, scale_qk), _rand((B, H, Nkv, d), 82, scale_qk)
    v = _rand((B, H, Nkv, d), 83, scale_v)
    out, views, desc, _, _ = run_gpu(q.cuda(), k.cuda(), v.cuda(), PV_16)
    Q, K, V = host(q), host(k), host(v)
    check_quantized(views, Q, K, V, PV_16, "bf16")
    o64, aux = emulate_like_gpu(Q, K, V, PV_16, "bf16", desc)
    og = host(out)
    assert_close(og, o64, aux, "bf16", PV_16)
    # With a nearly one-hot softmax, INT8 error in the scores can move the
    # weight between near-tied keys, so the scheme itself departs from fp64;
    # the kernel must lose nothing beyond what the exact emulation loses.
    o_ref = attention.attention_fp64(Q, K, V)
    cs, cs_emul = cosine(og, o_ref), cosine(o64, o_ref)
    print(f"  cosine vs fp64 {cs:.6f} (emulation {cs_emul:.6f})", flush=True)
    assert cs >= cs_emul - 1e-3
    if scale_qk < 1:
        assert cs >= 0.999


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8])
def test_largest_key_length_reads_its_last_block(lib, pv_mode):
    """Nkv = 8388480, d = 128: the last 64 keys are 25 e_0 and every query has
    20 in channel 0, so their logit is 500 / sqrt(128) = 44 nats (codes 127 x
    127 at scales 20/127 and 25/127, exact) against at most ~5 for the 8.4M
    random keys: all weight is on those 64 keys, equally.  With their V rows
    equal to a constant C, O = C in bf16 (FP8: C's e4m3 reconstruction)."""
    B, H, Nq, Nkv, d = 1, 1, 256, 8388480, 128
    g = torch.Generator(device="cuda").manual_seed(71)
    q = (torch.randn((B, H, Nq, d), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    q[..., 0] = 20.0
    k = (torch.randn((B, H, Nkv, d), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    k[:, :, -64:, :] = 0.0
    k[:, :, -64:, 0] = 25.0
    v = torch.randn((B, H, Nkv, d), generator=g, device="cuda").to(torch.bfloat16)
    c = _rand((1, 1, 1, d), 72)
    v[:, :, -64:, :] = c.cuda()
    print(f"  Nkv {Nkv}: V^T bytes per head {Nkv * d * 2} (< 2^31)", flush=True)
    out, _, desc, _, _ = run_gpu(q, k, v, pv_mode)
    print(f"  kv splits {sage.sage_attn_kv_splits(desc)}", flush=True)
    C = host(c)
    if pv_mode == PV_FP8:
        vc, ve, _ = quant.quantize_v_fp8(np.broadcast_to(C, (1, 1, 64, d)).copy())
        C = codecs.round_to(quant.dequant_v_fp8(vc, ve)[:, :, :1].astype(np.float32), "bf16")
    np.testing.assert_array_equal(host(out), np.broadcast_to(C, (B, H, Nq, d)))


def test_tiny_value_block_keeps_the_smallest_scale(lib):
    """FP8 mode, a V block of 32 keys whose values are about 1e-37 (below
    448 * 2^-127): its E8M0 byte is 0 (the scale 2^-127), its codes are
    finite, and the rows that read it give finite outputs within the bound
    of the emulation."""
    B, H, Nq, Nkv, d = 1, 1, 64, 256, 128
    q, k = _rand((B, H, Nq, d), 95), _rand((B, H, Nkv, d), 96)
    v = _rand((B, H, Nkv, d), 97)
    v[:, :, 64:96, :] = (_rand((1, 1, 32, d), 98).float() * 1e-37).to(torch.bfloat16)
    out, views, desc, _, _ = run_gpu(q.cuda(), k.cuda(), v.cuda(), PV_FP8)
    Q, K, V = host(q), host(k), host(v)
    check_quantized(views, Q, K, V, PV_FP8, "bf16")
    _, e, e8 = quant.quantize_v_fp8(V)
    assert (e8[0, 0, 2] == 0).all()                       # keys 64..95: block 2, byte 0
    og = host(out)
    assert np.isfinite(og).all()
    o64, aux = emulate_like_gpu(Q, K, V, PV_FP8, "bf16", desc)
    assert_close(og, o64, aux, "bf16", PV_FP8)
